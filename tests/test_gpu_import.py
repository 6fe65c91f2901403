"""GPU: q8kv_import_pages rewrites a row-order int8 cache ([block][row][kv
head][hd] bytes, [block][row][kv head] fp32 scales) into the library's page
layout, bit for bit.

* arbitrary bytes and scale bit patterns (NaN and infinities included) come
  back unchanged when the pages are read in row order through the byte
  order the header documents, for every hd and several kv_bs / n_kv;
* a cache the oracle quantised, handed over in row order, gives the same
  device bytes as q8kv_append of the same fp32 rows, and a decode over it
  gives the same output bits.
"""
import numpy as np
import pytest
import torch

import decode_attention_int8_amd as q8
from cases import build, small
from gpu_cases import DEV, decode, gpu_cache, natural_pages, say, to_dev

pytestmark = pytest.mark.gpu


def import_rows(nb, n_kv, kv_bs, hd, k_rows, v_rows, ks_rows, vs_rows):
    cache = q8.PagedKVCache(nb, n_kv, kv_bs, hd, device=DEV)
    for t in (cache.k_pages, cache.v_pages):
        t.fill_(0x55)
    for t in (cache.k_scale, cache.v_scale):
        t.fill_(-1.0)
    q8.import_pages(cache, to_dev(k_rows), to_dev(v_rows), to_dev(ks_rows), to_dev(vs_rows))
    torch.cuda.synchronize()
    return cache


@pytest.mark.parametrize("hd,kv_bs,n_kv,nb", [
    (64, 16, 3, 5), (128, 64, 8, 3), (256, 32, 2, 4), (128, 256, 1, 2), (64, 128, 5, 1), (256, 16, 7, 6),
    (96, 16, 3, 2), (160, 32, 2, 3), (32, 64, 1, 2), (224, 16, 2, 2),  # padded pages
])
def test_import_is_a_permutation(hd, kv_bs, n_kv, nb):
    rng = np.random.default_rng(hd * 1000 + kv_bs * 10 + n_kv)
    k_rows = rng.integers(-128, 128, (nb, kv_bs, n_kv, hd), dtype=np.int8)
    v_rows = rng.integers(-128, 128, (nb, kv_bs, n_kv, hd), dtype=np.int8)
    bits = rng.integers(0, 2 ** 32, (2, nb, kv_bs, n_kv), dtype=np.uint64).astype(np.uint32)
    bits[0, 0, 0, 0] = 0x7FC00001  # a NaN payload
    bits[1, -1, -1, -1] = 0xFF800000  # -inf
    ks_rows, vs_rows = bits[0].view(np.float32), bits[1].view(np.float32)
    say(f"import hd={hd} kv_bs={kv_bs} n_kv={n_kv} nb={nb}")
    c = import_rows(nb, n_kv, kv_bs, hd, k_rows, v_rows, ks_rows, vs_rows)
    kn = natural_pages(c.k_pages.cpu().numpy(), "k")
    vn = natural_pages(c.v_pages.cpu().numpy(), "v")
    assert np.array_equal(kn[..., :hd], k_rows.transpose(0, 2, 1, 3))
    assert np.array_equal(vn[..., :hd], v_rows.transpose(0, 2, 1, 3))
    assert not kn[..., hd:].any() and not vn[..., hd:].any()  # pad columns of a padded head
    assert np.array_equal(c.k_scale.cpu().numpy().view(np.uint32), bits[0].transpose(0, 2, 1))
    assert np.array_equal(c.v_scale.cpu().numpy().view(np.uint32), bits[1].transpose(0, 2, 1))


@pytest.mark.parametrize("name", ["gqa_batch", "ragged", "long_gqa"])
def test_imported_cache_decodes_like_appended(name):
    """The oracle's quantised cache, passed in row order, equals what
    q8kv_append writes from the same fp32 rows, and decodes to the same bits."""
    c = build({"gqa_batch": small("gqa_batch", batch=3, n_q=8, n_kv=2, seq_len=170),
               "ragged": small("ragged", batch=6, n_q=16, n_kv=2, seq_len=400),
               "long_gqa": small("long_gqa", n_q=16, n_kv=2, seq_len=1000)}[name])
    h = c.cache
    say(f"import vs append {name}")
    imp = import_rows(h.num_blocks, h.n_kv, h.kv_bs, h.hd,
                      h.k_pages.transpose(0, 2, 1, 3), h.v_pages.transpose(0, 2, 1, 3),
                      h.k_scale.transpose(0, 2, 1), h.v_scale.transpose(0, 2, 1))
    app = gpu_cache(c)
    torch.cuda.synchronize()
    for f in ("k_pages", "v_pages"):
        assert torch.equal(getattr(imp, f), getattr(app, f)), f
    for f in ("k_scale", "v_scale"):
        assert torch.equal(getattr(imp, f).view(torch.int32), getattr(app, f).view(torch.int32)), f
    a, b = decode(c, imp), decode(c, app)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_import_rejects_bad_shapes():
    cache = q8.PagedKVCache(2, 2, 16, 128, device=DEV)
    rows = torch.zeros((2, 16, 2, 128), dtype=torch.int8, device=DEV)
    sc = torch.zeros((2, 16, 2), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        q8.import_pages(cache, rows[:1], rows, sc, sc)
    with pytest.raises(ValueError):
        q8.import_pages(cache, rows, rows, sc.transpose(1, 2).contiguous(), sc)
    with pytest.raises(TypeError):
        q8.import_pages(q8.Fp8KVCache(2, 2, 16, 128, device=DEV), rows, rows, sc, sc)
