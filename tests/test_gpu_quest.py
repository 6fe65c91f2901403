"""GPU parity of the QUEST path: q8kv_quest_metadata, q8kv_quest_select and
q8kv_decode_attn_heads.

* Metadata against oracle/quest.py bit for bit (both take max / min of the
  same fp32 products), blocks the table does not reference left untouched.
* Selection: the kernel decides in fp32 with its own summation order, the
  oracle's bounds are fp64, so near-ties may go either way.  The test checks
  what is unique -- the kept count, the last block, logical order, the
  selected length -- and that the kept set is valid: every kept block's
  fp64 bound is at least every dropped block's minus a rounding margin; where
  the margin separates the k-th from the (k+1)-th bound the sets must be
  equal.
* Decode over the selection against the oracle decode over the same block
  lists (2e-4); with top_k at least the block count the selection is the
  whole sequence and the output is bitwise the dense decode's.
"""
import numpy as np
import pytest
import torch

import decode_attention_int8_amd as q8
import oracle
import workloads
from cases import build
from gpu_cases import DEV, gpu_cache, say, to_dev
from oracle import quest
from test_oracle_quest import quest_decode

pytestmark = pytest.mark.gpu

TOL = 2e-4


def run(c, top_k, cache=None):
    cache = cache or gpu_cache(c)
    q, bt, sl = to_dev(c.q), to_dev(c.table), to_dev(c.lens)
    kmax, kmin = q8.quest_metadata(cache, bt, sl)
    sel, sel_lens = q8.quest_select(q, cache, kmax, kmin, bt, sl, top_k)
    out = q8.decode_attn_heads(q, cache, sel, sel_lens, c.scale)
    torch.cuda.synchronize()
    return cache, kmax.cpu().numpy(), kmin.cpu().numpy(), sel.cpu().numpy(), sel_lens.cpu().numpy(), out.cpu().numpy()


def check_selection(c, kmax, kmin, sel, sel_lens, top_k):
    U = quest.bounds(c.q, kmax, kmin, c.table, c.lens, c.w.n_kv, c.w.kv_bs)
    _, want_tab, want_lens = quest.select(U, c.table, c.lens, c.w.kv_bs, top_k)
    assert np.array_equal(sel_lens, want_lens)
    q = c.q.astype(np.float64)
    G = c.w.n_q // c.w.n_kv
    for b in range(c.w.batch):
        nblk = -(-max(int(c.lens[b]), 0) // c.w.kv_bs)
        logical = {int(c.table[b, j]): j for j in range(nblk)}
        for kh in range(c.w.n_kv):
            row = sel[b, kh]
            kept = [int(x) for x in row if x >= 0]
            assert len(kept) == min(nblk, top_k) and np.all(row[len(kept):] == -1)
            if nblk == 0:
                continue
            js = [logical[p] for p in kept]
            assert js == sorted(js) and js[-1] == nblk - 1
            if nblk <= top_k:
                continue
            chosen = set(js[:-1])
            dropped = [j for j in range(nblk - 1) if j not in chosen]
            # rounding margin of an fp32 sum of hd terms
            mag = max(np.abs(np.maximum(q[b, h] * kmax[int(c.table[b, j]), kh], q[b, h] * kmin[int(c.table[b, j]), kh])).sum()
                      for h in range(kh * G, (kh + 1) * G) for j in range(nblk - 1))
            eps = mag * 2.0 ** -20
            lo = min(U[b, kh, j] for j in chosen) if chosen else np.inf
            hi = max(U[b, kh, j] for j in dropped) if dropped else -np.inf
            assert lo >= hi - eps, (b, kh, lo, hi)
            order = sorted(range(nblk - 1), key=lambda j: (-U[b, kh, j], j))
            k = top_k - 1
            separated = k == 0 or U[b, kh, order[k - 1]] - U[b, kh, order[k]] > 2 * eps
            if separated:
                assert np.array_equal(row, want_tab[b, kh]), (b, kh)


@pytest.mark.parametrize("hd,G,kv_bs,top_k", [(128, 4, 16, 4), (128, 8, 64, 3), (64, 1, 16, 6), (256, 2, 32, 2),
                                              (128, 5, 16, 1), (128, 2, 128, 8)])
def test_quest_metadata_selection_decode(hd, G, kv_bs, top_k):
    lens = [0, 1, kv_bs, kv_bs + 1, 5 * kv_bs + 3, 9 * kv_bs, 3 * kv_bs - 1, 12 * kv_bs + 7]
    w = workloads.Workload("questgpu", len(lens), 2 * G, 2, hd, kv_bs, max(lens), ragged=True, table="pool",
                           key=3100 + hd + G + kv_bs + top_k)
    c = build(w, lens=lens)
    say(f"quest hd={hd} G={G} kv_bs={kv_bs} top_k={top_k}")
    cache, kmax, kmin, sel, sel_lens, out = run(c, top_k)
    wmax, wmin = quest.metadata(c.cache.k_pages, c.cache.k_scale, c.table, c.lens, kv_bs)
    assert np.array_equal(kmax.view(np.uint32), wmax.view(np.uint32))
    assert np.array_equal(kmin.view(np.uint32), wmin.view(np.uint32))
    check_selection(c, kmax, kmin, sel, sel_lens, top_k)
    want = quest_decode(c.q, c.cache, sel, sel_lens, c.scale)
    assert np.all(np.isfinite(out))
    assert float(np.abs(out - want).max()) <= TOL
    assert not out[0].any()


def test_quest_full_selection_is_dense_decode():
    lens = [70, 33, 160, 1]
    w = workloads.Workload("questfull", 4, 8, 2, 128, 16, 160, ragged=True, table="pool", key=3200)
    c = build(w, lens=lens)
    cache = gpu_cache(c)
    _, _, _, sel, sel_lens, out = run(c, top_k=10, cache=cache)
    assert np.array_equal(sel_lens, c.lens)
    dense = q8.decode_attn(to_dev(c.q), cache, to_dev(c.table), to_dev(c.lens), c.scale).cpu().numpy()
    assert np.array_equal(out.view(np.uint32), dense.view(np.uint32))


def test_quest_long_sequence_many_blocks():
    """One 4000-token sequence in 250 blocks, keep 32: the selection path at
    a size where several blocks per thread are ranked, split decode plans."""
    w = workloads.Workload("questlong", 1, 8, 2, 128, 16, 4000, table="pool", key=3300)
    c = build(w)
    cache, kmax, kmin, sel, sel_lens, out = run(c, top_k=32)
    check_selection(c, kmax, kmin, sel, sel_lens, 32)
    want = quest_decode(c.q, c.cache, sel, sel_lens, c.scale)
    assert float(np.abs(out - want).max()) <= TOL
    for pt in (64, 160):
        got = q8.decode_attn_heads(to_dev(c.q), cache, to_dev(sel), to_dev(sel_lens), c.scale,
                                   part_tokens=pt).cpu().numpy()
        assert float(np.abs(got - want).max()) <= TOL


def test_quest_ties_keep_lower_blocks():
    """Identical K blocks give identical bounds: the kept blocks are the
    lowest-numbered ones."""
    w = workloads.Workload("questtie", 1, 4, 1, 128, 16, 160, key=3400)
    c = build(w, with_cache=False)
    k = c.k_src[0]
    k[:] = k[:16][np.arange(160) % 16]          # every block holds the same 16 rows
    c.cache = None
    from cases import host_cache
    c.cache = host_cache(c)
    _, kmax, kmin, sel, sel_lens, _ = run(c, top_k=4)
    logical = {int(c.table[0, j]): j for j in range(10)}
    assert [logical[int(p)] for p in sel[0, 0]] == [0, 1, 2, 9]


def test_quest_max_blocks():
    """4097 blocks in one sequence, the most the selection takes (16
    candidates per thread of the top-k workgroup), keeping 64."""
    w = workloads.Workload("questmax", 1, 4, 1, 128, 16, 4097 * 16, table="pool", key=3500)
    c = build(w)
    assert c.table.shape[1] == 4097
    cache, kmax, kmin, sel, sel_lens, out = run(c, top_k=64)
    check_selection(c, kmax, kmin, sel, sel_lens, 64)
    want = quest_decode(c.q, c.cache, sel, sel_lens, c.scale)
    assert float(np.abs(out - want).max()) <= TOL


@pytest.mark.parametrize("hd", [96, 160])
def test_decode_heads_padded_head_size(hd):
    """q8kv_decode_attn_heads over per-kv-head block lists at head sizes
    stored in padded pages (the QUEST selection itself takes 64, 128 or
    256): each kv head keeps its own subset of the sequence's blocks, the
    last block always kept, against the oracle over the same lists."""
    lens = [300, 65, 1, 0, 130]
    w = workloads.Workload("headspad", len(lens), 8, 2, hd, 16, max(lens), ragged=True, table="pool",
                           key=3500 + hd)
    c = build(w, lens=lens)
    say(f"decode over per-head block lists hd={hd}")
    cache = gpu_cache(c)
    rng = np.random.default_rng(3500 + hd)
    top = 8
    sel = np.full((w.batch, w.n_kv, top), -1, np.int32)
    sel_lens = np.zeros(w.batch, np.int32)
    for b in range(w.batch):
        nblk = -(-max(int(c.lens[b]), 0) // w.kv_bs)
        if nblk == 0:
            continue
        keep = min(nblk, top)
        last = (int(c.lens[b]) - 1) % w.kv_bs + 1
        sel_lens[b] = (keep - 1) * w.kv_bs + last
        for kh in range(w.n_kv):
            js = sorted(rng.choice(nblk - 1, keep - 1, replace=False).tolist()) + [nblk - 1]
            sel[b, kh, :keep] = c.table[b, js]
    want = quest_decode(c.q, c.cache, sel, sel_lens, c.scale)
    for pt in (0, 32):
        got = q8.decode_attn_heads(to_dev(c.q), cache, to_dev(sel), to_dev(sel_lens), c.scale,
                                   part_tokens=pt).cpu().numpy()
        assert float(np.abs(got - want).max()) <= TOL
