"""GPU parity of the q4_0 KV codec (q8kv_q40_append, q8kv_q40_decode_attn).

* Append: the device pages, unpacked through the nibble order include/q8kv.h
  defines, and the fp16 scale bits against oracle/q40.py bit for bit: unit
  normal rows, blocks spanning 2^-12 .. 2^12, all-zero blocks, negative
  maxima, ties of magnitude (the first element decides the sign of d), exact
  code multiples, bf16 sources.
* Decode: against the oracle's fp64 definition within 2e-4 max-abs on every
  hd, group sizes 1-8, kv_bs 16-256, split plans on both merge paths, the
  persistent grid (bitwise repeatable), static grids whose waves walk 0-10
  tiles (every tail of the two-tile pipeline), empty sequences and an
  out-of-pool table entry (NaN row for that sequence only).
"""
import numpy as np
import pytest
import torch

import decode_attention_int8_amd as q8
import workloads
from cases import build
from gpu_cases import DEV, q40_codes, say, to_dev
from oracle import q40

pytestmark = pytest.mark.gpu

TOL = 2e-4


def dev_cache(c, src_dtype=torch.float32):
    w = c.w
    cache = q8.Q40KVCache(c.num_blocks, w.n_kv, w.kv_bs, w.hd, device=DEV)
    cache.k_pages.fill_(0xA5)
    cache.v_pages.fill_(0xA5)
    cache.k_scale.fill_(float("nan"))
    cache.v_scale.fill_(float("nan"))
    for b in range(w.batch):
        if len(c.slots[b]):
            cache.append(to_dev(c.k_src[b], src_dtype), to_dev(c.v_src[b], src_dtype), to_dev(c.slots[b]))
    return cache


def host_cache(c, src_dtype=torch.float32):
    w = c.w
    h = q40.Q40Cache(c.num_blocks, w.n_kv, w.kv_bs, w.hd)
    for b in range(w.batch):
        if len(c.slots[b]):
            k, v = c.k_src[b], c.v_src[b]
            if src_dtype == torch.bfloat16:
                k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
                v = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
            h.append(k, v, c.slots[b])
    return h


def written_rows(c):
    """(block, row) of every written slot."""
    rows = []
    for b in range(c.w.batch):
        for sl in c.slots[b]:
            rows.append(divmod(int(sl), c.w.kv_bs))
    return tuple(np.array(x) for x in zip(*rows)) if rows else (np.array([], int), np.array([], int))


def assert_q40_equal(c, host, dev):
    blk, row = written_rows(c)
    for which in ("k", "v"):
        got = q40_codes(getattr(dev, which + "_pages").cpu().numpy(), which)
        want = getattr(host, which + "_codes")
        g, w_ = got[blk, :, row], want[blk, :, row]
        bad = np.argwhere(g != w_)
        assert bad.size == 0, f"{which} codes: {len(bad)} differ, first {bad[0].tolist()}"
        gs = getattr(dev, which + "_scale").cpu().numpy()[blk, :, row].view(np.uint16)
        ws = getattr(host, which + "_d")[blk, :, row].view(np.uint16)
        assert np.array_equal(gs, ws), which + " scales"


def special_rows(rng, n, hd):
    rows = rng.standard_normal((n, hd)).astype(np.float32)
    for i in range(n):
        for blk in range(hd // 32):
            seg = rows[i, 32 * blk:32 * (blk + 1)]
            kind = (i + blk) % 6
            if kind == 0:
                seg *= np.float32(2.0 ** rng.integers(-12, 13))
            elif kind == 1:
                seg[:] = 0
            elif kind == 2:
                seg[7] = -np.abs(seg).max() * 1.5        # a negative maximum
            elif kind == 3:
                m = np.abs(seg).max() * 1.25
                seg[3], seg[9] = m, -m                    # a tie: the first decides d's sign
            elif kind == 4:
                d = np.float32(2.0 ** rng.integers(-5, 3))
                c = rng.integers(0, 16, 32)
                c[11] = 0
                seg[:] = (c - 8) * d                      # exact code multiples
    return rows


@pytest.mark.parametrize("hd,kv_bs,n_kv,dtype", [
    (128, 16, 2, torch.float32), (64, 32, 3, torch.float32), (256, 64, 2, torch.float32),
    (128, 16, 2, torch.bfloat16), (256, 16, 1, torch.bfloat16),
])
def test_q40_append_bit_exact(hd, kv_bs, n_kv, dtype):
    w = workloads.Workload("q40app", 3, n_kv, n_kv, hd, kv_bs, 3 * kv_bs + 5, ragged=True, table="pool",
                           key=4000 + hd + kv_bs)
    c = build(w, with_cache=False)
    rng = np.random.default_rng(4100 + hd)
    for b in range(w.batch):
        L = len(c.slots[b])
        if L:
            c.k_src[b] = special_rows(rng, L * n_kv, hd).reshape(L, n_kv, hd)
            c.v_src[b] = special_rows(rng, L * n_kv, hd).reshape(L, n_kv, hd)
    say(f"q40 append hd={hd} kv_bs={kv_bs} n_kv={n_kv} dtype={dtype}")
    assert_q40_equal(c, host_cache(c, dtype), dev_cache(c, dtype))


def run_decode(c, dev, host, part_tokens=0):
    q, bt, sl = to_dev(c.q), to_dev(c.table), to_dev(c.lens)
    got = q8.q40_decode_attn(q, dev, bt, sl, c.scale, part_tokens=part_tokens)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = q40.decode(c.q, host, c.table, c.lens, c.scale)
    assert np.all(np.isfinite(got))
    err = float(np.abs(got - want).max()) if got.size else 0.0
    assert err <= TOL, f"max-abs error {err:.3g} > {TOL}"
    return got


@pytest.mark.parametrize("hd,G,kv_bs", [(64, 1, 16), (64, 8, 32), (128, 3, 16), (128, 8, 128),
                                        (256, 2, 64), (256, 8, 16), (128, 5, 256), (128, 4, 64),
                                        (128, 16, 64), (64, 12, 16)])  # more heads than one MFMA column set
def test_q40_decode_shapes(hd, G, kv_bs):
    lens = [1, 0, 16, 17, 33, kv_bs, kv_bs + 1, 2 * kv_bs + 7, 300]
    w = workloads.Workload("q40shape", len(lens), 2 * G, 2, hd, kv_bs, max(lens), ragged=True, table="pool",
                           key=4200 + hd + G + kv_bs)
    c = build(w, lens=lens, with_cache=False)
    say(f"q40 decode hd={hd} G={G} kv_bs={kv_bs}")
    dev, host = dev_cache(c), host_cache(c)
    assert_q40_equal(c, host, dev)
    got = run_decode(c, dev, host)
    assert not got[1].any()
    for pt in (32, 96):
        run_decode(c, dev, host, part_tokens=pt)


def test_q40_decode_persistent_grid():
    rng = np.random.default_rng(4300)
    lens = [int(x) for x in rng.integers(1, 600, size=64)]
    lens[:5] = [0, 1, 32, 33, 64]
    w = workloads.Workload("q40persist", 64, 8, 2, 128, 16, 600, ragged=True, table="pool", key=4300)
    c = build(w, lens=lens, with_cache=False)
    dev, host = dev_cache(c), host_cache(c)
    for pt in (32, 64):
        a = run_decode(c, dev, host, part_tokens=pt)
        b = run_decode(c, dev, host, part_tokens=pt)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_q40_decode_small_workload_shapes():
    for name, kw in {"gqa": dict(batch=3, n_q=8, n_kv=2, kv_bs=16, seq_len=170),
                     "long": dict(batch=1, n_q=16, n_kv=2, kv_bs=64, seq_len=1000)}.items():
        w = workloads.Workload("q40_" + name, kw["batch"], kw["n_q"], kw["n_kv"], 128, kw["kv_bs"], kw["seq_len"],
                               ragged=name == "gqa", table="pool", key=4400 + len(name))
        c = build(w, with_cache=False)
        dev, host = dev_cache(c), host_cache(c)
        run_decode(c, dev, host)
        run_decode(c, dev, host, part_tokens=64)


@pytest.mark.parametrize("hd,kv_bs", [(128, 64), (128, 16), (64, 32)])
def test_q40_decode_static_tile_counts(hd, kv_bs):
    """One partition per sequence on a static grid, so that the waves walk 0 to
    10 tiles each: the two-tile pipeline's steady loop and every tail after it
    (one, two or three tiles), and waves with no tile."""
    lens = [1, 33, 100, 129, 300, 555, 700, 1000, 1153, 0, 1280]
    w = workloads.Workload("q40tiles", len(lens), 8, 2, hd, kv_bs, max(lens), ragged=True, table="pool",
                           key=4500 + hd + kv_bs)
    c = build(w, lens=lens, with_cache=False)
    say(f"q40 static tile counts hd={hd} kv_bs={kv_bs}")
    dev, host = dev_cache(c), host_cache(c)
    got = run_decode(c, dev, host, part_tokens=2048)
    assert not got[9].any()


def test_q40_decode_bad_table_entry():
    lens = [40, 17, 33]
    w = workloads.Workload("q40bad", 3, 4, 2, 128, 16, 40, ragged=True, table="pool", key=4500)
    c = build(w, lens=lens, with_cache=False)
    dev, host = dev_cache(c), host_cache(c)
    c.table = c.table.copy()
    c.table[1, 1] = c.num_blocks + 5
    got = q8.q40_decode_attn(to_dev(c.q), dev, to_dev(c.table), to_dev(c.lens), c.scale).cpu().numpy()
    assert np.all(np.isnan(got[1]))
    ok = [0, 2]
    want = q40.decode(c.q[ok], host, c.table[ok], c.lens[ok], c.scale)
    assert float(np.abs(got[ok] - want).max()) <= TOL
