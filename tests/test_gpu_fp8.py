"""GPU parity of the FP8 KV codec (q8kv_fp8_append, q8kv_fp8_decode_attn).

* Append: the device pages (read back in row order through the byte map
  include/q8kv.h defines) and UE8M0 scale bytes against the oracle's
  (oracle/fp8kv.py), bit for bit: rows of unit normals, rows whose 64-element
  blocks span 2^-30 .. 2^30 in magnitude, all-zero blocks, exact powers of
  two times 448, ties between E4M3 neighbours, bf16 sources.
* Decode: the output against the oracle's fp64 definition (softmax over the
  dequantised K and V) within 2e-4 max-abs, on every hd, group sizes 1-8,
  kv_bs 16-256, split plans on both merge paths, the persistent grid, empty
  sequences and an out-of-pool table entry (NaN row for that sequence only).
"""
import numpy as np
import pytest
import torch

import decode_attention_int8_amd as q8
import workloads
from cases import build
from gpu_cases import DEV, natural_fp8_pages, say, to_dev
from oracle import fp8kv

pytestmark = pytest.mark.gpu

TOL = 2e-4


def dev_cache(c, src_dtype=torch.float32, fill=0x7F):
    w = c.w
    cache = q8.Fp8KVCache(c.num_blocks, w.n_kv, w.kv_bs, w.hd, device=DEV)
    cache.k_pages.fill_(fill)
    cache.v_pages.fill_(fill)
    cache.k_scale.fill_(0xFF)
    cache.v_scale.fill_(0xFF)
    for b in range(w.batch):
        if len(c.slots[b]):
            cache.append(to_dev(c.k_src[b], src_dtype), to_dev(c.v_src[b], src_dtype), to_dev(c.slots[b]))
    return cache


def host_cache(c, src_dtype=torch.float32):
    w = c.w
    h = fp8kv.Fp8Cache(c.num_blocks, w.n_kv, w.kv_bs, w.hd)
    for b in range(w.batch):
        if len(c.slots[b]):
            k, v = c.k_src[b], c.v_src[b]
            if src_dtype == torch.bfloat16:
                k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
                v = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
            h.append(k, v, c.slots[b])
    return h


def assert_fp8_cache_equal(host, dev):
    for f in ("k_pages", "v_pages"):
        got = natural_fp8_pages(getattr(dev, f).cpu().numpy(), f[0])
        want = getattr(host, f)
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{f}: {len(bad)} bytes differ, first at {bad[0].tolist()}: " \
                              f"{got[tuple(bad[0])]:#04x} vs {want[tuple(bad[0])]:#04x}"
    for f in ("k_scale", "v_scale"):
        assert np.array_equal(getattr(dev, f).cpu().numpy(), getattr(host, f)), f


def run_decode(c, dev, host, part_tokens=0):
    q, bt, sl = to_dev(c.q), to_dev(c.table), to_dev(c.lens)
    got = q8.fp8_decode_attn(q, dev, bt, sl, c.scale, part_tokens=part_tokens)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = fp8kv.decode(c.q, host, c.table, c.lens, c.scale)
    assert np.all(np.isfinite(got))
    err = float(np.abs(got - want).max()) if got.size else 0.0
    assert err <= TOL, f"max-abs error {err:.3g} > {TOL}"
    return got, err


def special_rows(rng, n, hd):
    """Rows whose 64-element blocks stress the codec: wide magnitude ranges,
    zero blocks, exact 448 * 2^k maxima, E4M3 midpoints."""
    rows = rng.standard_normal((n, hd)).astype(np.float32)
    nb = hd // 64
    for i in range(n):
        for blk in range(nb):
            seg = rows[i, 64 * blk:64 * (blk + 1)]
            kind = (i + blk) % 5
            if kind == 0:
                seg *= np.float32(2.0 ** rng.integers(-30, 31))
            elif kind == 1:
                seg[:] = 0
            elif kind == 2:
                seg[0] = np.float32(448.0 * 2.0 ** rng.integers(-10, 10))
                seg[1:] = np.clip(seg[1:], -abs(seg[0]) * 0.9, abs(seg[0]) * 0.9)
            elif kind == 3:
                # midpoints between neighbouring E4M3 values at scale 2^0
                # (the block max 448 fixes e = 0)
                seg[0] = 448.0
                seg[1:9] = [1.0625, 1.1875, 2.125, -2.375, 0.01171875, 208.0, 3.0 * 2 ** -10, -5.0 * 2 ** -10]
            else:
                seg[5] = -seg.__abs__().max() * 1.0000001
    return rows


@pytest.mark.parametrize("hd,kv_bs,n_kv,dtype", [
    (128, 16, 2, torch.float32), (64, 32, 3, torch.float32), (256, 64, 2, torch.float32),
    (128, 16, 2, torch.bfloat16), (256, 16, 1, torch.bfloat16),
])
def test_fp8_append_bit_exact(hd, kv_bs, n_kv, dtype):
    w = workloads.Workload("fp8app", 3, n_kv, n_kv, hd, kv_bs, 3 * kv_bs + 5, ragged=True, table="pool",
                           key=2000 + hd + kv_bs)
    c = build(w, with_cache=False)
    rng = np.random.default_rng(2100 + hd)
    for b in range(w.batch):
        L = len(c.slots[b])
        if L:
            c.k_src[b] = special_rows(rng, L * n_kv, hd).reshape(L, n_kv, hd)
            c.v_src[b] = special_rows(rng, L * n_kv, hd).reshape(L, n_kv, hd)
    say(f"fp8 append hd={hd} kv_bs={kv_bs} n_kv={n_kv} dtype={dtype} lens={c.lens.tolist()}")
    dev = dev_cache(c, dtype)
    host = host_cache(c, dtype)
    assert_fp8_cache_equal(host, dev)


def test_fp8_append_every_code():
    """Rows that hit every finite E4M3 code: block max 448 (e = 0) and the
    other 63 elements walk the code table."""
    hd, n = 128, 8
    vals = np.array([fp8kv.e4m3_value(cd) for cd in range(256) if not np.isnan(fp8kv.e4m3_value(cd))],
                    np.float32)
    rows = np.zeros((n, hd), np.float32)
    flat = np.resize(vals, n * 2 * 63)
    for i in range(n):
        for blk in range(2):
            rows[i, 64 * blk] = 448.0
            rows[i, 64 * blk + 1:64 * (blk + 1)] = flat[(2 * i + blk) * 63:(2 * i + blk + 1) * 63]
    w = workloads.Workload("fp8codes", 1, 1, 1, hd, 16, n, key=2200)
    c = build(w, with_cache=False)
    c.k_src[0] = rows.reshape(n, 1, hd)
    c.v_src[0] = -rows.reshape(n, 1, hd)
    dev = dev_cache(c)
    host = host_cache(c)
    assert_fp8_cache_equal(host, dev)


SMALL = {
    "mha": dict(batch=1, n_q=8, n_kv=8, hd=128, kv_bs=16, seq_len=300),
    "gqa": dict(batch=3, n_q=8, n_kv=2, hd=128, kv_bs=16, seq_len=170),
    "long": dict(batch=1, n_q=16, n_kv=2, hd=128, kv_bs=64, seq_len=1000),
    "ragged": dict(batch=6, n_q=16, n_kv=2, hd=128, kv_bs=64, seq_len=400),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_fp8_decode_small(name):
    kw = SMALL[name]
    w = workloads.Workload("fp8_" + name, kw["batch"], kw["n_q"], kw["n_kv"], kw["hd"], kw["kv_bs"],
                           kw["seq_len"], ragged=name in ("gqa", "ragged"), table="pool", key=2300 + len(name))
    c = build(w, with_cache=False)
    say(f"fp8 decode {name} lens={c.lens.tolist()}")
    dev, host = dev_cache(c), host_cache(c)
    assert_fp8_cache_equal(host, dev)
    run_decode(c, dev, host)
    run_decode(c, dev, host, part_tokens=64)


@pytest.mark.parametrize("hd,G,kv_bs", [(64, 1, 16), (64, 8, 32), (128, 3, 16), (128, 8, 128),
                                        (256, 2, 64), (256, 8, 16), (128, 5, 256),
                                        (128, 16, 64), (64, 12, 16)])  # more heads than one MFMA column set
def test_fp8_decode_shapes(hd, G, kv_bs):
    lens = [1, 0, 16, 17, 33, kv_bs, kv_bs + 1, 2 * kv_bs + 7, 300]
    w = workloads.Workload("fp8shape", len(lens), 2 * G, 2, hd, kv_bs, max(lens), ragged=True, table="pool",
                           key=2400 + hd + G + kv_bs)
    c = build(w, lens=lens, with_cache=False)
    say(f"fp8 decode hd={hd} G={G} kv_bs={kv_bs}")
    dev, host = dev_cache(c), host_cache(c)
    got, _ = run_decode(c, dev, host)
    assert not got[1].any()
    for pt in (32, 96):
        run_decode(c, dev, host, part_tokens=pt)


@pytest.mark.parametrize("hd", [128, 64, 256])
def test_fp8_decode_persistent_grid(hd):
    """More items than resident workgroups (the persistent kernel's rolled
    tile loop) at every page width."""
    rng = np.random.default_rng(2500 + hd)
    lens = [int(x) for x in rng.integers(1, 600, size=64)]
    lens[:5] = [0, 1, 32, 33, 64]
    w = workloads.Workload("fp8persist", 64, 8, 2, hd, 16, 600, ragged=True, table="pool", key=2500 + hd)
    c = build(w, lens=lens, with_cache=False)
    dev, host = dev_cache(c), host_cache(c)
    for pt in (32, 64):
        a, _ = run_decode(c, dev, host, part_tokens=pt)
        b, _ = run_decode(c, dev, host, part_tokens=pt)
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_fp8_decode_wide_magnitudes():
    """K and V rows whose blocks span 2^-30 .. 2^30: the per-block exponents
    must reach the scores and the weights exactly."""
    w = workloads.Workload("fp8wide", 2, 8, 2, 128, 16, 90, key=2600)
    c = build(w, with_cache=False)
    rng = np.random.default_rng(2601)
    for b in range(2):
        L = len(c.slots[b])
        k = c.k_src[b] * np.exp2(rng.integers(-6, 7, size=(L, 2, 1))).astype(np.float32)
        v = c.v_src[b] * np.exp2(rng.integers(-30, 31, size=(L, 2, 1))).astype(np.float32)
        c.k_src[b], c.v_src[b] = k, v
    dev, host = dev_cache(c), host_cache(c)
    q, bt, sl = to_dev(c.q), to_dev(c.table), to_dev(c.lens)
    got = q8.fp8_decode_attn(q, dev, bt, sl, c.scale).cpu().numpy()
    want = fp8kv.decode(c.q, host, c.table, c.lens, c.scale)
    # V spans 2^60: compare relative to each output row's largest value
    rel = np.abs(got - want) / np.maximum(np.abs(want).max(-1, keepdims=True), 1e-30)
    assert float(rel.max()) <= 1e-4


def test_fp8_decode_bad_table_entry():
    lens = [40, 17, 33]
    w = workloads.Workload("fp8bad", 3, 4, 2, 128, 16, 40, ragged=True, table="pool", key=2700)
    c = build(w, lens=lens, with_cache=False)
    dev, host = dev_cache(c), host_cache(c)
    c.table = c.table.copy()
    c.table[1, 1] = c.num_blocks + 5
    got = q8.fp8_decode_attn(to_dev(c.q), dev, to_dev(c.table), to_dev(c.lens), c.scale).cpu().numpy()
    assert np.all(np.isnan(got[1]))
    ok = [0, 2]
    want = fp8kv.decode(c.q[ok], host, c.table[ok], c.lens[ok], c.scale)
    assert float(np.abs(got[ok] - want).max()) <= TOL
