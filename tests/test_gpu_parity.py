"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

* quantisation and integer dot products are compared bit for bit: the paged
  K/V rows and scales written by q8kv_append, the decode prologue's int8
  query and block scales, and the int32 per-32-block dots of the matrix-core
  scoring step;
* decode outputs are compared element by element with the oracle's fp32
  single pass, max-abs error <= 2e-4 (unit-scale V);
* edge cases: lengths around tiles, pages and partitions, every head-group
  size, every hd x kv_bs, forced split plans, empty sequences, poisoned
  unreferenced rows, an out-of-range table entry, determinism.
"""
import numpy as np
import pytest
import torch

import decode_attention_int8_amd as q8
import oracle
import workloads
from cases import build, small
from gpu_cases import DEV, assert_cache_equal, decode, dev_inputs, gpu_cache, say, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-4
# The GPU against the oracle's fp64 twin (same int8 inputs and fp32 scales).
# The fp32 oracle itself drifts from fp64 by up to ~1.8e-4 on long peaked
# contexts (tail terms far below an ulp of the accumulator vanish one token at
# a time); the kernel adds 32 tokens per matrix-core step and stays ~1e-6 away.
TOL64 = 2e-5

SMALL = {
    "tiny": small("tiny", seq_len=200),
    "mha7b": small("mha7b", n_q=8, n_kv=8, seq_len=300),
    "gqa_batch": small("gqa_batch", batch=3, n_q=8, n_kv=2, seq_len=170),
    "long_gqa": small("long_gqa", n_q=16, n_kv=2, seq_len=1000),
    "ragged": small("ragged", batch=6, n_q=16, n_kv=2, seq_len=400),
}


def check_decode(c, cache=None, part_tokens=0, tol=TOL, tol64=TOL64):
    if cache is None:
        cache = gpu_cache(c)
    got = decode(c, cache, part_tokens=part_tokens)
    want = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, threads=8)
    want64 = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, use_f64=True, threads=8)
    assert np.all(np.isfinite(got)), "non-finite output"
    err = float(np.abs(got - want).max()) if got.size else 0.0
    err64 = float(np.abs(got - want64).max()) if got.size else 0.0
    assert err <= tol, f"max-abs error {err:.3g} > {tol} (fp32 oracle)"
    assert err64 <= tol64, f"max-abs error {err64:.3g} > {tol64} (fp64 oracle)"
    return err


@pytest.mark.parametrize("hd,kv_bs,n_kv,dtype", [
    (128, 16, 2, torch.float32), (128, 64, 8, torch.float32), (64, 16, 1, torch.float32),
    (256, 32, 7, torch.float32), (128, 16, 2, torch.bfloat16), (256, 128, 3, torch.bfloat16),
    # head sizes stored in padded pages (hd rounded up to 64, 128 or 256)
    (32, 16, 3, torch.float32), (96, 64, 2, torch.float32), (160, 32, 2, torch.bfloat16),
    (192, 16, 5, torch.float32), (224, 128, 1, torch.float32),
])
def test_append_bit_exact(hd, kv_bs, n_kv, dtype):
    w = workloads.Workload("app", 3, n_kv, n_kv, hd, kv_bs, 5 * kv_bs + 3, ragged=True,
                           table="pool", spare_blocks=4, key=300 + hd + kv_bs + n_kv)
    c = build(w, with_cache=False)
    if dtype == torch.bfloat16:
        bits = [to_dev(k).to(torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16) for k in c.k_src]
        vbits = [to_dev(v).to(torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16) for v in c.v_src]
        host = oracle.Cache(c.num_blocks, n_kv, kv_bs, hd, fill_int8=127, fill_scale=np.nan)
        for b in range(w.batch):
            host.append(bits[b], vbits[b], c.slots[b])
    else:
        from cases import host_cache
        host = host_cache(c)
    say(f"append hd={hd} kv_bs={kv_bs} n_kv={n_kv} {dtype}")
    dev = gpu_cache(c, src_dtype=dtype)
    torch.cuda.synchronize()
    assert_cache_equal(host, dev)


def test_append_skips_negative_and_out_of_pool_slots():
    w = workloads.Workload("skip", 1, 2, 2, 128, 16, 40, key=320)
    c = build(w)
    slots = c.slots[0].copy()
    slots[3] = -1
    slots[7] = c.num_blocks * w.kv_bs  # past the pool
    dev = q8.PagedKVCache(c.num_blocks, 2, 16, 128, device=DEV)
    for t in (dev.k_pages, dev.v_pages):
        t.fill_(127)
    for t in (dev.k_scale, dev.v_scale):
        t.fill_(float("nan"))
    dev.append(to_dev(c.k_src[0]), to_dev(c.v_src[0]), to_dev(slots))
    host = oracle.Cache(c.num_blocks, 2, 16, 128, fill_int8=127, fill_scale=np.nan)
    keep = slots >= 0
    keep &= slots < c.num_blocks * 16
    host.append(c.k_src[0][keep], c.v_src[0][keep], slots[keep])
    torch.cuda.synchronize()
    assert_cache_equal(host, dev)


@pytest.mark.parametrize("hd", [64, 128, 256])
def test_quantize_q_bit_exact(hd):
    rng = np.random.default_rng(hd)
    q = rng.standard_normal((37, hd)).astype(np.float32)
    q[3] = 0.0
    q[5, :32] = 5e-7
    q[6] *= 1e-3
    q[7] *= 1e4
    q[8, 40] = 0.5 * np.abs(q[8, 32:64]).max()
    say(f"quantize_q hd={hd}")
    qi, qsc = q8.debug_quantize_q(to_dev(q))
    torch.cuda.synchronize()
    want_qi, want_sc = oracle.quantize_q(q)
    assert np.array_equal(qi.cpu().numpy(), want_qi)
    assert np.array_equal(qsc.cpu().numpy().view(np.uint32), want_sc.view(np.uint32))


@pytest.mark.parametrize("name", list(SMALL))
def test_block_dots_bit_exact(name):
    c = build(SMALL[name])
    cache = gpu_cache(c)
    q, bt, sl = dev_inputs(c)
    max_tok = int(c.lens.max())
    say(f"block dots {name}")
    got = q8.debug_block_dots(q, cache, bt, sl, max_tok).cpu().numpy()
    want = oracle.block_dots(c.q, c.cache, c.table, c.lens, max_tok)
    for b in range(c.w.batch):
        L = int(c.lens[b])
        assert np.array_equal(got[b, :, :L], want[b, :, :L])


@pytest.mark.parametrize("hd,G", [(64, 8), (256, 3), (128, 1), (128, 5)])
def test_block_dots_other_shapes(hd, G):
    w = workloads.Workload("dots", 2, 2 * G, 2, hd, 32, 77, ragged=True, table="pool", key=400 + hd + G)
    c = build(w)
    cache = gpu_cache(c)
    q, bt, sl = dev_inputs(c)
    say(f"block dots hd={hd} G={G}")
    got = q8.debug_block_dots(q, cache, bt, sl, 77).cpu().numpy()
    want = oracle.block_dots(c.q, c.cache, c.table, c.lens, 77)
    for b in range(2):
        L = int(c.lens[b])
        assert np.array_equal(got[b, :, :L], want[b, :, :L])


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_small_workloads(name):
    c = build(SMALL[name])
    say(f"decode {name} lens={c.lens.tolist()[:8]}")
    dev = gpu_cache(c)
    torch.cuda.synchronize()
    assert_cache_equal(c.cache, dev)
    check_decode(c, dev)
    for pt in (32, 96):
        check_decode(c, dev, part_tokens=pt)


@pytest.mark.parametrize("name", ["gqa_batch", "ragged"])
def test_decode_attn_entry_point(name):
    """q8kv_decode_attn itself, called through the C ABI with raw pointers
    (the binding's decode goes through q8kv_decode_attn_split): the oracle's
    parity bar, and bit for bit what the split entry gives with the automatic
    plan (part_tokens 0)."""
    c = build(SMALL[name])
    say(f"q8kv_decode_attn {name}")
    dev = gpu_cache(c)
    q, bt, sl = dev_inputs(c)
    out = torch.full_like(q, float("nan"))
    st = torch.cuda.current_stream(DEV).cuda_stream
    rc = q8.lib.q8kv_decode_attn(out.data_ptr(), q.data_ptr(), dev.k_pages.data_ptr(), dev.v_pages.data_ptr(),
                                 dev.k_scale.data_ptr(), dev.v_scale.data_ptr(), bt.data_ptr(), sl.data_ptr(),
                                 bt.shape[1], dev.num_blocks, c.w.batch, c.w.n_q, c.w.n_kv, c.w.hd, c.w.kv_bs,
                                 c.scale, st)
    assert rc == q8.Q8KV_OK, q8.last_error()
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), decode(c, dev).view(np.uint32))
    want = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, threads=8)
    want64 = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, use_f64=True, threads=8)
    assert float(np.abs(got - want).max()) <= TOL
    assert float(np.abs(got - want64).max()) <= TOL64


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_edge_lengths(G):
    lens = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 300]
    w = workloads.Workload("edge", len(lens), 2 * G, 2, 128, 16, 320, ragged=True, table="pool",
                           spare_blocks=5, key=500 + G)
    c = build(w, lens=lens)
    say(f"edge lengths G={G}")
    dev = gpu_cache(c)
    for pt in (0, 32, 64, 128):
        check_decode(c, dev, part_tokens=pt)


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("kv_bs", [16, 32, 64, 128, 256])
def test_decode_hd_kv_bs(hd, kv_bs):
    w = workloads.Workload("hdbs", 3, 8, 2, hd, kv_bs, 2 * kv_bs + 37, ragged=True, table="pool",
                           spare_blocks=2, k_outlier_p=0.05, k_outlier_amp=6.0,
                           key=600 + hd + kv_bs)
    c = build(w)
    say(f"decode hd={hd} kv_bs={kv_bs} lens={c.lens.tolist()}")
    dev = gpu_cache(c)
    check_decode(c, dev)
    check_decode(c, dev, part_tokens=64)


@pytest.mark.parametrize("hd,kv_bs", [(32, 16), (32, 256), (96, 16), (96, 64), (160, 32), (192, 128),
                                      (224, 16), (224, 256)])
def test_decode_padded_head_sizes(hd, kv_bs):
    """Head sizes that are multiples of 32 but not of 64, 128 or 256 live in
    pages hd rounded up to 64, 128 or 256 wide whose pad columns hold zero
    codes: q and out stay hd floats a row, and the results are those of the
    unpadded oracle."""
    w = workloads.Workload("padhd", 3, 8, 2, hd, kv_bs, 2 * kv_bs + 37, ragged=True, table="pool",
                           spare_blocks=2, k_outlier_p=0.05, k_outlier_amp=6.0,
                           key=1600 + hd + kv_bs)
    c = build(w)
    say(f"decode padded hd={hd} kv_bs={kv_bs} lens={c.lens.tolist()}")
    dev = gpu_cache(c)
    assert dev.k_pages.shape[-1] == q8.page_hd(hd) > hd
    check_decode(c, dev)
    check_decode(c, dev, part_tokens=64)


def test_decode_padded_persistent_grid():
    """A padded head size on the persistent grid with the in-kernel merge
    and the combine kernel."""
    rng = np.random.default_rng(1700)
    lens = rng.integers(1, 1025, size=64)
    lens[:6] = [0, 1, 31, 32, 33, 1024]
    w = workloads.Workload("padpersist", 64, 8, 2, 96, 32, 1024, ragged=True, table="pool",
                           spare_blocks=3, key=1700)
    c = build(w, lens=[int(x) for x in lens])
    say(f"persistent grid hd=96 tokens={int(c.lens.sum())}")
    dev = gpu_cache(c)
    for pt in (32, 128):
        got = decode(c, dev, part_tokens=pt)
        assert not got[0].any()
        check_decode(c, dev, part_tokens=pt)


@pytest.mark.parametrize("hd,G", [(64, 1), (64, 8), (128, 1), (128, 3), (128, 5), (128, 8),
                                  (256, 2), (256, 5), (256, 8),
                                  (32, 8), (96, 3), (96, 8), (160, 5), (192, 8), (224, 2)])
def test_decode_split_merge_paths(hd, G):
    """Partition states of a (sequence, head group) are merged inside the
    decode kernel by the workgroup that stores the last one when there are
    at most 64 of them (partitions x query heads), else by the combine
    kernel.  The partition lengths here give 3 to 19 partitions, so each
    shape takes one or both paths, the in-kernel one with one or several
    float4 slices per thread; each call is made twice, since the merge
    leaves its arrival counters at zero for the next call."""
    w = workloads.Workload("merge", 3, 2 * G, 2, hd, 32, 600, ragged=True, table="pool",
                           key=800 + hd + G)
    c = build(w)
    say(f"split merge hd={hd} G={G} lens={c.lens.tolist()}")
    dev = gpu_cache(c)
    for pt in (32, 64, 128, 192):
        first = decode(c, dev, part_tokens=pt)
        again = decode(c, dev, part_tokens=pt)
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
        check_decode(c, dev, part_tokens=pt)


@pytest.mark.parametrize("G,kv_bs", [(4, 16), (1, 32), (8, 64)])
def test_decode_persistent_grid(G, kv_bs):
    """Shapes with more (sequence, kv head, partition) items than fit on the
    device at once run on the persistent grid, whose item order puts every
    full partition first and the partial last partitions after them by
    decreasing length.  64 sequences of up to 1024 tokens split into 32-96
    token partitions give 1300-4100 items; the lengths include empty
    sequences, exact multiples of the partition length and sequences shorter
    than one partition."""
    rng = np.random.default_rng(900 + G + kv_bs)
    lens = rng.integers(1, 1025, size=64)
    lens[:12] = [0, 1, 31, 32, 33, 96, 192, 1024, 0, 95, 97, 1000]
    w = workloads.Workload("persist", 64, 2 * G, 2, 128, kv_bs, 1024, ragged=True, table="pool",
                           spare_blocks=3, key=900 + G + kv_bs)
    c = build(w, lens=[int(x) for x in lens])
    say(f"persistent grid G={G} kv_bs={kv_bs} tokens={int(c.lens.sum())}")
    dev = gpu_cache(c)
    for pt in (32, 64, 96):
        got = decode(c, dev, part_tokens=pt)
        assert not got[0].any() and not got[8].any()
        again = decode(c, dev, part_tokens=pt)
        assert np.array_equal(got.view(np.uint32), again.view(np.uint32))
        check_decode(c, dev, part_tokens=pt)


def test_decode_max_batch():
    """2048 sequences, the most one call takes: the persistent grid's
    per-sequence prefix sums and remainder classes in LDS at their full size,
    with empty sequences and a spread of lengths."""
    rng = np.random.default_rng(950)
    lens = rng.integers(0, 97, size=2048)
    lens[:6] = [0, 1, 32, 33, 96, 64]
    w = workloads.Workload("maxbatch", 2048, 8, 2, 128, 16, 96, ragged=True, table="pool", key=950)
    c = build(w, lens=[int(x) for x in lens])
    say(f"max batch 2048 tokens={int(c.lens.sum())}")
    dev = gpu_cache(c)
    for pt in (0, 32):
        got = decode(c, dev, part_tokens=pt)
        assert not got[0].any()
        check_decode(c, dev, part_tokens=pt)


@pytest.mark.parametrize("hd,G", [(64, 1), (128, 8), (256, 4)])
def test_decode_max_partitions(hd, G):
    """256 partitions of one sequence, the most a call plans: the combine
    kernel's per-thread state arrays at their full length for every hd."""
    w = workloads.Workload("maxparts", 2, 2 * G, 2, hd, 32, 256 * 32, ragged=True, table="pool", key=960 + hd)
    c = build(w, lens=[256 * 32, 5000])
    say(f"max partitions hd={hd} G={G}")
    dev = gpu_cache(c)
    check_decode(c, dev, part_tokens=32)


@pytest.mark.parametrize("hd,G,n_kv,lens,pt", [
    (128, 8, 2, [256 * 32, 5000, 300, 0], 32),   # 256 partitions: runs of 16
    (128, 8, 4, [128 * 64], 64),                 # the 128K step's plan: 512 static items, 128 partitions
    (64, 1, 2, [100 * 32, 70 * 32 + 5, 64], 32),  # one head: 100 states, runs of 10
    (256, 8, 1, [40 * 64 + 3, 9 * 64], 64),      # hd 256: two slices per thread
    (128, 3, 2, [30 * 32, 23 * 32 - 1, 1, 0], 32),
    (64, 8, 1, [9 * 32, 17 * 32 + 1], 32),       # just past the one-level limit
])
def test_decode_many_partition_states(hd, G, n_kv, lens, pt):
    """Groups of more than 64 partition states (the 128K step's plan among
    them) go to the combine kernel, static and persistent grids alike:
    checked against the oracle and repeated bit for bit over several
    calls."""
    w = workloads.Workload("merge2", len(lens), n_kv * G, n_kv, hd, 32 if pt == 32 else 64, max(lens),
                           ragged=True, table="pool", key=1100 + hd + G + n_kv)
    c = build(w, lens=lens)
    say(f"many partition states hd={hd} G={G} n_kv={n_kv} lens={lens} part_tokens={pt}")
    dev = gpu_cache(c)
    first = decode(c, dev, part_tokens=pt)
    for _ in range(4):
        again = decode(c, dev, part_tokens=pt)
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
    check_decode(c, dev, part_tokens=pt)


def test_decode_many_partition_states_persistent():
    """Many partition states on the persistent grid: 24 sequences of up to
    6000 tokens in 32-token partitions are ~9000 items, more than fit at
    once."""
    rng = np.random.default_rng(1200)
    lens = [int(x) for x in rng.integers(1, 6001, size=24)]
    lens[:4] = [6000, 0, 33, 64 * 32]
    w = workloads.Workload("merge2p", 24, 16, 2, 128, 32, 6000, ragged=True, table="pool", key=1200)
    c = build(w, lens=lens)
    say(f"many partition states, persistent grid, tokens={int(c.lens.sum())}")
    dev = gpu_cache(c)
    first = decode(c, dev, part_tokens=32)
    assert not first[1].any()
    again = decode(c, dev, part_tokens=32)
    assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
    check_decode(c, dev, part_tokens=32)


@pytest.mark.parametrize("hd,G,n_kv,pt", [
    (128, 16, 2, 0), (128, 16, 2, 64),   # two groups of 8 heads per kv head
    (64, 12, 1, 32),                     # two groups of 6
    (256, 10, 1, 0),                     # two groups of 5
    (128, 32, 1, 0),                     # one kv head for 32 query heads: four groups of 8
    (128, 13, 1, 64),                    # a prime group size: thirteen groups of 1
    (96, 12, 1, 32),                     # a padded head size in groups of 6
])
def test_decode_large_groups(hd, G, n_kv, pt):
    """More query heads per kv head than the matrix cores' 8-head column
    set: the heads are split into equal groups (the largest divisor of G up
    to 8 heads), each its own work item over the same K/V."""
    lens = [1, 0, 31, 300, 700, 1500]
    w = workloads.Workload("biggroup", len(lens), n_kv * G, n_kv, hd, 32, max(lens), ragged=True, table="pool",
                           key=1400 + hd + G)
    c = build(w, lens=lens)
    say(f"large group hd={hd} G={G} n_kv={n_kv} part_tokens={pt}")
    dev = gpu_cache(c)
    got = decode(c, dev, part_tokens=pt)
    assert not got[1].any()
    check_decode(c, dev, part_tokens=pt)


@pytest.mark.parametrize("amp", [1e-6, 1e-3, 1e3, 1e4, 1e6])
def test_decode_v_amplitude(amp):
    """V rows scaled by amp: V scales absmax / 127 from ~1e-8 to ~4e4.  The
    P.V weights are carried as f16 (hi, lo) pairs of w * v_scale; they must
    neither overflow (V scales of 256 and more once made whole rows NaN) nor
    lose precision in the f16 subnormals (tiny V scales).  The output is
    checked against the oracle's fp64 twin relative to the output's size."""
    w = workloads.Workload("vamp", 3, 16, 2, 128, 32, 700, ragged=True, table="pool", key=1300)
    c = build(w, lens=[700, 333, 64], with_cache=False)
    for b in range(w.batch):
        c.v_src[b] = (c.v_src[b] * np.float32(amp)).astype(np.float32)
    from cases import host_cache
    c.cache = host_cache(c)
    say(f"V amplitude {amp:g}")
    dev = gpu_cache(c)
    for pt in (0, 64):
        got = decode(c, dev, part_tokens=pt)
        want64 = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, use_f64=True, threads=8)
        assert np.all(np.isfinite(got))
        ref = float(np.abs(want64).max())
        err = float(np.abs(got - want64).max())
        assert err <= 2e-5 * ref, f"amp {amp:g} split {pt}: max-abs error {err:.3g} vs output size {ref:.3g}"


def test_decode_mixed_v_amplitudes():
    """Tokens whose V rows span 2^-20 .. 2^20 in one sequence (the largest
    V scale of each tile varies, so the kernel's V-scale exponent grows
    mid-sequence): against the oracle's fp64 twin relative to the output."""
    w = workloads.Workload("vmix", 2, 16, 2, 128, 32, 900, ragged=True, table="pool", key=1310)
    c = build(w, lens=[900, 517], with_cache=False)
    rng = np.random.default_rng(1310)
    for b in range(w.batch):
        f = np.exp2(rng.uniform(-20, 20, size=(c.v_src[b].shape[0], 1, 1))).astype(np.float32)
        c.v_src[b] = (c.v_src[b] * f).astype(np.float32)
    from cases import host_cache
    c.cache = host_cache(c)
    dev = gpu_cache(c)
    got = decode(c, dev, part_tokens=64)
    want64 = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, use_f64=True, threads=8)
    assert np.all(np.isfinite(got))
    for b in range(w.batch):
        for h in range(w.n_q):
            ref = float(np.abs(want64[b, h]).max())
            err = float(np.abs(got[b, h] - want64[b, h]).max())
            assert err <= 2e-5 * ref, f"seq {b} head {h}: {err:.3g} vs {ref:.3g}"


def test_decode_long_peaked_tail_precision():
    """Long contexts whose softmax is dominated by a few tokens put most of
    the sequence into tiny weights.  Their P.V weights must not fall into the
    f16 subnormals (2^-24 steps), or the rounding of tens of thousands of
    them adds up: 3.9e-5 from fp64 on sequence 23 of the ragged workload
    (lognormal K channels) before the kernel offset the weight exponent,
    4e-6 after.  Sequences 23 and 62 of that workload, all 64 heads; the
    other sequences are empty."""
    w = workloads.WORKLOADS["ragged"]
    full = workloads.seq_lens(w)
    lens = np.zeros_like(full)
    lens[[23, 62]] = full[[23, 62]]
    c = build(w, lens=lens)
    say(f"long peaked tails lens={lens[[23, 62]].tolist()}")
    dev = gpu_cache(c)
    check_decode(c, dev, tol64=1e-5)


def test_decode_empty_sequences_give_zero_rows():
    w = workloads.Workload("empty", 4, 8, 2, 128, 16, 100, ragged=True, table="pool", key=700)
    c = build(w, lens=[0, 50, 0, 100])
    dev = gpu_cache(c)
    got = decode(c, dev)
    assert not got[0].any() and not got[2].any()
    check_decode(c, dev)
    check_decode(c, dev, part_tokens=32)


def test_decode_bad_table_entry_gives_nan_row_only():
    w = workloads.Workload("bad", 3, 4, 2, 128, 16, 64, key=710)
    c = build(w)
    dev = gpu_cache(c)
    table = c.table.copy()
    table[1, 2] = c.num_blocks + 5
    q, _, sl = dev_inputs(c)
    for pt in (0, 32):
        out = q8.decode_attn(q, dev, to_dev(table), sl, c.scale, part_tokens=pt).cpu().numpy()
        assert np.all(np.isnan(out[1]))
        want = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
        assert np.abs(out[[0, 2]] - want[[0, 2]]).max() <= TOL
    # a length past the table's capacity is flagged the same way
    lens = c.lens.copy()
    lens[2] = w.max_blocks * w.kv_bs + 1
    out = q8.decode_attn(q, dev, to_dev(c.table), to_dev(lens), c.scale).cpu().numpy()
    assert np.all(np.isnan(out[2])) and np.all(np.isfinite(out[:2]))


def test_decode_deterministic():
    c = build(SMALL["ragged"])
    dev = gpu_cache(c)
    a = decode(c, dev)
    b = decode(c, dev)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_decode_zero_query_and_dominant_token():
    w = small("long_gqa", n_q=8, n_kv=1, seq_len=700)
    c = build(w, with_cache=False)
    c.q[0, :4] = 0.0
    c.k_src[0][333, 0] = c.q[0, 5] * np.float32(30.0)
    from cases import host_cache
    c.cache = host_cache(c)
    dev = gpu_cache(c)
    check_decode(c, dev)
    check_decode(c, dev, part_tokens=64)
