"""Pins for the oracle's decode recurrence (CPU only).

The oracle follows the single-pass recurrence of page "Day 9-2:
flash_attn_single_q_q8_neon" (trdm.cn), section 2, segments 2-3.  It is
pinned against things other than itself:

* C1 the textbook three passes -- all scores, max-subtracted softmax,
  weighted V (llama2.c attention walkthrough, aicoding.csdn.net, sections 2-3)
  -- written separately in numpy float64, reading the pages through numpy
  indexing; the oracle's float64 twin must agree to 1e-6 relative, the fp32
  oracle within 2e-4 absolute;
* C2 seq_len = 1 returns the dequantised V row bit for bit;
* C3 the trace invariants the page's debugging exercise names (the token loop
  runs exactly seq_len times, M never decreases) plus sum_t exp(s_t - M)/S = 1;
* C4 q = 0: every score is 0, so the output is the plain mean of V*vs;
* C5 one K row aligned with q and amplified dominates: out -> its V row;
* C6 brute force on tiny inputs: the definitional softmax evaluated with
  exact rational scores and 40-digit Decimal exponentials;
* the split-range merge: one range is bitwise the plain pass, any split agrees;
* the page walk: permuting physical blocks (and the table with them) leaves
  the output bitwise unchanged; GQA: a group-shared kv head equals the MHA
  cache with that head duplicated (kv head of q head h is h / group);
* the int32 block dots against an int64 numpy product.
A dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of these.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from cases import build, small

SMALL = {
    "tiny": small("tiny", seq_len=200),
    "mha7b": small("mha7b", n_q=8, n_kv=8, seq_len=300),
    "gqa_batch": small("gqa_batch", batch=3, n_q=8, n_kv=2, seq_len=170),
    "long_gqa": small("long_gqa", n_q=16, n_kv=2, seq_len=1000),
    "ragged": small("ragged", batch=6, n_q=16, n_kv=2, seq_len=400),
}


@pytest.fixture(scope="module", params=list(SMALL))
def case(request):
    return build(SMALL[request.param])


def test_c1_single_pass_equals_three_pass(case):
    c = case
    ref = oracle.three_pass_f64(c.q, c.cache, c.table, c.lens, c.scale)
    sp64 = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, use_f64=True)
    assert np.all(np.isfinite(sp64))
    tol = 1e-6 * np.abs(ref).max()
    assert np.abs(sp64 - ref).max() <= tol
    sp32 = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
    assert np.abs(sp32 - ref).max() <= 2e-4


def test_c2_one_token_returns_dequantised_v():
    w = small("gqa_batch", batch=2, n_q=4, n_kv=2, seq_len=1)
    c = build(w)
    out = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
    for b in range(w.batch):
        for h in range(w.n_q):
            k, v, ks, vs = oracle.gather_rows(c.cache, c.table, b, h // w.group, 1)
            want = v[0].astype(np.float32) * np.float32(vs[0])
            assert np.array_equal(out[b, h], want)


def test_c3_trace_invariants(case):
    c = case
    b = int(np.argmax(c.lens))
    L = int(c.lens[b])
    for h in (0, c.w.n_q - 1):
        out, (s, m, S, wts) = oracle.decode_trace(c.q, c.cache, c.table, c.lens, c.scale, b, h)
        assert len(s) == L and np.all(np.isfinite(s))
        assert np.all(np.diff(m.astype(np.float64)) >= 0.0)
        assert m[-1] == s.max() and m[0] == s[0]
        # the exp-sum is the sum of exp(s_t - M_final), to fp32 accumulation error
        total = np.exp(s.astype(np.float64) - float(m[-1])).sum()
        assert abs(total / float(S[-1]) - 1.0) <= L * 2.0 ** -23
        # a new maximum gets weight 1; otherwise exp(s - M) <= 1
        assert np.all(wts[s > np.maximum.accumulate(np.concatenate([[oracle.m_init()], s[:-1]]))] == 1.0)
        assert np.all((wts > 0) & (wts <= 1.0))
        full = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)[b, h]
        assert np.array_equal(out, full)


def test_c4_zero_query_is_uniform_mean():
    w = small("ragged", batch=3, n_q=4, n_kv=2, seq_len=150)
    c = build(w)
    c.q[:] = 0.0
    out = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
    for b in range(w.batch):
        for kh in range(w.n_kv):
            k, v, ks, vs = oracle.gather_rows(c.cache, c.table, b, kh, int(c.lens[b]))
            mean = (v.astype(np.float64) * vs.astype(np.float64)[:, None]).mean(axis=0)
            for h in range(kh * w.group, (kh + 1) * w.group):
                assert np.abs(out[b, h] - mean).max() <= 1e-6 * max(np.abs(mean).max(), 1e-3)


def test_c5_dominant_token():
    w = small("mha7b", n_q=2, n_kv=2, seq_len=64)
    c = build(w, with_cache=False)
    t_star = 37
    for kh in range(w.n_kv):
        c.k_src[0][t_star, kh] = c.q[0, kh] * np.float32(40.0)
    from cases import host_cache
    c.cache = host_cache(c)
    out = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
    for h in range(w.n_q):
        k, v, ks, vs = oracle.gather_rows(c.cache, c.table, 0, h, w.seq_len)
        want = v[t_star].astype(np.float64) * float(vs[t_star])
        assert np.abs(out[0, h] - want).max() < 1e-4


def _decimal_reference(c, b, h):
    """Definitional softmax from the oracle's ints and fp32 scales: scores as
    exact rationals, exponentials in 40-digit Decimal."""
    getcontext().prec = 40
    w = c.w
    L = int(c.lens[b])
    qi, qsc = oracle.quantize_q(c.q[b, h])
    k, v, ks, vs = oracle.gather_rows(c.cache, c.table, b, h // w.group, L)
    scores = []
    for t in range(L):
        s = Fraction(0)
        for blk in range(w.hd // 32):
            d = sum(int(qi[blk * 32 + i]) * int(k[t, blk * 32 + i]) for i in range(32))
            s += d * Fraction(float(qsc[blk]))
        scores.append(s * Fraction(float(ks[t])) * Fraction(c.scale))
    mx = max(scores)
    e = [(Decimal((s - mx).numerator) / Decimal((s - mx).denominator)).exp() for s in scores]
    tot = sum(e)
    out = []
    for i in range(w.hd):
        acc = sum(e[t] * Decimal(int(v[t, i])) * Decimal(float(vs[t])) for t in range(L))
        out.append(float(acc / tot))
    return np.array(out)


@pytest.mark.parametrize("hd,L,G", [(32, 1, 1), (32, 5, 2), (64, 8, 1), (64, 7, 2), (32, 8, 2), (96, 6, 2)])
def test_c6_brute_force_tiny(hd, L, G):
    w = workloads.Workload("bf", 2, 2 * G, 2, hd, 4, L, key=900 + hd + L + G)
    c = build(w, with_cache=False)
    # edges: a zero K row, a duplicated K row (a tie), a clamp-edge value
    c.k_src[0][0, 0] = 0.0
    if L > 2:
        c.k_src[1][2] = c.k_src[1][1]
        c.v_src[1][2, 1, 3] = 1e-9
    c.q[1, 0, :] = 0.0
    c.q[0, -1, 5] = 50.0
    from cases import host_cache
    c.cache = host_cache(c)
    out = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
    for b in range(w.batch):
        for h in range(w.n_q):
            ref = _decimal_reference(c, b, h)
            assert np.abs(out[b, h] - ref).max() <= 2e-6


def test_split_ranges_merge(case):
    c = case
    plain = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
    whole = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, part_tokens=int(c.lens.max()))
    assert np.array_equal(plain, whole)
    ref = oracle.three_pass_f64(c.q, c.cache, c.table, c.lens, c.scale)
    for pt in (1, 16, 33, 128):
        split = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, part_tokens=pt)
        assert np.abs(split - plain).max() <= 2e-5
        assert np.abs(split - ref).max() <= 2e-4


def test_page_walk_invariant_to_physical_placement():
    w = small("gqa_batch", batch=2, n_q=4, n_kv=2, seq_len=90, spare_blocks=3)
    c = build(w)
    out = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
    perm = np.random.default_rng(11).permutation(c.num_blocks)
    moved = oracle.Cache(c.num_blocks, w.n_kv, w.kv_bs, w.hd)
    for f in ("k_pages", "v_pages", "k_scale", "v_scale"):
        arr = getattr(c.cache, f)
        new = np.empty_like(arr)
        new[perm] = arr
        setattr(moved, f, new)
    table = np.where(c.table >= 0, perm[np.maximum(c.table, 0)], -1).astype(np.int32)
    out2 = oracle.decode(c.q, moved, table, c.lens, c.scale)
    assert np.array_equal(out, out2)
    # every referenced row was read, nothing else: poisoned rows never leak
    assert np.all(np.isfinite(out))


def test_gqa_mapping_equals_duplicated_mha():
    w = small("long_gqa", n_q=8, n_kv=2, seq_len=120)
    c = build(w)
    out = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
    mha = oracle.Cache(c.num_blocks, w.n_q, w.kv_bs, w.hd)
    for f in ("k_pages", "v_pages", "k_scale", "v_scale"):
        setattr(mha, f, np.ascontiguousarray(np.repeat(getattr(c.cache, f), w.group, axis=1)))
    out2 = oracle.decode(c.q, mha, c.table, c.lens, c.scale)
    assert np.array_equal(out, out2)
    # and a different grouping (h % n_kv) would not match
    assert not np.array_equal(out[0, 1], out[0, 4])


def test_block_dots_int64_brute_force(case):
    c = case
    dots = oracle.block_dots(c.q, c.cache, c.table, c.lens)
    qi, _ = oracle.quantize_q(c.q)
    w = c.w
    for b in range(w.batch):
        L = int(c.lens[b])
        for kh in range(w.n_kv):
            k, _, _, _ = oracle.gather_rows(c.cache, c.table, b, kh, L)
            kb = k.astype(np.int64).reshape(L, -1, 32)
            for h in range(kh * w.group, (kh + 1) * w.group):
                want = np.einsum("tbi,bi->tb", kb, qi[b, h].astype(np.int64).reshape(-1, 32))
                assert np.array_equal(dots[b, h, :L], want)


def test_openmp_twin_is_bitwise(case):
    c = case
    a = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, threads=1)
    b = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, threads=4)
    assert np.array_equal(a, b)


def test_empty_sequence_gives_zero_row():
    w = small("ragged", batch=3, n_q=4, n_kv=2, seq_len=40)
    c = build(w, lens=[0, 17, 0])
    out = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
    assert not out[0].any() and not out[2].any() and np.all(np.isfinite(out[1]))


def test_q8_error_vs_unquantised_is_small(case):
    # Report-level sanity (the q8-vs-fp32 error is measured, not gated): the
    # q8 output must sit far closer to unquantised attention than an output
    # that ignores the scores altogether (the plain mean of V) does.
    c = case
    out = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
    w = c.w
    ex = np.zeros(out.shape)
    flat = np.zeros(out.shape)
    for b in range(w.batch):
        for h in range(w.n_q):
            k, v = c.k_src[b][:, h // w.group], c.v_src[b][:, h // w.group]
            ex[b, h] = oracle.exact_f64(c.q[b, h], k, v, c.scale)
            flat[b, h] = v.astype(np.float64).mean(axis=0)
    rel = np.linalg.norm(out - ex) / np.linalg.norm(ex)
    rel_flat = np.linalg.norm(flat - ex) / np.linalg.norm(ex)
    assert rel < 0.2 and rel < 0.5 * rel_flat, (rel, rel_flat)


def test_exact_f64_closed_forms():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((9, 16))
    k = np.tile(rng.standard_normal(16), (9, 1))
    assert np.allclose(oracle.exact_f64(rng.standard_normal(16), k, v, 0.25), v.mean(axis=0), atol=1e-12)
    q = rng.standard_normal(16)
    k2 = rng.standard_normal((9, 16))
    k2[4] = q * 1e3
    assert np.allclose(oracle.exact_f64(q, k2, v, 1.0), v[4], atol=1e-12)


def test_three_pass_reference_closed_forms():
    # the float64 three-pass reference on its own: one token returns the
    # dequantised V row; q = 0 gives the plain mean of the dequantised rows
    w = small("gqa_batch", batch=2, n_q=4, n_kv=2, seq_len=1)
    c = build(w)
    ref = oracle.three_pass_f64(c.q, c.cache, c.table, c.lens, c.scale)
    for b in range(2):
        for h in range(4):
            _, v, _, vs = oracle.gather_rows(c.cache, c.table, b, h // 2, 1)
            assert np.allclose(ref[b, h], v[0].astype(np.float64) * float(vs[0]), rtol=0, atol=1e-12)
    w = small("ragged", batch=2, n_q=4, n_kv=2, seq_len=90)
    c = build(w)
    c.q[:] = 0.0
    ref = oracle.three_pass_f64(c.q, c.cache, c.table, c.lens, c.scale)
    for b in range(2):
        for kh in range(2):
            _, v, _, vs = oracle.gather_rows(c.cache, c.table, b, kh, int(c.lens[b]))
            mean = (v.astype(np.float64) * vs.astype(np.float64)[:, None]).mean(axis=0)
            assert np.allclose(ref[b, 2 * kh], mean, rtol=0, atol=1e-12)
