"""Pins of the q4_0 codec oracle (oracle/q40.py).

* Quantiser properties that follow from the block format rather than from
  its formula: codes stay in 0..15; the block's first element of largest
  magnitude gets code 0 and comes back exactly up to the fp16 rounding of d;
  every other element comes back within half a step |d| / 2 (a full step
  where the top code saturates at 15); an all-zero block is code 8 with
  d = 0; a block made of exact multiples (c - 8) * d of an fp16-exact d
  returns its codes; negating a block keeps d's magnitude.
* Decode: a cache whose rows use one fp16-exact scale for all their blocks is
  the same attention as an int8 cache with codes c - 8 and that scale, so
  the q4_0 decode must equal the independent three-pass fp64 reference of
  the int8 oracle (oracle.three_pass_f64) on it; one token returns its
  dequantised V row; a zero query gives the mean of the dequantised rows;
  Decimal brute force on a tiny case.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from oracle import q40


@pytest.mark.parametrize("seed", range(6))
def test_block_properties(seed):
    rng = np.random.default_rng(seed)
    for scale in (1.0, 1e-3, 37.0):
        x = (rng.standard_normal(32) * scale).astype(np.float32)
        codes, d16 = q40.quantize_block(x)
        assert codes.max() <= 15
        j = int(np.argmax(np.abs(x)))  # first occurrence of the largest magnitude
        assert codes[j] == 0
        d = np.float32(x[j] / np.float32(-8))
        assert d16 == np.float16(d)
        rec = (codes.astype(np.float64) - 8) * float(d)
        err = np.abs(rec - x)
        step = abs(float(d))
        sat = codes == 15
        assert np.all(err[~sat] <= step / 2 * (1 + 1e-5))
        assert np.all(err[sat] <= step * (1 + 1e-5))
        # negating the block keeps the scale's magnitude
        c2, d2 = q40.quantize_block(-x)
        assert np.float16(-d2) == d16


def test_zero_block_and_exact_multiples():
    codes, d16 = q40.quantize_block(np.zeros(32, np.float32))
    assert np.all(codes == 8) and d16 == 0
    rng = np.random.default_rng(9)
    for d in (0.25, -0.125, 3.0, 1.0 / 1024):
        c = rng.integers(0, 16, 32)
        c[5] = 0                      # the block's largest magnitude: -8 d
        x = ((c - 8) * d).astype(np.float32)
        # another element of magnitude 8 |d| would come first only if it also had code 0
        got, d16 = q40.quantize_block(x)
        assert np.array_equal(got, c) and float(d16) == d


def test_ties_take_the_first_largest():
    x = np.zeros(32, np.float32)
    x[3], x[7] = -2.0, 2.0
    codes, d16 = q40.quantize_block(x)
    assert float(d16) == 0.25 and codes[3] == 0 and codes[7] == 15   # 2 / 0.25 + 8.5 = 16.5 -> 15
    x[3], x[7] = 2.0, -2.0
    codes, d16 = q40.quantize_block(x)
    assert float(d16) == -0.25 and codes[3] == 0


def test_quantize_rows_equals_block_by_block():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((30, 2, 128)) * np.exp2(rng.integers(-12, 12, size=(30, 2, 4))).repeat(32, -1)).astype(np.float32)
    x[2, 1, :32] = 0
    x[4, 0, 40] = -x[4, 0, 33:64].__abs__().max() * 2      # a negative maximum
    x[5, 0, 70], x[5, 0, 75] = 9.0, -9.0                   # a tie of magnitudes
    codes, d16 = q40.quantize_rows(x)
    for t in range(30):
        for h in range(2):
            c1, d1 = q40.quantize_row(x[t, h])
            assert np.array_equal(codes[t, h], c1) and np.array_equal(d16[t, h].view(np.uint16), d1.view(np.uint16))


def shared_scale_cache(rng, L, n_kv, hd, kv_bs=16):
    """A q4_0 cache whose rows use one fp16-exact scale for every block, and
    the int8 cache holding the same values as codes - 8 with that scale."""
    nblk = -(-L // kv_bs)
    table = np.arange(nblk, dtype=np.int32)[None, :]
    c4 = q40.Q40Cache(nblk, n_kv, kv_bs, hd)
    c8 = oracle.Cache(nblk, n_kv, kv_bs, hd)
    for t in range(L):
        blk, row = divmod(t, kv_bs)
        for kh in range(n_kv):
            for which in ("k", "v"):
                codes = rng.integers(0, 16, hd).astype(np.uint8)
                d = np.float16(2.0 ** rng.integers(-6, 3) * (1 + rng.integers(0, 8) / 8))
                getattr(c4, which + "_codes")[blk, kh, row] = codes
                getattr(c4, which + "_d")[blk, kh, row] = d
                getattr(c8, which + "_pages")[blk, kh, row] = codes.astype(np.int16) - 8
                getattr(c8, which + "_scale")[blk, kh, row] = np.float32(d)
    return c4, c8, table


@pytest.mark.parametrize("G,L", [(1, 1), (2, 37), (4, 70)])
def test_decode_equals_int8_three_pass_on_shared_scales(G, L):
    rng = np.random.default_rng(10 + G + L)
    c4, c8, table = shared_scale_cache(rng, L, 2, 128)
    q = rng.standard_normal((1, 2 * G, 128)).astype(np.float32)
    got = q40.decode(q, c4, table, [L], 0.088)
    want = oracle.three_pass_f64(q, c8, table, [L], 0.088)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_decode_one_token_and_zero_query():
    rng = np.random.default_rng(20)
    c4 = q40.Q40Cache(2, 1, 16, 64)
    k = rng.standard_normal((20, 1, 64)).astype(np.float32)
    v = rng.standard_normal((20, 1, 64)).astype(np.float32)
    c4.append(k, v, np.arange(20))
    table = np.array([[0, 1]], np.int32)
    q = rng.standard_normal((1, 2, 64)).astype(np.float32)
    q[0, 1] = 0
    out = q40.decode(q, c4, table, [1], 0.125)
    _, _, vd = c4.rows(table, 0, 0, 1)
    assert np.array_equal(out[0, 0], vd[0])
    out = q40.decode(q, c4, table, [20], 0.125)
    _, _, vd = c4.rows(table, 0, 0, 20)
    assert np.allclose(out[0, 1], vd.mean(0), rtol=0, atol=1e-15)


def test_decode_decimal_brute_force():
    rng = np.random.default_rng(21)
    c4 = q40.Q40Cache(1, 1, 16, 64)
    k = rng.standard_normal((6, 1, 64)).astype(np.float32)
    v = rng.standard_normal((6, 1, 64)).astype(np.float32)
    c4.append(k, v, np.arange(6))
    table = np.array([[0]], np.int32)
    q = rng.standard_normal((1, 1, 64)).astype(np.float32)
    out = q40.decode(q, c4, table, [6], 0.125)
    qi, qsc = oracle.quantize_q(q)
    getcontext().prec = 50
    s = []
    for t in range(6):
        tot = Decimal(0)
        for blk in range(2):
            dot = sum(int(qi[0, 0, 32 * blk + i]) * (int(c4.k_codes[0, 0, t, 32 * blk + i]) - 8) for i in range(32))
            tot += Decimal(dot) * Decimal(float(qsc[0, 0, blk])) * Decimal(float(c4.k_d[0, 0, t, blk]))
        s.append(tot * Decimal(float(np.float32(0.125))))
    m = max(s)
    w = [(x - m).exp() for x in s]
    W = sum(w)
    for i in range(64):
        vv = [(int(c4.v_codes[0, 0, t, i]) - 8) * Decimal(float(c4.v_d[0, 0, t, i // 32])) for t in range(6)]
        ref = sum(w[t] * vv[t] for t in range(6)) / W
        assert abs(float(ref) - out[0, 0, i]) < 1e-13
