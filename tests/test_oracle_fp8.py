"""Pins of the FP8 (E4M3 + UE8M0 per 64 elements) KV codec oracle.

The page (deepseek-attention-div64, beaiera.top, section on the FP8
quantisation scaling) fixes: 64-element blocks, one 1-byte scale per block,
exponent = ceil(log2(absmax / 448)), inverse scale 2^-exponent, clamp to
[-448, 448], conversion to E4M3.  These tests pin the oracle against that
and against the E4M3 format itself, not against the oracle's own formulas:

* the code table against the format's closed form at the values the page
  and the format fix (tests/golden/fp8_e4m3.txt);
* the encoder against brute force (exhaustive nearest search on many
  inputs), exact round trips of every finite code, midpoints tying to the
  even code, monotonicity and the half-spacing error bound;
* the exponent against exact rational arithmetic (Fraction) on the fp32
  quotient, including quotients exactly at and one ulp above powers of two;
* the block quantiser: every block's absmax lands in (224, 448] after the
  scaling (so no block wastes its top binade), the dequantisation error
  bound of E4M3, block independence;
* attention over the codec: one token returns its dequantised V row, a zero
  query gives the plain mean, and the fp64 softmax agrees with Decimal
  brute force on a tiny case.
"""
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from oracle import fp8kv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_e4m3.txt")


def read_golden():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            code, value = line.split()
            rows.append((int(code, 16), value))
    return rows


def test_code_table_golden():
    rows = read_golden()
    assert len(rows) >= 10
    for code, value in rows:
        got = fp8kv.e4m3_value(code)
        if value == "nan":
            assert np.isnan(got), hex(code)
        else:
            want = float(Fraction(value))
            assert got == want and np.signbit(got) == value.startswith("-"), (hex(code), got, value)


def test_code_table_closed_form():
    """Every code against sign * 2^(E-7) * (1 + m/8), subnormals m/8 * 2^-6,
    evaluated with exact fractions."""
    for code in range(256):
        s, E, m = code >> 7, (code >> 3) & 15, code & 7
        got = fp8kv.e4m3_value(code)
        if E == 15 and m == 7:
            assert np.isnan(got)
            continue
        mag = Fraction(m, 8) * Fraction(1, 64) if E == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (E - 7)
        assert Fraction(abs(got)) == mag
        assert np.signbit(got) == bool(s)
    assert max(fp8kv.e4m3_value(c) for c in range(0x7F)) == 448.0


def test_encode_round_trips_every_finite_code():
    for code in list(range(0x7F)) + list(range(0x80, 0xFF)):
        v = fp8kv.e4m3_value(code)
        assert fp8kv.e4m3_encode_one(v) == code, hex(code)
        assert int(fp8kv.e4m3_encode(np.array([v]))[0]) == code, hex(code)


def test_encode_matches_brute_force():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-448, 448, 400), rng.standard_normal(400) * 0.05,
                        rng.standard_normal(200) * 2.0 ** -8, [0.0, -0.0, 448.0, -448.0]])
    got = fp8kv.e4m3_encode(x)
    for xi, gi in zip(x, got):
        assert int(gi) == fp8kv.e4m3_encode_one(xi), xi


def test_midpoints_tie_to_even_and_error_bound():
    vals = [fp8kv.e4m3_value(c) for c in range(0x7F)]
    for c in range(0x7E):
        lo, hi = vals[c], vals[c + 1]
        mid = (lo + hi) / 2            # exact in float64
        want = c if c % 2 == 0 else c + 1
        assert fp8kv.e4m3_encode_one(mid) == want
        assert int(fp8kv.e4m3_encode(np.array([mid]))[0]) == want
        # just off the midpoint goes to the nearer code
        assert fp8kv.e4m3_encode_one(np.nextafter(mid, -np.inf)) == c
        assert fp8kv.e4m3_encode_one(np.nextafter(mid, np.inf)) == c + 1
    x = np.linspace(0, 448, 20001)
    dec = fp8kv.e4m3_decode(fp8kv.e4m3_encode(x))
    assert np.all(np.diff(dec) >= 0)
    # half the spacing of the binade: 2^(floor(log2 x) - 3) / 2, subnormal spacing 2^-9
    spacing = np.where(x < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(x, 2.0 ** -6))) - 3))
    assert np.all(np.abs(dec - x) <= spacing / 2 + 1e-300)


def exact_exponent(absmax):
    """ceil(log2 r) for the fp32 quotient r, by exact rational search."""
    r = Fraction(float(np.float32(np.float32(absmax) / np.float32(448.0))))
    e = 0
    while Fraction(2) ** e < r:
        e += 1
    while Fraction(2) ** (e - 1) >= r:
        e -= 1
    return max(-126, min(127, e))


def test_block_exponent_exact():
    cases = [448.0, 224.0, 1.0, 3.5, 1e-3, 5.0e-38, 3e38, 448.0 * 2 ** -20]
    for k in range(-30, 30):
        p = np.float32(448.0 * 2.0 ** k)
        cases += [p, np.nextafter(p, np.float32(np.inf)), np.nextafter(p, np.float32(0))]
    rng = np.random.default_rng(4)
    cases += list(np.abs(rng.standard_normal(300)).astype(np.float32))
    for a in cases:
        assert fp8kv.block_exponent(a) == exact_exponent(a), a
    assert fp8kv.block_exponent(0.0) == 0
    # the page's example range: absmax exactly 448 * 2^k gives k
    assert fp8kv.block_exponent(448.0 * 8) == 3


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_quantize_row_properties(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(256) * np.exp(rng.standard_normal(4)).repeat(64)).astype(np.float32)
    x[70] = 0.0
    x[128:192] = 0.0                      # an all-zero block
    codes, sc = fp8kv.quantize_row(x)
    assert codes.dtype == np.uint8 and sc.shape == (4,)
    assert sc[2] == 127 and np.all(codes[128:192] == 0)
    deq = fp8kv.dequantize_row(codes, sc)
    for blk in (0, 1, 3):
        seg = x[64 * blk:64 * (blk + 1)].astype(np.float64)
        e = int(sc[blk]) - 127
        top = np.abs(seg).max() * 2.0 ** -e
        assert 224.0 < top <= 448.0 or np.isclose(top, 448.0)
        # E4M3 keeps 3 mantissa bits: relative error <= 2^-4 for normals,
        # absolute error <= 2^-10 * 2^e in the subnormal range
        err = np.abs(deq[64 * blk:64 * (blk + 1)] - seg)
        bound = np.maximum(np.abs(seg) * 2.0 ** -4, 2.0 ** (e - 10))
        assert np.all(err <= bound)
    # blocks are independent: changing block 3 leaves blocks 0-2 alone
    y = x.copy()
    y[200] *= 1000
    c2, s2 = fp8kv.quantize_row(y)
    assert np.array_equal(c2[:192], codes[:192]) and np.array_equal(s2[:3], sc[:3])
    assert s2[3] > sc[3]


def test_quantize_rows_equals_row_by_row():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((40, 3, 128)) * np.exp2(rng.integers(-20, 20, size=(40, 3, 2))).repeat(64, -1)).astype(np.float32)
    x[3, 1, :64] = 0
    x[5, 0, 64] = 448.0 * 2 ** 7
    codes, sc = fp8kv.quantize_rows(x)
    for t in range(40):
        for h in range(3):
            c1, s1 = fp8kv.quantize_row(x[t, h])
            assert np.array_equal(codes[t, h], c1) and np.array_equal(sc[t, h], s1)


def tiny_cache(L, hd=128, seed=5):
    rng = np.random.default_rng(seed)
    c = fp8kv.Fp8Cache(num_blocks=4, n_kv=1, kv_bs=16, hd=hd)
    k = rng.standard_normal((L, 1, hd)).astype(np.float32)
    v = rng.standard_normal((L, 1, hd)).astype(np.float32)
    table = np.array([[2, 0, 3, 1]], np.int32)
    slots = np.array([table[0, t // 16] * 16 + t % 16 for t in range(L)])
    c.append(k, v, slots)
    return c, table, k, v


def test_decode_one_token_and_zero_query():
    c, table, k, v = tiny_cache(20)
    q = np.random.default_rng(6).standard_normal((1, 2, 128)).astype(np.float32)
    q[0, 1] = 0
    out = fp8kv.decode(q, c, table, [1], 0.088)
    _, vd = c.rows(table, 0, 0, 1)
    assert np.array_equal(out[0, 0], vd[0])
    out = fp8kv.decode(q, c, table, [20], 0.088)
    _, vd = c.rows(table, 0, 0, 20)
    assert np.allclose(out[0, 1], vd.mean(0), rtol=0, atol=1e-15)


def test_decode_decimal_brute_force():
    c, table, k, v = tiny_cache(5, hd=64, seed=7)
    q = np.random.default_rng(8).standard_normal((1, 1, 64)).astype(np.float32)
    out = fp8kv.decode(q, c, table, [5], 0.125)
    kd, vd = c.rows(table, 0, 0, 5)
    getcontext().prec = 50
    qs = [Decimal(float(x)) for x in q[0, 0]]
    s = [sum(Decimal(float(kd[t, i])) * qs[i] for i in range(64)) * Decimal(float(np.float32(0.125))) for t in range(5)]
    m = max(s)
    w = [(x - m).exp() for x in s]
    tot = sum(w)
    for i in range(64):
        ref = sum(w[t] * Decimal(float(vd[t, i])) for t in range(5)) / tot
        assert abs(float(ref) - out[0, 0, i]) < 1e-13
