"""Pins of the q4_0 codec oracle (oracle/q40.py).

* Quantiser properties that follow from the block format rather than from
  its formula: codes stay in 0..15; the block's first element of largest
  magnitude gets code 0 and comes back exactly up to the fp16 rounding of d;
  every other element comes back within half a step |d| / 2 (a full step
  where the top code saturates at 15); an all-zero block is code 8 with
  d = 0; a block made of exact multiples (c - 8) * d of an fp16-exact d
  returns its codes; negating a block keeps d's magnitude.
* The rounding of the code (reading of llama.cpp's q4_0 rule): x * id and
  + 8.5 are two fp32 roundings and the sum is truncated.  Elements whose
  x * id is exactly a half step (k + 1/2, with d a power of two) take the
  codes written out by hand below (trunc(k + 9) = k + 9; rounding x * id to
  nearest even, then adding 8, gives k + 8 for even k); elements whose
  exact x * id + 8.5 lies within half an ulp of an integer (found by an
  exact-rational search) take the code of the two roundings, which differs
  there from a single fused rounding.  Both are checked against the rule
  evaluated in exact rational arithmetic, and a battery of planted mistakes
  (round-half-even, a fused multiply-add, no clamp at 15, the scale's sign,
  ties to the last element) must each fail one of these pins.
* Decode: a cache whose rows use one fp16-exact scale for all their blocks is
  the same attention as an int8 cache with codes c - 8 and that scale, so
  the q4_0 decode must equal the independent three-pass fp64 reference of
  the int8 oracle (oracle.three_pass_f64) on it; one token returns its
  dequantised V row; a zero query gives the mean of the dequantised rows;
  Decimal brute force on a tiny case.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import q40
from test_oracle_quant import F, f32_round


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


# ---------------------------------------------------------------------------
# the code's rounding

def exact_q40_block(xs, fused=False):
    """The q4_0 rule in exact rational arithmetic, one fp32 rounding per
    operation: m = the first element of largest magnitude, d = rn(m / -8),
    id = rn(1 / d) (0 for d = 0), code = min(15, trunc(rn(rn(x id) + 17/2)))
    -- or, with fused, a single rounding of x id + 17/2.  The sum is at
    least 1/2, so truncation is the floor."""
    a, m = Fraction(0), Fraction(0)
    for x in xs:
        if abs(F(x)) > a:
            a, m = abs(F(x)), F(x)
    d = f32_round(m / -8)
    idv = f32_round(1 / d) if d != 0 else Fraction(0)
    codes = []
    for x in xs:
        y = F(x) * idv
        y = f32_round(y + Fraction(17, 2)) if fused else f32_round(f32_round(y) + Fraction(17, 2))
        codes.append(min(15, math.floor(y)))
    return codes, d


# (x, code) with d = 1: x * id = x exactly; code = trunc(x + 8.5), written out
HALF_STEPS = [(-8.0, 0), (0.5, 9), (2.5, 11), (4.5, 13), (6.5, 15), (-1.5, 7), (-3.5, 5), (-5.5, 3),
              (-7.5, 1), (1.5, 10), (3.5, 12), (-0.5, 8), (-2.5, 6), (0.0, 8), (7.5, 15), (-6.5, 2)]


def half_step_blocks():
    xs = np.zeros(32, np.float32)
    want = np.full(32, 8, np.uint8)
    for i, (x, c) in enumerate(HALF_STEPS):
        xs[i], want[i] = x, c
    for k in (0, -20, -3, 5, 20):   # d = 2^k: the same codes
        yield (xs * np.float32(2.0 ** k)).astype(np.float32), want


def test_half_steps_truncate():
    for xs, want in half_step_blocks():
        codes, d16 = q40.quantize_block(xs)
        assert np.array_equal(codes, want), (xs[:4], codes[:16], want[:16])
        assert list(want) == exact_q40_block(xs)[0]


def two_rounding_blocks(n=4):
    """Blocks in which x * id + 8.5 falls where the two fp32 roundings and
    a fused one disagree: x * id just past -1/2 - 2^-22 (so x * id rounds to
    exactly -1/2 - 2^-22 and the sum to the tie 8 - 2^-22, which goes to the
    even 8, while the exact sum rounds down to 8 - 2^-21).  Found by an
    exact-rational search over seeded block maxima."""
    rng = np.random.default_rng(2024)
    target = -Fraction(1, 2) - Fraction(17, 4) * Fraction(1, 2 ** 24)
    found = []
    while len(found) < n:
        m = np.float32(-rng.uniform(1.0, 8.0) * 2.0 ** int(rng.integers(-6, 7)))
        d = f32_round(F(m) / -8)
        idv = f32_round(1 / d)
        x0 = np.float32(float(target / idv))
        for cand in (x0, np.nextafter(x0, np.float32(-np.inf)), np.nextafter(x0, np.float32(np.inf))):
            xs = np.zeros(32, np.float32)
            xs[0], xs[1 + len(found) % 31] = m, cand
            two, _ = exact_q40_block(xs)
            fused, _ = exact_q40_block(xs, fused=True)
            if two != fused:
                found.append((xs, two))
                break
    return found


def test_two_roundings_not_fused():
    blocks = two_rounding_blocks()
    assert len(blocks) == 4
    for xs, want in blocks:
        codes, _ = q40.quantize_block(xs)
        assert list(codes) == want
        rows, _ = q40.quantize_rows(xs[None])
        assert list(rows[0]) == want


def test_rule_exact_on_random_blocks():
    """The oracle's codes and scales equal the rule evaluated exactly, on
    random blocks of several magnitudes (scale: fp16 of the exact d)."""
    rng = np.random.default_rng(77)
    for scale in (1.0, 3e-4, 250.0):
        for _ in range(20):
            xs = (rng.standard_normal(32) * scale).astype(np.float32)
            codes, d16 = q40.quantize_block(xs)
            want, d = exact_q40_block(xs)
            assert list(codes) == want and d16 == np.float16(float(d))


# planted mistakes in the quantiser; each must fail one of the pins above

def _mutant(kind):
    def block(x):
        x = np.asarray(x, np.float32)
        amax, m = np.float32(0), np.float32(0)
        for v in x:
            if abs(v) > amax or (kind == "ties_last" and abs(v) == amax and amax > 0):
                amax, m = np.float32(abs(v)), v
        d = np.float32(m / np.float32(8.0 if kind == "d_sign" else -8.0))
        idv = np.float32(1.0) / d if d != 0 else np.float32(0.0)
        codes = np.empty(32, np.uint8)
        for i, v in enumerate(x):
            if kind == "round_half_even":
                c = int(np.rint(np.float32(v * idv))) + 8
            elif kind == "fused":
                c = math.floor(f32_round(F(v) * F(idv) + Fraction(17, 2)))
            else:
                c = int(np.float32(np.float32(v * idv) + np.float32(8.5)))
            codes[i] = c if kind == "no_clamp" else min(15, c)
        return codes, np.float16(d)

    def rows(x):
        x = np.asarray(x, np.float32)
        n = x.shape[-1]
        flat = x.reshape(-1, n)
        codes = np.empty(flat.shape, np.uint8)
        d16 = np.empty((flat.shape[0], n // 32), np.float16)
        for r in range(flat.shape[0]):
            for b in range(n // 32):
                codes[r, 32 * b:32 * b + 32], d16[r, b] = block(flat[r, 32 * b:32 * b + 32])
        return codes.reshape(x.shape), d16.reshape(x.shape[:-1] + (n // 32,))
    return block, rows


PINS = [lambda: test_block_properties(0), test_zero_block_and_exact_multiples, test_ties_take_the_first_largest,
        test_half_steps_truncate, test_two_roundings_not_fused, test_rule_exact_on_random_blocks]


@pytest.mark.parametrize("kind", ["round_half_even", "fused", "no_clamp", "d_sign", "ties_last"])
def test_mutants_fail_a_pin(kind, monkeypatch):
    block, rows = _mutant(kind)
    monkeypatch.setattr(q40, "quantize_block", block)
    monkeypatch.setattr(q40, "quantize_rows", rows)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, OverflowError, ValueError):
            failed.append(pin)
    assert failed, f"mutant {kind} passes every pin"


def test_unmutated_blockwise_passes_every_pin(monkeypatch):
    """The battery's own control: the rule written the same way as the
    mutants, unchanged, passes every pin."""
    block, rows = _mutant("none")
    monkeypatch.setattr(q40, "quantize_block", block)
    monkeypatch.setattr(q40, "quantize_rows", rows)
    for pin in PINS:
        pin()
