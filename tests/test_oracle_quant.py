"""Pins for the oracle's quantiser, constants and append (CPU only).

What pins what, without another implementation of the method to compare to:

* the constants against the values the pages print (tests/golden), each
  rounded once to fp32 by an exact-rational rounding written here;
* the quantiser against exact rational arithmetic: every fp32 operation of
  the page's rule (page "Day 9-2: flash_attn_single_q_q8_neon", section 2,
  segment 1) is evaluated exactly and rounded to nearest-even fp32 by
  ``f32_round`` below, and the conversion to int8 truncates toward zero; a
  round-to-nearest conversion, a different guard, or scale = a/127 instead of
  a * fp32(1/127) each fail ``test_quantizer_exact_rational``;
* properties that hold for any correct quantiser of this form: range, sign
  symmetry, power-of-two scale invariance, the absmax element landing on
  +-126 or +-127, the dequantisation error bound, the all-zero and tiny rows;
* the paged append against its definition: the row lands at
  [block][kv head][row] of slot = block * kv_bs + row, negative slots are
  skipped, bf16 sources are widened exactly.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.txt")


def f32_round(x):
    """Round a rational to the nearest fp32 value (ties to even); returns a
    Fraction.  Covers normal and subnormal magnitudes (no overflow)."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    e = max(e, -126)
    quantum = Fraction(2) ** (e - 23)
    n = x / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def F(v):
    return Fraction(float(v))


def exact_quant(xs):
    """The quantiser rule evaluated in exact arithmetic with one fp32 rounding
    per operation; returns (list of ints, scale as Fraction)."""
    a = max(abs(F(x)) for x in xs)
    if a < f32_round(Fraction(1, 10 ** 6)):
        a = Fraction(1)
    inv127 = f32_round(Fraction(1, 127))
    scale = f32_round(a * inv127)
    inv = f32_round(Fraction(127) / a)
    out = []
    for x in xs:
        y = f32_round(F(x) * inv)
        y = min(max(y, Fraction(-128)), Fraction(127))
        out.append(int(y))  # int() of a Fraction truncates toward zero
    return out, scale


def read_golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        k, v = [s.strip() for s in line.split("=")]
        vals[k] = v
    return vals


def test_f32_round_matches_numpy_on_doubles():
    rng = np.random.default_rng(0)
    for v in np.concatenate([rng.standard_normal(300) * 10.0 ** rng.integers(-40, 30, 300),
                             [1e-45, 3e-39, 1.0 / 3.0]]):
        assert f32_round(Fraction(float(v))) == F(np.float32(v))


def test_constants_match_pages():
    g = read_golden()
    assert int(g["q_block"]) == 32
    assert F(oracle.inv127()) == f32_round(Fraction(1, 127))
    assert np.float32(oracle.inv127()).view(np.uint32) == 0x3C010204
    assert F(oracle.m_init()) == f32_round(Fraction(-10 ** 9))
    assert np.float32(oracle.m_init()).view(np.uint32) == 0xCE6E6B28
    assert int(g["two_pass_bytes"]) == int(g["two_pass_tokens"]) * 4
    assert g["inv127"] == "1/127" and g["m_init"] == "-1e9" and g["guard"] == "1e-6"


def test_quantizer_exact_rational():
    rng = np.random.default_rng(1)
    rows = [rng.standard_normal(32).astype(np.float32) for _ in range(60)]
    rows += [(rng.standard_normal(32) * 10.0 ** rng.integers(-5, 5)).astype(np.float32) for _ in range(40)]
    rows += [(rng.standard_normal(128) * 3).astype(np.float32) for _ in range(10)]
    # hand-picked edges: exact .5 products (a = 1 gives inv = 127 exactly),
    # the clamp edge, values at the guard, a lone nonzero element.
    rows.append(np.array([1.0, 0.5 / 127 * 127, 63.5 / 127, -63.5 / 127, -1.0, 0.0, 1e-7, -0.25] * 4, np.float32))
    rows.append(np.array([9.9e-7, -5e-7, 0.0, 1e-9] * 8, np.float32))
    rows.append(np.array([1e-6] + [5e-7] * 31, np.float32))
    rows.append(np.array([0.0] * 31 + [-3.0], np.float32))
    for x in rows:
        qv, sc = oracle.quantize(x)
        want_q, want_sc = exact_quant(x)
        assert list(qv.astype(int)) == want_q
        assert F(sc) == want_sc


def test_truncation_not_rounding():
    # a = 1 -> inv = 127 exactly; 0.5 -> 63.5 -> 63, -0.5 -> -63.5 -> -63.
    x = np.zeros(32, np.float32)
    x[0], x[1], x[2] = 1.0, 0.5, -0.5
    qv, sc = oracle.quantize(x)
    assert (qv[0], qv[1], qv[2]) == (127, 63, -63)
    assert F(sc) == f32_round(Fraction(1, 127))


def test_zero_and_tiny_rows():
    qv, sc = oracle.quantize(np.zeros(128, np.float32))
    assert not qv.any() and F(sc) == F(oracle.inv127())
    tiny = np.full(32, 9e-7, np.float32)
    qv, sc = oracle.quantize(tiny)
    assert not qv.any() and F(sc) == F(oracle.inv127())


def test_quantizer_properties():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4000, 32)).astype(np.float32)
    qv, sc = oracle.quantize(x)
    assert qv.min() >= -127 and qv.max() <= 127
    # sign symmetry
    qn, scn = oracle.quantize(-x)
    assert np.array_equal(qn, -qv) and np.array_equal(scn, sc)
    # power-of-two invariance: same ints, scale doubled exactly
    q2, sc2 = oracle.quantize(x * np.float32(2.0))
    assert np.array_equal(q2, qv) and np.array_equal(sc2, sc * np.float32(2.0))
    # the absmax element lands on +-126 or +-127 (126 when a*(127/a) < 127)
    idx = np.abs(x).argmax(axis=1)
    top = np.abs(qv[np.arange(len(x)), idx])
    assert set(np.unique(top)) <= {126, 127}
    frac126 = float(np.mean(top == 126))
    assert 0.05 < frac126 < 0.25, frac126
    # truncation: 0 <= |x|*inv - |q| < 1, so up to the few fp32 roundings in
    # inv and scale (a few ulps of |x|) the dequantised value never exceeds |x|
    # and is off by less than one step
    ax = np.abs(x.astype(np.float64))
    deq = qv.astype(np.float64) * sc.astype(np.float64)[:, None]
    step = sc.astype(np.float64)[:, None]
    err = ax - np.abs(deq)
    assert np.all(err > -4.0 * 2.0 ** -24 * ax) and np.all(err < step * (1 + 1e-5))


def test_quantize_q_is_per_32_block():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((3, 5, 128)).astype(np.float32)
    q[1, 2, 32:64] = 0.0
    qi, qsc = oracle.quantize_q(q)
    qb, sb = oracle.quantize(q.reshape(3, 5, 4, 32))
    assert np.array_equal(qi, qb.reshape(3, 5, 128)) and np.array_equal(qsc, sb)
    assert F(qsc[1, 2, 1]) == F(oracle.inv127()) and not qi[1, 2, 32:64].any()


@pytest.mark.parametrize("hd,kv_bs,n_kv", [(128, 16, 2), (64, 64, 3), (256, 32, 1), (96, 16, 2)])
def test_append_places_rows(hd, kv_bs, n_kv):
    rng = np.random.default_rng(4)
    nb, n = 7, 20
    k = rng.standard_normal((n, n_kv, hd)).astype(np.float32)
    v = rng.standard_normal((n, n_kv, hd)).astype(np.float32)
    slots = rng.choice(nb * kv_bs, size=n, replace=False).astype(np.int32)
    slots[3] = -1
    c = oracle.Cache(nb, n_kv, kv_bs, hd, fill_int8=99, fill_scale=np.nan)
    c.append(k, v, slots)
    kq, ks = oracle.quantize(k)
    vq, vs = oracle.quantize(v)
    written = np.zeros((nb, n_kv, kv_bs), bool)
    for t in range(n):
        if slots[t] < 0:
            continue
        blk, r = divmod(int(slots[t]), kv_bs)
        assert np.array_equal(c.k_pages[blk, :, r], kq[t]) and np.array_equal(c.v_pages[blk, :, r], vq[t])
        assert np.array_equal(c.k_scale[blk, :, r], ks[t]) and np.array_equal(c.v_scale[blk, :, r], vs[t])
        written[blk, :, r] = True
    assert np.all(c.k_pages[~written] == 99) and np.all(np.isnan(c.v_scale[~written]))


def test_append_bf16_widens_exactly():
    import torch
    rng = np.random.default_rng(5)
    n, n_kv, hd, kv_bs = 9, 2, 128, 16
    k = torch.from_numpy(rng.standard_normal((n, n_kv, hd)).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((n, n_kv, hd)).astype(np.float32)).to(torch.bfloat16)
    slots = np.arange(n, dtype=np.int32)
    a = oracle.Cache(1, n_kv, kv_bs, hd)
    a.append(k.view(torch.int16).numpy().view(np.uint16), v.view(torch.int16).numpy().view(np.uint16), slots)
    b = oracle.Cache(1, n_kv, kv_bs, hd)
    b.append(k.float().numpy(), v.float().numpy(), slots)
    for f in ("k_pages", "v_pages", "k_scale", "v_scale"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_score_variance_matches_page():
    # The generator's N(0,1) q and K give q.k/sqrt(128) of variance ~1 (page
    # on 1/sqrt(d_k): the dot of i.i.d. unit-variance vectors has variance d_k).
    import workloads
    w = workloads.WORKLOADS["mha7b"].scaled(seq_len=512)
    q = workloads.query(w)
    k, _ = workloads.kv_rows(w, 0, 512)
    s = np.einsum("hd,thd->th", q[0].astype(np.float64), k.astype(np.float64)) * workloads.softmax_scale(128)
    assert abs(s.var() - 1.0) < 0.05
    assert np.float32(workloads.softmax_scale(128)).view(np.uint32) == 0x3DB504F3
    assert F(workloads.softmax_scale(128)) == f32_round(Fraction(1) / Fraction(math.sqrt(128)))
