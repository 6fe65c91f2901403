"""FP8 (E4M3) KV codec with UE8M0 per-64-element scales -- TEST INFRASTRUCTURE ONLY.

Plain numpy definitions of the second KV codec the pages describe (page
"deepseek-attention-div64", beaiera.top, section on the FP8 quantisation
scaling): every 64 consecutive elements of a K or V row share one scale
byte; the block's absolute maximum fixes the exponent
e = ceil(log2(absmax / 448)), the elements are multiplied by 2^-e, clamped
to [-448, 448] and rounded to FP8 E4M3; the scale is stored as the unsigned
8-bit exponent UE8M0 (e + 127), one byte per block.

Used by tests, the smoke check and the benchmark's CPU-baseline leg only;
the product path never imports it, and it imports nothing of the product.

Readings where the page is silent (each one is a pin in
tests/test_oracle_fp8.py):

* E4M3 is the 4-exponent-bit, bias-7, 3-mantissa-bit format whose largest
  finite value is the page's 448 (so codes 0x7f / 0xff are NaN and there is
  no infinity); conversion rounds to nearest, ties to the even code.
* absmax / 448 is one fp32 division; e is the exact ceiling of the base-2
  logarithm of that fp32 quotient (an integer computed from its bits, not a
  rounded log2), clamped to [-126, 127] so that the scale 2^e is a normal
  fp32 number (2^-e stays exact).  An all-zero block takes e = 0.
* x * 2^-e is one fp32 multiplication (exact unless it underflows).

Attention over the codec is the plain definition, in fp64: softmax of the
scaled dot products of the fp32 query with the dequantised K rows
(code value * 2^e), weights applied to the dequantised V rows.
"""
import numpy as np

QBLOCK = 64          # elements per scale
FP8_MAX = 448.0      # largest finite E4M3 value
E_MIN, E_MAX = -126, 127


def e4m3_value(code):
    """Value of an E4M3 code (0..255) from the format definition; NaN for
    0x7f / 0xff."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def _positive_table():
    """The 127 finite non-negative codes 0x00..0x7e and their values,
    ascending (the format is monotonic in its code for non-negative values)."""
    codes = np.arange(0x7F, dtype=np.int64)
    vals = np.array([e4m3_value(c) for c in codes], np.float64)
    assert np.all(np.diff(vals) > 0)
    return codes, vals


_CODES, _VALS = _positive_table()


def e4m3_encode_one(x):
    """Nearest E4M3 code to a finite |x| <= 448 (ties to the even code),
    by exhaustive search over the finite non-negative codes; the sign bit
    carries the sign of x (so -0.0 and negative values that round to zero
    give 0x80)."""
    x = float(x)
    ax = abs(x)
    best = None
    for c, v in zip(_CODES, _VALS):
        d = abs(ax - v)
        if best is None or d < best[1] or (d == best[1] and (c & 1) == 0 and (best[0] & 1) == 1):
            best = (int(c), d)
    code = best[0]
    if np.signbit(x):
        code |= 0x80
    return code


def e4m3_encode(x):
    """Vectorised e4m3_encode_one for arrays of finite values in [-448, 448]."""
    x = np.asarray(x, np.float64)
    ax = np.abs(x)
    hi = np.clip(np.searchsorted(_VALS, ax, side="left"), 0, len(_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_VALS) - 1)
    dlo = ax - _VALS[lo]
    dhi = _VALS[hi] - ax
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_CODES[hi] % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, _CODES[hi], _CODES[lo]).astype(np.int64)
    code = np.where(ax == _VALS[hi], _CODES[hi], code)
    code |= np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def e4m3_decode(codes):
    """Values of an array of codes (float64)."""
    table = np.array([e4m3_value(c) for c in range(256)], np.float64)
    return table[np.asarray(codes, np.uint8)]


def block_exponent(absmax):
    """e = ceil(log2(fp32(absmax / 448))) from the bits of the fp32 quotient,
    clamped to [-126, 127]; 0 for an all-zero block."""
    a = np.float32(absmax)
    if a == 0:
        return 0
    r = np.float32(a / np.float32(FP8_MAX))
    m, k = np.frexp(np.float64(r))   # r = m * 2^k exactly, m in [0.5, 1)
    e = int(k) - 1 if m == 0.5 else int(k)
    return max(E_MIN, min(E_MAX, e))


def quantize_row(x):
    """One K or V row (fp32, length a multiple of 64) -> (uint8 codes, uint8
    UE8M0 scale bytes, one per 64 elements)."""
    x = np.asarray(x, np.float32)
    n = x.shape[-1]
    assert n % QBLOCK == 0
    codes = np.empty(n, np.uint8)
    sc = np.empty(n // QBLOCK, np.uint8)
    for blk in range(n // QBLOCK):
        seg = x[QBLOCK * blk:QBLOCK * (blk + 1)]
        e = block_exponent(np.max(np.abs(seg)))
        inv = np.float32(2.0 ** -e)
        y = np.clip(seg * inv, np.float32(-FP8_MAX), np.float32(FP8_MAX))  # one fp32 multiply each
        codes[QBLOCK * blk:QBLOCK * (blk + 1)] = e4m3_encode(y)
        sc[blk] = e + 127
    return codes, sc


def quantize_rows(x):
    """quantize_row over the last axis of x [..., n], all rows at once (the
    same fp32 steps, vectorised) -> (codes [..., n], scale bytes [..., n/64])."""
    x = np.asarray(x, np.float32)
    n = x.shape[-1]
    blocks = x.reshape(-1, n // QBLOCK, QBLOCK)
    am = np.max(np.abs(blocks), axis=-1)
    r = (am / np.float32(FP8_MAX)).astype(np.float32)
    m, k = np.frexp(r.astype(np.float64))
    e = np.where(m == 0.5, k - 1, k)
    e = np.clip(e, E_MIN, E_MAX)
    e = np.where(am == 0, 0, e).astype(np.int64)
    inv = np.exp2(-e.astype(np.float64)).astype(np.float32)[..., None]
    y = np.clip(blocks * inv, np.float32(-FP8_MAX), np.float32(FP8_MAX))
    codes = e4m3_encode(y).reshape(x.shape)
    return codes, (e + 127).astype(np.uint8).reshape(x.shape[:-1] + (n // QBLOCK,))


def dequantize_row(codes, sc):
    """codes [n] uint8, sc [n/64] uint8 -> float64 values code * 2^(sc - 127)."""
    v = e4m3_decode(codes)
    e = np.repeat(np.asarray(sc, np.int64) - 127, QBLOCK)
    return v * np.exp2(e.astype(np.float64))


class Fp8Cache:
    """Host copy of a paged FP8 KV cache, pages in row order:
    k_pages, v_pages uint8 [num_blocks][n_kv][kv_bs][hd] (E4M3 codes);
    k_scale, v_scale uint8 [num_blocks][n_kv][kv_bs][hd/64] (UE8M0)."""

    def __init__(self, num_blocks, n_kv, kv_bs, hd, fill_code=0x7F, fill_scale=0xFF):
        self.num_blocks, self.n_kv, self.kv_bs, self.hd = num_blocks, n_kv, kv_bs, hd
        self.k_pages = np.full((num_blocks, n_kv, kv_bs, hd), fill_code, np.uint8)
        self.v_pages = np.full_like(self.k_pages, fill_code)
        self.k_scale = np.full((num_blocks, n_kv, kv_bs, hd // QBLOCK), fill_scale, np.uint8)
        self.v_scale = np.full_like(self.k_scale, fill_scale)

    def append(self, k_src, v_src, slot_mapping):
        """Quantise [n_tokens][n_kv][hd] fp32 rows into their slots
        (block * kv_bs + row); negative slots are skipped."""
        k_src = np.asarray(k_src, np.float32)
        v_src = np.asarray(v_src, np.float32)
        slots = np.asarray(slot_mapping, np.int64)
        keep = slots >= 0
        blk, row = slots[keep] // self.kv_bs, slots[keep] % self.kv_bs
        kc, ks = quantize_rows(k_src[keep])
        vc, vs = quantize_rows(v_src[keep])
        self.k_pages[blk, :, row], self.k_scale[blk, :, row] = kc, ks
        self.v_pages[blk, :, row], self.v_scale[blk, :, row] = vc, vs

    def rows(self, block_table, b, kh, L):
        """Dequantised K and V rows [L][hd] (float64) of tokens 0..L-1."""
        t = np.arange(L)
        blk = np.asarray(block_table)[b, t // self.kv_bs]
        r = t % self.kv_bs
        kc, ks = self.k_pages[blk, kh, r], self.k_scale[blk, kh, r]
        vc, vs = self.v_pages[blk, kh, r], self.v_scale[blk, kh, r]
        k = e4m3_decode(kc) * np.exp2(np.repeat(ks.astype(np.int64) - 127, QBLOCK, axis=-1).astype(np.float64))
        v = e4m3_decode(vc) * np.exp2(np.repeat(vs.astype(np.int64) - 127, QBLOCK, axis=-1).astype(np.float64))
        return k, v


def decode(q, cache, block_table, seq_lens, scale):
    """out[b][h] = softmax(scale * q[b][h] . K_b) V_b over tokens 0..L-1 of
    sequence b, K and V dequantised, fp64 throughout (q taken as given, fp32).
    Query head h reads kv head h / (n_q / n_kv).  Rows with L <= 0 are zero."""
    q = np.asarray(q, np.float32)
    batch, n_q, hd = q.shape
    G = n_q // cache.n_kv
    out = np.zeros((batch, n_q, hd), np.float64)
    sc = float(np.float32(scale))
    for b in range(batch):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        for kh in range(cache.n_kv):
            k, v = cache.rows(block_table, b, kh, L)
            for h in range(kh * G, (kh + 1) * G):
                s = (k @ q[b, h].astype(np.float64)) * sc
                p = np.exp(s - s.max())
                out[b, h] = (p / p.sum()) @ v
    return out
