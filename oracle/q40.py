"""q4_0 KV codec -- TEST INFRASTRUCTURE ONLY.

Plain numpy definitions, used by tests, the smoke check and the benchmark's
CPU-baseline leg only; the product path never imports this module.

The pages name the codec only (page "FlashAttention" tag, baguaai.com, news
item on llama.cpp's SYCL decode path for q4_0 / q8_0 KV caches and its
--kv-cache-type q4_0 option); they give no format.  Reading: llama.cpp's
published q4_0 block format --
  * blocks of 32 consecutive elements of a row, one fp16 scale each;
  * m is the block element of largest magnitude (sign kept; the first one
    on ties), d = m / -8 in fp32, id = 1 / d (0 when d is 0);
  * code q = min(15, trunc(x * id + 8.5)) with x * id and + 8.5 two fp32
    roundings (no fused multiply-add), so q is in 0 .. 15;
  * the stored scale is d rounded to fp16 (to nearest even), and an element
    is (q - 8) * d16.
Decode over the codec follows the same method as the int8 cache (page
"Day 9-2: flash_attn_single_q_q8_neon", section 2): the query is quantised
per 32-element block to int8 (oracle.quantize_q), and since K's blocks are
the query's blocks, a token's score is
    scale * sum_b qsc[b] * d16_K[b] * sum_{i in b} qi[i] * (qk[i] - 8)
with exact integer block dots; the output is the softmax-weighted sum of the
dequantised V rows.  The oracle evaluates that definition in float64.
"""
import numpy as np

import oracle

QBLOCK = 32


def quantize_block(x):
    """One 32-element block (fp32) -> (codes uint8 [32], d16 as np.float16)."""
    x = np.asarray(x, np.float32)
    amax, m = np.float32(0), np.float32(0)
    for v in x:  # first element of largest magnitude, sign kept
        if abs(v) > amax:
            amax, m = np.float32(abs(v)), v
    d = np.float32(m / np.float32(-8.0))
    idv = np.float32(1.0) / d if d != 0 else np.float32(0.0)
    codes = np.empty(QBLOCK, np.uint8)
    for i, v in enumerate(x):
        y = np.float32(np.float32(v * idv) + np.float32(8.5))  # two roundings
        codes[i] = min(15, int(y))  # int() truncates toward zero; y >= 0.5 here
    return codes, np.float16(d)


def quantize_row(x):
    """A row whose length is a multiple of 32 -> (codes uint8 [n], d16 [n/32])."""
    x = np.asarray(x, np.float32)
    n = x.shape[-1]
    codes = np.empty(n, np.uint8)
    d16 = np.empty(n // QBLOCK, np.float16)
    for b in range(n // QBLOCK):
        codes[QBLOCK * b:QBLOCK * (b + 1)], d16[b] = quantize_block(x[QBLOCK * b:QBLOCK * (b + 1)])
    return codes, d16


def quantize_rows(x):
    """quantize_row over the last axis of x [..., n], vectorised with the same
    fp32 steps -> (codes uint8 [..., n], d16 float16 [..., n/32])."""
    x = np.asarray(x, np.float32)
    n = x.shape[-1]
    blocks = x.reshape(-1, n // QBLOCK, QBLOCK)
    j = np.argmax(np.abs(blocks), axis=-1)  # first occurrence of the largest magnitude
    m = np.take_along_axis(blocks, j[..., None], axis=-1)[..., 0]
    d = (m / np.float32(-8.0)).astype(np.float32)
    safe = np.where(d != 0, d, np.float32(1.0))
    idv = np.where(d != 0, np.float32(1.0) / safe, np.float32(0.0)).astype(np.float32)
    y = (blocks * idv[..., None]).astype(np.float32) + np.float32(8.5)
    codes = np.minimum(15, np.trunc(y)).astype(np.uint8)
    return codes.reshape(x.shape), d.astype(np.float16).reshape(x.shape[:-1] + (n // QBLOCK,))


def dequantize_row(codes, d16):
    return (np.asarray(codes, np.float64) - 8.0) * np.repeat(np.asarray(d16, np.float64), QBLOCK)


class Q40Cache:
    """Host copy of a paged q4_0 KV cache, codes unpacked and in row order:
    k_codes, v_codes uint8 [num_blocks][n_kv][kv_bs][hd] (0..15);
    k_d, v_d float16 [num_blocks][n_kv][kv_bs][hd/32]."""

    def __init__(self, num_blocks, n_kv, kv_bs, hd, fill_code=0xFF, fill_d=np.nan):
        self.num_blocks, self.n_kv, self.kv_bs, self.hd = num_blocks, n_kv, kv_bs, hd
        self.k_codes = np.full((num_blocks, n_kv, kv_bs, hd), fill_code, np.uint8)
        self.v_codes = np.full_like(self.k_codes, fill_code)
        self.k_d = np.full((num_blocks, n_kv, kv_bs, hd // QBLOCK), fill_d, np.float16)
        self.v_d = np.full_like(self.k_d, fill_d)

    def append(self, k_src, v_src, slot_mapping):
        """Quantise [n_tokens][n_kv][hd] fp32 rows into their slots; negative
        slots are skipped."""
        k_src = np.asarray(k_src, np.float32)
        v_src = np.asarray(v_src, np.float32)
        slots = np.asarray(slot_mapping, np.int64)
        keep = slots >= 0
        blk, row = slots[keep] // self.kv_bs, slots[keep] % self.kv_bs
        kc, kd = quantize_rows(k_src[keep])
        vc, vd = quantize_rows(v_src[keep])
        self.k_codes[blk, :, row], self.k_d[blk, :, row] = kc, kd
        self.v_codes[blk, :, row], self.v_d[blk, :, row] = vc, vd

    def rows(self, block_table, b, kh, L):
        """(K codes [L][hd], K d16 [L][hd/32], dequantised V [L][hd] float64)."""
        t = np.arange(L)
        blk = np.asarray(block_table)[b, t // self.kv_bs]
        r = t % self.kv_bs
        v = (self.v_codes[blk, kh, r].astype(np.float64) - 8.0) * np.repeat(
            self.v_d[blk, kh, r].astype(np.float64), QBLOCK, axis=-1)
        return self.k_codes[blk, kh, r], self.k_d[blk, kh, r], v


def decode(q, cache, block_table, seq_lens, scale):
    """out [batch][n_q][hd] float64 by the definition in the module header."""
    q = np.asarray(q, np.float32)
    batch, n_q, hd = q.shape
    G = n_q // cache.n_kv
    nb = hd // QBLOCK
    qi, qsc = oracle.quantize_q(q)
    out = np.zeros((batch, n_q, hd), np.float64)
    sc = float(np.float32(scale))
    for b in range(batch):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        for kh in range(cache.n_kv):
            kc, kd, v = cache.rows(block_table, b, kh, L)
            kb = kc.astype(np.int64).reshape(L, nb, QBLOCK) - 8
            for h in range(kh * G, (kh + 1) * G):
                dots = (kb * qi[b, h].astype(np.int64).reshape(nb, QBLOCK)).sum(-1)  # exact
                s = (dots.astype(np.float64) * qsc[b, h].astype(np.float64) * kd.astype(np.float64)).sum(-1) * sc
                p = np.exp(s - s.max())
                out[b, h] = (p / p.sum()) @ v
    return out
