"""Seeded synthetic inputs for q8-KV decode attention (shared by the tests,
the benchmark and the smoke check).

This module only draws inputs -- fp32 query and K/V source rows, sequence
lengths, block tables, slot mappings and the softmax scale argument.  It holds
none of the method's arithmetic: quantisation happens in the library
(``q8kv_append``) on the GPU and in the oracle on the CPU, from these same
fp32 rows.

Every stream is derived from base seed 42 with ``SeedSequence`` spawn keys
(workload key, stream id, sequence index), so any single sequence can be
regenerated alone -- the large workloads never need their whole fp32 source in
host memory at once.

The five named workloads follow the decode shapes the pages discuss: a tiny
single head, an MHA 7B-like step (32/32 heads, hd 128), a GQA batch (32/8), a
128K-token long context (32/4, kv_bs 64, rare 10x-amplitude K tokens) and a
ragged batch of 64 sequences (64/8, lengths U{1..32768}, per-channel
lognormal K scaling).
"""
from dataclasses import dataclass, replace

import numpy as np

BASE_SEED = 42

# stream ids
_S_Q, _S_K, _S_V, _S_TABLE, _S_LENS, _S_CHAN, _S_OUTLIER = range(7)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q: int
    n_kv: int
    hd: int
    kv_bs: int
    seq_len: int                  # every sequence's length, or the maximum when ragged
    ragged: bool = False          # lengths drawn uniformly from 1..seq_len
    table: str = "perm"           # "identity" | "perm" | "pool"
    k_outlier_p: float = 0.0      # per-token chance that a K row is amplified
    k_outlier_amp: float = 1.0    # amplification of such a token (all kv heads)
    k_channel_lognormal: bool = False  # K channel c of kv head kh scaled by exp(N(0,1))
    key: int = 0                  # seed key (distinct per workload)
    spare_blocks: int = 0         # extra physical blocks never referenced by the table

    @property
    def group(self):
        return self.n_q // self.n_kv

    @property
    def max_blocks(self):
        return -(-self.seq_len // self.kv_bs)

    def scaled(self, **kw):
        """A copy with some fields replaced (same generator recipe)."""
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 128, 16, 512, table="identity", key=1),
    "mha7b": Workload("mha7b", 1, 32, 32, 128, 16, 4096, key=2),
    "gqa_batch": Workload("gqa_batch", 16, 32, 8, 128, 16, 8192, key=3),
    "long_gqa": Workload("long_gqa", 1, 32, 4, 128, 64, 131072, k_outlier_p=0.02,
                         k_outlier_amp=10.0, key=4),
    "ragged": Workload("ragged", 64, 64, 8, 128, 64, 32768, ragged=True, table="pool",
                       k_channel_lognormal=True, key=5),
}
ORDER = ["tiny", "mha7b", "gqa_batch", "long_gqa", "ragged"]


def rng(w, *stream):
    return np.random.default_rng(np.random.SeedSequence(BASE_SEED, spawn_key=(w.key,) + stream))


def softmax_scale(hd):
    """The scale argument: 1/sqrt(hd) computed in double, rounded once to fp32."""
    return float(np.float32(1.0 / np.sqrt(float(hd))))


def seq_lens(w):
    if w.ragged:
        return rng(w, _S_LENS).integers(1, w.seq_len + 1, size=w.batch).astype(np.int32)
    return np.full(w.batch, w.seq_len, np.int32)


def block_table(w, lens=None):
    """(table int32 [batch][max_blocks], num_blocks).

    identity: sequence b's logical block j is physical block b*max_blocks + j.
    perm:     a random permutation of all batch*max_blocks physical blocks.
    pool:     a shared pool of exactly the blocks needed (sum of ceil(L/kv_bs)),
              permuted and handed out in sequence order; unused entries are -1.
    spare_blocks extra physical blocks are mixed into the pool and never used.
    """
    if lens is None:
        lens = seq_lens(w)
    need = [-(-int(L) // w.kv_bs) for L in lens]
    table = np.full((w.batch, w.max_blocks), -1, np.int32)
    if w.table in ("identity", "perm"):
        total = w.batch * w.max_blocks
    else:
        total = sum(need)
    num_blocks = total + w.spare_blocks
    if w.table == "identity":
        ids = np.arange(num_blocks, dtype=np.int64)
    else:
        ids = rng(w, _S_TABLE).permutation(num_blocks)
    pos = 0
    for b in range(w.batch):
        if w.table == "pool":
            table[b, :need[b]] = ids[pos:pos + need[b]]
            pos += need[b]
        else:
            table[b, :need[b]] = ids[b * w.max_blocks:b * w.max_blocks + need[b]]
    return table, num_blocks


def query(w):
    return rng(w, _S_Q).standard_normal((w.batch, w.n_q, w.hd), dtype=np.float32)


def channel_scale(w):
    """Per (kv head, channel) K multiplier exp(N(0,1)), drawn once per workload."""
    return np.exp(rng(w, _S_CHAN).standard_normal((w.n_kv, w.hd))).astype(np.float32)


def kv_rows(w, b, L):
    """fp32 K and V source rows [L][n_kv][hd] of sequence b, tokens 0..L-1."""
    k = rng(w, _S_K, b).standard_normal((L, w.n_kv, w.hd), dtype=np.float32)
    v = rng(w, _S_V, b).standard_normal((L, w.n_kv, w.hd), dtype=np.float32)
    if w.k_outlier_p > 0.0:
        hit = rng(w, _S_OUTLIER, b).random(L) < w.k_outlier_p
        k[hit] *= np.float32(w.k_outlier_amp)
    if w.k_channel_lognormal:
        k *= channel_scale(w)[None]
    return k, v


def slot_mapping(w, table, b, L):
    """Cache slot (physical block * kv_bs + row) of tokens 0..L-1 of sequence b."""
    t = np.arange(L, dtype=np.int64)
    return (table[b, t // w.kv_bs].astype(np.int64) * w.kv_bs + t % w.kv_bs).astype(np.int32)


def kv_bytes(w, lens):
    """Algorithmic KV bytes of one decode step: per (token, kv head) one int8
    K row, one int8 V row and two fp32 scales."""
    return int(np.sum(lens, dtype=np.int64)) * w.n_kv * (2 * w.hd + 8)


def fp8_kv_bytes(w, lens):
    """Algorithmic KV bytes of one decode step over the FP8 codec: per (token,
    kv head) one E4M3 K row, one E4M3 V row and one scale byte per 64
    elements of each."""
    return int(np.sum(lens, dtype=np.int64)) * w.n_kv * (2 * w.hd + 2 * (w.hd // 64))


def q40_kv_bytes(w, lens):
    """Algorithmic KV bytes of one decode step over the q4_0 codec: per
    (token, kv head) hd / 2 bytes of 4-bit K codes, as many of V codes, and
    one fp16 scale per 32 elements of each."""
    return int(np.sum(lens, dtype=np.int64)) * w.n_kv * (w.hd + 4 * (w.hd // 32))


def step_bytes(w, lens, codec="q8"):
    """All algorithmic bytes of one step: KV + scales, q and out (fp32), the
    used block-table entries and the seq_lens array."""
    used_blocks = sum(-(-int(L) // w.kv_bs) for L in lens)
    kv = {"q8": kv_bytes, "fp8": fp8_kv_bytes, "q40": q40_kv_bytes}[codec](w, lens)
    return (kv + 2 * w.batch * w.n_q * w.hd * 4 + 4 * used_blocks + 4 * w.batch)
