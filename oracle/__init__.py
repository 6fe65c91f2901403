"""q8kv CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct CPU implementations of what the GPU library
computes, used by the tests, the smoke check and the benchmark's CPU-baseline
leg and by nothing else.  The product path (``decode_attention_int8_amd``)
never imports this package; this package never imports the product.

Two layers:

* ``liboracle_q8kv.so`` (``q8kv_oracle.c``): the page's single-pass recurrence
  in fp32, in the page's order (page "Day 9-2: flash_attn_single_q_q8_neon",
  trdm.cn, section 2, segments 1-3), its double-precision twin, the
  split-range merge, a per-token trace, the int32 block dots and the K/V
  append quantiser.
* plain numpy references in float64:
    - ``three_pass_f64``: the textbook three passes (all scores, then a
      max-subtracted softmax, then the weighted sum of V) as in the llama2.c
      attention walkthrough (aicoding.csdn.net page, section 2 "attention
      core" and section 3 "softmax"), fed with the same int8 values and
      scales as the single pass;
    - ``exact_f64``: softmax attention on the unquantised fp32 q, K, V, used to
      report how far q8 KV moves the output.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(closed forms, invariants, exact-rational quantiser checks, int64 brute force,
Decimal brute force of the softmax); see the module docstrings of
``tests/test_oracle_*.py``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _configure(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    F = ctypes.c_float
    lib.orc_inv127.restype = F
    lib.orc_m_init.restype = F
    lib.orc_max_threads.restype = I
    lib.orc_quantize.argtypes = [P, I, P, P]
    lib.orc_quantize.restype = None
    lib.orc_quantize_q.argtypes = [P, P, P, I, I]
    lib.orc_quantize_q.restype = None
    lib.orc_append.argtypes = [P, P, P, P, P, P, I, P, I, I, I, I]
    lib.orc_append.restype = None
    lib.orc_decode.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I, I]
    lib.orc_decode.restype = I
    lib.orc_decode_trace.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, I]
    lib.orc_decode_trace.restype = I
    lib.orc_block_dots.argtypes = [P, I, P, P, P, P, I, I, I, I, I, I]
    lib.orc_block_dots.restype = I
    return lib


def _load():
    """The oracle library: oracle/liboracle_q8kv.so (built on first use), or
    the build named by Q8KV_ORACLE_LIB (the sanitizer test points it at an
    instrumented copy)."""
    global _LIB
    if _LIB is None:
        path = os.environ.get("Q8KV_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        _LIB = _configure(ctypes.CDLL(path))
    return _LIB


def _use_library(path):
    """Point this wrapper at another build of the oracle (the mutation tests
    load deliberately broken copies) and return the handle it replaced;
    ``_use_library(None)`` goes back to the real one."""
    global _LIB
    prev = _LIB
    _LIB = None if path is None else _configure(ctypes.CDLL(path))
    return prev


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def inv127():
    """fp32(1/127) as the oracle uses it."""
    return float(np.float32(_load().orc_inv127()))


def m_init():
    """Initial running maximum of the recurrence (-1e9 in fp32)."""
    return float(np.float32(_load().orc_m_init()))


def max_threads():
    return int(_load().orc_max_threads())


def quantize(x):
    """Quantise each row of x (any leading shape, last axis = one scale group).

    Returns (int8 values of x's shape, fp32 scales of shape x.shape[:-1]).
    """
    x = _c(x, np.float32)
    n = x.shape[-1]
    rows = x.reshape(-1, n)
    qv = np.empty(rows.shape, np.int8)
    sc = np.empty(rows.shape[0], np.float32)
    lib = _load()
    for r in range(rows.shape[0]):
        lib.orc_quantize(_p(rows[r]), n, _p(qv[r:]), _p(sc[r:]))
    return qv.reshape(x.shape), sc.reshape(x.shape[:-1])


def quantize_q(q):
    """q [..., hd] -> (int8 [..., hd], fp32 scales [..., hd/32])."""
    q = _c(q, np.float32)
    hd = q.shape[-1]
    rows = q.reshape(-1, hd)
    qi = np.empty(rows.shape, np.int8)
    qsc = np.empty((rows.shape[0], hd // 32), np.float32)
    _load().orc_quantize_q(_p(qi), _p(qsc), _p(rows), rows.shape[0], hd)
    return qi.reshape(q.shape), qsc.reshape(q.shape[:-1] + (hd // 32,))


class Cache:
    """Host copy of a paged q8 KV cache in the library's layout.

    k_pages, v_pages int8 [num_blocks][n_kv][kv_bs][hd];
    k_scale, v_scale fp32 [num_blocks][n_kv][kv_bs].
    ``fill`` sets every byte/scale first (poison for never-read rows).
    """

    def __init__(self, num_blocks, n_kv, kv_bs, hd, fill_int8=0, fill_scale=0.0):
        self.num_blocks, self.n_kv, self.kv_bs, self.hd = num_blocks, n_kv, kv_bs, hd
        self.k_pages = np.full((num_blocks, n_kv, kv_bs, hd), fill_int8, np.int8)
        self.v_pages = np.full((num_blocks, n_kv, kv_bs, hd), fill_int8, np.int8)
        self.k_scale = np.full((num_blocks, n_kv, kv_bs), fill_scale, np.float32)
        self.v_scale = np.full((num_blocks, n_kv, kv_bs), fill_scale, np.float32)

    def append(self, k_src, v_src, slot_mapping):
        """Quantise [n_tokens][n_kv][hd] fp32 (or bf16 as uint16/torch bf16 bits)."""
        if k_src.dtype == np.uint16:
            dt = 1
        else:
            dt = 0
            k_src = _c(k_src, np.float32)
            v_src = _c(v_src, np.float32)
        k_src = np.ascontiguousarray(k_src)
        v_src = np.ascontiguousarray(v_src)
        sm = _c(slot_mapping, np.int32)
        n = sm.shape[0]
        assert k_src.shape == (n, self.n_kv, self.hd) and v_src.shape == k_src.shape
        assert np.all(sm < self.num_blocks * self.kv_bs)
        _load().orc_append(_p(self.k_pages), _p(self.v_pages), _p(self.k_scale), _p(self.v_scale),
                           _p(k_src), _p(v_src), dt, _p(sm), n, self.n_kv, self.hd, self.kv_bs)


def decode(q, cache, block_table, seq_lens, scale, part_tokens=0, use_f64=False, threads=1):
    """Decode attention out [batch][n_q][hd] fp32 via the page's recurrence.

    part_tokens > 0 runs the split-range form (each range its own recurrence,
    then the ordered log-sum-exp merge).  use_f64 runs the double twin.
    threads > 1 spreads (b, h) pairs over OpenMP threads (bitwise the same).
    """
    q = _c(q, np.float32)
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    batch, n_q, hd = q.shape
    out = np.empty_like(q)
    rc = _load().orc_decode(_p(out), _p(q), _p(cache.k_pages), _p(cache.v_pages),
                            _p(cache.k_scale), _p(cache.v_scale), _p(bt), _p(sl),
                            bt.shape[1], batch, n_q, cache.n_kv, hd, cache.kv_bs,
                            float(np.float32(scale)), int(part_tokens), int(bool(use_f64)),
                            int(threads))
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments")
    return out


def decode_trace(q, cache, block_table, seq_lens, scale, b, h):
    """One (b, h) row plus the per-token trace (s_t, M_t, S_t, w_t)."""
    q = _c(q, np.float32)
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    batch, n_q, hd = q.shape
    L = max(int(sl[b]), 1)
    out = np.empty(hd, np.float32)
    tr = [np.zeros(L, np.float32) for _ in range(4)]
    rc = _load().orc_decode_trace(_p(out), *[_p(t) for t in tr], _p(q), _p(cache.k_pages),
                                  _p(cache.v_pages), _p(cache.k_scale), _p(cache.v_scale),
                                  _p(bt), _p(sl), bt.shape[1], batch, n_q, cache.n_kv, hd,
                                  cache.kv_bs, float(np.float32(scale)), b, h)
    if rc != 0:
        raise ValueError("oracle trace rejected its arguments")
    n = int(sl[b])
    return out, tuple(t[:max(n, 0)] for t in tr)


def block_dots(q, cache, block_table, seq_lens, max_tok=None):
    """int32 dots [batch][n_q][max_tok][hd/32]; entries at t >= seq_len are 0."""
    q = _c(q, np.float32)
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    batch, n_q, hd = q.shape
    if max_tok is None:
        max_tok = int(sl.max()) if sl.size else 0
    dots = np.zeros((batch, n_q, max_tok, hd // 32), np.int32)
    rc = _load().orc_block_dots(_p(dots), max_tok, _p(q), _p(cache.k_pages), _p(bt), _p(sl),
                                bt.shape[1], batch, n_q, cache.n_kv, hd, cache.kv_bs)
    if rc != 0:
        raise ValueError("oracle block_dots rejected its arguments")
    return dots


def new_token_slots(block_table, seq_lens, kv_bs, num_blocks):
    """Cache slot of each sequence's newest token, position L - 1 with
    L = seq_lens[b]: physical block block_table[b][(L-1) // kv_bs] times kv_bs
    plus the row (L-1) % kv_bs -- the block-number x block-size + offset rule
    for turning a sequence position into a global cache slot (page
    "deepseek-attention-div64", beaiera.top, section on mapping top-k indices
    to global slot ids).  -1 (skip) where L <= 0, where L - 1 lies past the
    table row, or where the entry is outside [0, num_blocks)."""
    bt = np.asarray(block_table)
    slots = np.full(bt.shape[0], -1, np.int32)
    for b in range(bt.shape[0]):
        L = int(seq_lens[b])
        if L <= 0 or (L - 1) // kv_bs >= bt.shape[1]:
            continue
        blk = int(bt[b, (L - 1) // kv_bs])
        if 0 <= blk < num_blocks:
            slots[b] = blk * kv_bs + (L - 1) % kv_bs
    return slots


def append_decode(q, cache, k_new, v_new, block_table, seq_lens, scale, part_tokens=0,
                  use_f64=False, threads=1):
    """One decode step that first stores the step's own token: quantise the
    new K/V rows k_new, v_new [batch][n_kv][hd] into ``cache`` (in place) at
    each sequence's newest slot (``new_token_slots``), then ``decode`` over
    positions 0 .. seq_lens[b] - 1, the new token included.  Returns out."""
    slots = new_token_slots(block_table, seq_lens, cache.kv_bs, cache.num_blocks)
    cache.append(k_new, v_new, slots)
    return decode(q, cache, block_table, seq_lens, scale, part_tokens=part_tokens,
                  use_f64=use_f64, threads=threads)


# ----------------------------------------------------------------------------
# float64 references in plain numpy


def gather_rows(cache, block_table, b, kh, L):
    """Logical token rows 0..L-1 of sequence b, kv head kh, read through the
    block table with numpy indexing: (k int8 [L][hd], v int8, ks [L], vs [L])."""
    t = np.arange(L)
    blk = np.asarray(block_table)[b, t // cache.kv_bs]
    r = t % cache.kv_bs
    return (cache.k_pages[blk, kh, r], cache.v_pages[blk, kh, r],
            cache.k_scale[blk, kh, r], cache.v_scale[blk, kh, r])


def three_pass_f64(q, cache, block_table, seq_lens, scale):
    """All scores first, then softmax (max-subtracted exp, sum, divide), then
    the weighted sum of dequantised V -- three passes, all float64, on the very
    int8 values and fp32 scales the single pass uses.  Rows with seq_len <= 0
    are zero."""
    q = np.asarray(q, np.float32)
    batch, n_q, hd = q.shape
    G = n_q // cache.n_kv
    qi, qsc = quantize_q(q)
    out = np.zeros((batch, n_q, hd), np.float64)
    for b in range(batch):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        for kh in range(cache.n_kv):
            k, v, ks, vs = gather_rows(cache, block_table, b, kh, L)
            kb = k.astype(np.int64).reshape(L, hd // 32, 32)
            vd = v.astype(np.float64) * vs.astype(np.float64)[:, None]
            for h in range(kh * G, (kh + 1) * G):
                qb = qi[b, h].astype(np.int64).reshape(hd // 32, 32)
                dots = np.einsum("tbi,bi->tb", kb, qb)  # int64, exact
                s = (dots.astype(np.float64) @ qsc[b, h].astype(np.float64))
                s = s * ks.astype(np.float64) * float(np.float32(scale))
                p = np.exp(s - s.max())
                p = p / p.sum()
                out[b, h] = p @ vd
    return out


def exact_f64(q, k_rows, v_rows, scale):
    """Softmax attention of one query row over unquantised rows, float64.

    q [hd]; k_rows, v_rows [L][hd] (any float dtype).  Returns [hd].
    """
    qd = np.asarray(q, np.float64)
    kd = np.asarray(k_rows, np.float64)
    vd = np.asarray(v_rows, np.float64)
    s = (kd @ qd) * float(np.float32(scale))
    p = np.exp(s - s.max())
    return (p / p.sum()) @ vd
