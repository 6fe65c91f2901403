"""decode_attention_int8_amd -- q8-KV single-query decode attention on MI355X.

A thin ctypes binding over ``libq8kv.so`` (C ABI declared in
``include/q8kv.h``).  This module only marshals arguments: it checks tensor
dtypes, devices and contiguity, reads shapes, and passes raw device pointers
and the current HIP stream to the library.  Every step of the computation runs
in the library's HIP kernels; there is no fallback of any kind -- if the
library is not built, importing this package raises.

PyTorch supplies device memory and streams only.
"""
import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# Q8KV_LIBRARY names another build of the same library (the sanitizer test
# loads one whose host code is instrumented); the default is the in-tree one.
LIB_PATH = os.environ.get("Q8KV_LIBRARY") or os.path.join(_HERE, "libq8kv.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "q8kv.h")

Q8KV_OK, Q8KV_EINVAL, Q8KV_ENULL, Q8KV_EHIP, Q8KV_ENOMEM = 0, -1, -2, -3, -4


class Q8KVError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"q8kv error {code}: {message}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; build it with `python decode_attention_int8_amd/build.py` "
            "or __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    sig = {
        "q8kv_decode_attn": [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P],
        "q8kv_decode_attn_split": [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P],
        "q8kv_decode_attn_noalloc": [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P],
        "q8kv_append_decode_attn": [P, P, P, P, I, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P],
        "q8kv_plan": [I, I, I, I, I, I, P, P],
        "q8kv_fp8_append": [P, P, P, P, P, P, I, P, I, I, I, I, I, P],
        "q8kv_quest_metadata": [P, P, P, P, P, P, I, I, I, I, I, I, P],
        "q8kv_q40_append": [P, P, P, P, P, P, I, P, I, I, I, I, I, P],
        "q8kv_q40_decode_attn": [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P],
        "q8kv_quest_select": [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P],
        "q8kv_decode_attn_heads": [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P],
        "q8kv_fp8_decode_attn": [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P],
        "q8kv_append": [P, P, P, P, P, P, I, P, I, I, I, I, I, P],
        "q8kv_import_pages": [P, P, P, P, P, P, P, P, I, I, I, I, P],
        "q8kv_release": [],
        "q8kv_debug_quantize_q": [P, P, P, I, I, P],
        "q8kv_debug_block_dots": [P, I, P, P, P, P, I, I, I, I, I, I, I, P],
        "q8kv_debug_stream_read": [P, ctypes.c_size_t, P, ctypes.c_size_t, P],
        "q8kv_debug_load_probe": [P, P, P, P, I, I, I, I, I, P],
        "q8kv_debug_set_wide": [I],
        "q8kv_debug_set_stage": [I],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = I
    lib.q8kv_last_error.argtypes = []
    lib.q8kv_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def header_symbols():
    """Names of the functions include/q8kv.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(q8kv_\w+)\s*\(", text, re.M)))


def last_error():
    return lib.q8kv_last_error().decode()


def _check(rc):
    if rc != Q8KV_OK:
        raise Q8KVError(rc, last_error())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _call(dev, fn, args):
    """One library call on device dev's current stream, with dev current
    (the library keeps its workspaces per current device)."""
    if torch.cuda.current_device() == dev:
        _check(fn(*args, torch.cuda.current_stream(dev).cuda_stream))
    else:
        with torch.cuda.device(dev):
            _check(fn(*args, torch.cuda.current_stream(dev).cuda_stream))


def _ok(t, dtype, dev, ndim):
    """The per-call check of a tensor argument, kept to a few attribute reads
    (decode calls are issued every few microseconds)."""
    return (isinstance(t, torch.Tensor) and t.dtype is dtype and t.is_cuda and t.get_device() == dev
            and t.dim() == ndim and t.is_contiguous())


def _need(t, name, dtype, device, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def page_hd(hd):
    """Width of an int8 page row for head size hd (a multiple of 32 up to
    256): hd rounded up to 64, 128 or 256; the pad columns hold zero codes."""
    return 64 if hd <= 64 else 128 if hd <= 128 else 256


class PagedKVCache:
    """Device page pool of one layer's q8 KV cache.

    k_pages, v_pages int8 [num_blocks][n_kv][kv_bs][hp], hp = page_hd(hd);
    k_scale, v_scale fp32 [num_blocks][n_kv][kv_bs].
    """

    _TENSORS = ("k_pages", "v_pages", "k_scale", "v_scale")

    def __setattr__(self, name, value):
        # replacing a tensor drops the checked pointers
        if name in PagedKVCache._TENSORS:
            object.__setattr__(self, "_meta", None)
        object.__setattr__(self, name, value)

    def __init__(self, num_blocks, n_kv, kv_bs, hd, device="cuda"):
        dev = torch.device(device)
        self.num_blocks, self.n_kv, self.kv_bs, self.hd = num_blocks, n_kv, kv_bs, hd
        self.hp = page_hd(hd)
        self.k_pages = torch.empty((num_blocks, n_kv, kv_bs, self.hp), dtype=torch.int8, device=dev)
        self.v_pages = torch.empty_like(self.k_pages)
        self.k_scale = torch.empty((num_blocks, n_kv, kv_bs), dtype=torch.float32, device=dev)
        self.v_scale = torch.empty_like(self.k_scale)

    @classmethod
    def wrap(cls, k_pages, v_pages, k_scale, v_scale, hd=None):
        """Use existing tensors as the pool; hd (default: the page width)
        is the head size the pages hold."""
        self = cls.__new__(cls)
        object.__setattr__(self, "_meta", None)
        self.k_pages, self.v_pages, self.k_scale, self.v_scale = k_pages, v_pages, k_scale, v_scale
        self.num_blocks, self.n_kv, self.kv_bs, self.hp = k_pages.shape
        self.hd = self.hp if hd is None else hd
        if page_hd(self.hd) != self.hp:
            raise ValueError(f"pages {self.hp} wide cannot hold head size {self.hd}")
        return self

    @property
    def device(self):
        return self.k_pages.device

    def validate(self):
        d = self.device
        shp = (self.num_blocks, self.n_kv, self.kv_bs, getattr(self, "hp", self.hd))
        for name in ("k_pages", "v_pages"):
            t = getattr(self, name)
            _need(t, name, torch.int8, d, 4)
            if tuple(t.shape) != shp:
                raise ValueError(f"{name} shape {tuple(t.shape)} != {shp}")
        for name in ("k_scale", "v_scale"):
            t = getattr(self, name)
            _need(t, name, torch.float32, d, 3)
            if tuple(t.shape) != shp[:3]:
                raise ValueError(f"{name} shape {tuple(t.shape)} != {shp[:3]}")

    def _pointers(self):
        """(device index, k_pages, v_pages, k_scale, v_scale pointers), checked
        once and kept until a tensor is replaced."""
        meta = getattr(self, "_meta", None)
        if meta is None:
            self.validate()
            if not self.k_pages.is_cuda:
                raise ValueError("the cache must live on a GPU")
            meta = (self.k_pages.get_device(),) + tuple(getattr(self, n).data_ptr() for n in PagedKVCache._TENSORS)
            object.__setattr__(self, "_meta", meta)
        return meta

    _APPEND = "q8kv_append"  # the codec's append entry point

    def append(self, k_src, v_src, slot_mapping):
        """Quantise k_src/v_src [n_tokens][n_kv][hd] (fp32 or bf16) into slots."""
        dev, kp, vp, ks, vs = self._pointers()
        sd = k_src.dtype if isinstance(k_src, torch.Tensor) else None
        if not (sd in (torch.float32, torch.bfloat16) and _ok(k_src, sd, dev, 3) and _ok(v_src, sd, dev, 3)
                and _ok(slot_mapping, torch.int32, dev, 1)):
            d = self.device
            if sd not in (torch.float32, torch.bfloat16):
                raise TypeError("k_src must be a float32 or bfloat16 tensor")
            _need(k_src, "k_src", sd, d, 3)
            _need(v_src, "v_src", sd, d, 3)
            _need(slot_mapping, "slot_mapping", torch.int32, d, 1)
        n = slot_mapping.shape[0]
        if tuple(k_src.shape) != (n, self.n_kv, self.hd) or v_src.shape != k_src.shape:
            raise ValueError("k_src/v_src must be [n_tokens][n_kv][hd] matching slot_mapping")
        args = (kp, vp, ks, vs, k_src.data_ptr(), v_src.data_ptr(), 1 if sd is torch.bfloat16 else 0,
                slot_mapping.data_ptr(), n, self.num_blocks, self.n_kv, self.hd, self.kv_bs)
        _call(dev, getattr(lib, self._APPEND), args)


def import_pages(cache, k_rows, v_rows, k_row_scale, v_row_scale):
    """Fill cache from an int8 cache in row order: k_rows, v_rows int8
    [num_blocks][kv_bs][n_kv][hd], k_row_scale, v_row_scale fp32
    [num_blocks][kv_bs][n_kv], on the cache's device.  Every page and scale
    of cache is rewritten, bit for bit.  Returns cache."""
    if not isinstance(cache, PagedKVCache) or cache.k_pages.dtype != torch.int8:
        raise TypeError("import_pages fills an int8 PagedKVCache")
    dev, kp, vp, ks, vs = cache._pointers()
    d = cache.device
    nb, n_kv, kv_bs, hd = cache.num_blocks, cache.n_kv, cache.kv_bs, cache.hd
    for t, name in ((k_rows, "k_rows"), (v_rows, "v_rows")):
        _need(t, name, torch.int8, d, 4)
        if tuple(t.shape) != (nb, kv_bs, n_kv, hd):
            raise ValueError(f"{name} must be [num_blocks][kv_bs][n_kv][hd] = {(nb, kv_bs, n_kv, hd)}")
    for t, name in ((k_row_scale, "k_row_scale"), (v_row_scale, "v_row_scale")):
        _need(t, name, torch.float32, d, 3)
        if tuple(t.shape) != (nb, kv_bs, n_kv):
            raise ValueError(f"{name} must be [num_blocks][kv_bs][n_kv] = {(nb, kv_bs, n_kv)}")
    args = (kp, vp, ks, vs, k_rows.data_ptr(), v_rows.data_ptr(), k_row_scale.data_ptr(),
            v_row_scale.data_ptr(), nb, n_kv, hd, kv_bs)
    _call(dev, lib.q8kv_import_pages, args)
    return cache


def _decode_io(cache, q, table, seq_lens, out, table_ndim=2):
    """Check q, the block table (table_ndim 2: per sequence; 3: per kv head),
    seq_lens and out against cache; returns (cache pointers, out)."""
    meta = cache._pointers()
    dev = meta[0]
    if not (_ok(q, torch.float32, dev, 3) and _ok(table, torch.int32, dev, table_ndim)
            and _ok(seq_lens, torch.int32, dev, 1)):
        d = cache.device
        _need(q, "q", torch.float32, d, 3)
        _need(table, "block_table", torch.int32, d, table_ndim)
        _need(seq_lens, "seq_lens", torch.int32, d, 1)
    batch, n_q, hd = q.shape
    if (hd != cache.hd or table.shape[0] != batch or seq_lens.shape[0] != batch
            or (table_ndim == 3 and table.shape[1] != cache.n_kv)):
        raise ValueError("q / block_table / seq_lens / cache shapes disagree")
    if out is None:
        out = torch.empty_like(q)
    elif not (_ok(out, torch.float32, dev, 3) and out.shape == q.shape):
        _need(out, "out", torch.float32, cache.device, 3)
        raise ValueError("out must have q's shape")
    return meta, out


def _decode(fn, q, cache, table, seq_lens, scale, out, part_tokens, table_ndim=2):
    """The decode entry points' common call: (out, q, pages and scales,
    table, lengths, table row length, shape, scale, part_tokens)."""
    (dev, kp, vp, ks, vs), out = _decode_io(cache, q, table, seq_lens, out, table_ndim)
    batch, n_q, hd = q.shape
    args = (out.data_ptr(), q.data_ptr(), kp, vp, ks, vs, table.data_ptr(), seq_lens.data_ptr(),
            table.shape[-1], cache.num_blocks, batch, n_q, cache.n_kv, hd, cache.kv_bs, float(scale),
            int(part_tokens))
    _call(dev, fn, args)
    return out


def decode_attn(q, cache, block_table, seq_lens, scale, out=None, part_tokens=0):
    """out[b][h] = softmax(q8 scores) @ q8 V for every sequence b and head h.

    q fp32 [batch][n_q][hd]; block_table int32 [batch][max_blocks];
    seq_lens int32 [batch]; all on the cache's device.  part_tokens 0 picks the
    automatic split plan.  Returns out (fp32 [batch][n_q][hd]).
    """
    return _decode(lib.q8kv_decode_attn_split, q, cache, block_table, seq_lens, scale, out, part_tokens)


def decode_attn_noalloc(q, cache, block_table, seq_lens, scale, out, part_tokens=0):
    """decode_attn through q8kv_decode_attn_noalloc: the same result, bit for
    bit, with no device allocation by the library or this binding (out is
    required).  The library's one scratch array per device is shared by
    every such call: calls that overlap on one device race."""
    if out is None:
        raise ValueError("out is required (the call allocates nothing)")
    return _decode(lib.q8kv_decode_attn_noalloc, q, cache, block_table, seq_lens, scale, out, part_tokens)


def append_decode_attn(q, cache, k_new, v_new, block_table, seq_lens, scale, out=None, part_tokens=0):
    """One decode step that also stores the step's own token, in one launch.

    k_new, v_new [batch][n_kv][hd] fp32 or bf16: the new token's K and V
    rows.  For every sequence with seq_lens[b] >= 1 they are quantised into
    the cache at position seq_lens[b] - 1 (seq_lens already counts the new
    token), then out is decode_attn over positions 0 .. seq_lens[b] - 1.
    Same result, cache bytes and output bits, as cache.append at those slots
    followed by decode_attn.  Returns out (fp32 [batch][n_q][hd]).
    """
    (dev, kp, vp, ks, vs), out = _decode_io(cache, q, block_table, seq_lens, out)
    nd = k_new.dtype if isinstance(k_new, torch.Tensor) else None
    if not (nd in (torch.float32, torch.bfloat16) and _ok(k_new, nd, dev, 3) and _ok(v_new, nd, dev, 3)):
        if nd not in (torch.float32, torch.bfloat16):
            raise TypeError("k_new must be a float32 or bfloat16 tensor")
        _need(k_new, "k_new", nd, cache.device, 3)
        _need(v_new, "v_new", nd, cache.device, 3)
    batch, n_q, hd = q.shape
    if tuple(k_new.shape) != (batch, cache.n_kv, hd) or v_new.shape != k_new.shape:
        raise ValueError("k_new / v_new must be [batch][n_kv][hd]")
    args = (out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
            1 if nd is torch.bfloat16 else 0, kp, vp, ks, vs, block_table.data_ptr(),
            seq_lens.data_ptr(), block_table.shape[1], cache.num_blocks, batch, n_q, cache.n_kv, hd,
            cache.kv_bs, float(scale), int(part_tokens))
    _call(dev, lib.q8kv_append_decode_attn, args)
    return out


class Fp8KVCache(PagedKVCache):
    """Device page pool of one layer's FP8 KV cache (E4M3 codes, one UE8M0
    scale byte per 64 elements of a row).

    k_pages, v_pages uint8 [num_blocks][n_kv][kv_bs][hd] (sub-tile byte order);
    k_scale, v_scale uint8 [num_blocks][n_kv][kv_bs][hd/64].
    """

    _APPEND = "q8kv_fp8_append"

    def __init__(self, num_blocks, n_kv, kv_bs, hd, device="cuda"):
        dev = torch.device(device)
        self.num_blocks, self.n_kv, self.kv_bs, self.hd = num_blocks, n_kv, kv_bs, hd
        self.k_pages = torch.empty((num_blocks, n_kv, kv_bs, hd), dtype=torch.uint8, device=dev)
        self.v_pages = torch.empty_like(self.k_pages)
        self.k_scale = torch.empty((num_blocks, n_kv, kv_bs, hd // 64), dtype=torch.uint8, device=dev)
        self.v_scale = torch.empty_like(self.k_scale)

    @classmethod
    def wrap(cls, k_pages, v_pages, k_scale, v_scale):
        self = cls.__new__(cls)
        object.__setattr__(self, "_meta", None)
        self.k_pages, self.v_pages, self.k_scale, self.v_scale = k_pages, v_pages, k_scale, v_scale
        self.num_blocks, self.n_kv, self.kv_bs, self.hd = k_pages.shape
        return self

    def validate(self):
        d = self.device
        shp = (self.num_blocks, self.n_kv, self.kv_bs, self.hd)
        for name in ("k_pages", "v_pages"):
            t = getattr(self, name)
            _need(t, name, torch.uint8, d, 4)
            if tuple(t.shape) != shp:
                raise ValueError(f"{name} shape {tuple(t.shape)} != {shp}")
        for name in ("k_scale", "v_scale"):
            t = getattr(self, name)
            _need(t, name, torch.uint8, d, 4)
            if tuple(t.shape) != shp[:3] + (self.hd // 64,):
                raise ValueError(f"{name} shape {tuple(t.shape)} != {shp[:3] + (self.hd // 64,)}")


class Q40KVCache(PagedKVCache):
    """Device page pool of one layer's q4_0 KV cache (4-bit codes, one fp16
    scale per 32 elements of a row).

    k_pages, v_pages uint8 [num_blocks][n_kv][kv_bs][hd/2] (sub-tile nibble order);
    k_scale, v_scale float16 [num_blocks][n_kv][kv_bs][hd/32].
    """

    _APPEND = "q8kv_q40_append"

    def __init__(self, num_blocks, n_kv, kv_bs, hd, device="cuda"):
        dev = torch.device(device)
        self.num_blocks, self.n_kv, self.kv_bs, self.hd = num_blocks, n_kv, kv_bs, hd
        self.k_pages = torch.empty((num_blocks, n_kv, kv_bs, hd // 2), dtype=torch.uint8, device=dev)
        self.v_pages = torch.empty_like(self.k_pages)
        self.k_scale = torch.empty((num_blocks, n_kv, kv_bs, hd // 32), dtype=torch.float16, device=dev)
        self.v_scale = torch.empty_like(self.k_scale)

    @classmethod
    def wrap(cls, k_pages, v_pages, k_scale, v_scale):
        self = cls.__new__(cls)
        object.__setattr__(self, "_meta", None)
        self.k_pages, self.v_pages, self.k_scale, self.v_scale = k_pages, v_pages, k_scale, v_scale
        nb, n_kv, kv_bs, half = k_pages.shape
        self.num_blocks, self.n_kv, self.kv_bs, self.hd = nb, n_kv, kv_bs, 2 * half
        return self

    def validate(self):
        d = self.device
        shp = (self.num_blocks, self.n_kv, self.kv_bs)
        for name in ("k_pages", "v_pages"):
            t = getattr(self, name)
            _need(t, name, torch.uint8, d, 4)
            if tuple(t.shape) != shp + (self.hd // 2,):
                raise ValueError(f"{name} shape {tuple(t.shape)} != {shp + (self.hd // 2,)}")
        for name in ("k_scale", "v_scale"):
            t = getattr(self, name)
            _need(t, name, torch.float16, d, 4)
            if tuple(t.shape) != shp + (self.hd // 32,):
                raise ValueError(f"{name} shape {tuple(t.shape)} != {shp + (self.hd // 32,)}")


def q40_decode_attn(q, cache, block_table, seq_lens, scale, out=None, part_tokens=0):
    """decode_attn over a Q40KVCache.  Returns out (fp32 [batch][n_q][hd])."""
    if not isinstance(cache, Q40KVCache):
        raise TypeError("cache must be a Q40KVCache")
    return _decode(lib.q8kv_q40_decode_attn, q, cache, block_table, seq_lens, scale, out, part_tokens)


def fp8_decode_attn(q, cache, block_table, seq_lens, scale, out=None, part_tokens=0):
    """decode_attn over an Fp8KVCache: out[b][h] = softmax(scale q . K) V with
    the dequantised E4M3 K and V.  Returns out (fp32 [batch][n_q][hd])."""
    if not isinstance(cache, Fp8KVCache):
        raise TypeError("cache must be an Fp8KVCache")
    return _decode(lib.q8kv_fp8_decode_attn, q, cache, block_table, seq_lens, scale, out, part_tokens)


def quest_metadata(cache, block_table, seq_lens, kmax=None, kmin=None):
    """Per-block channel max / min of the dequantised K cache (QUEST
    metadata): kmax, kmin fp32 [num_blocks][n_kv][hd], filled for the blocks
    the table references below each sequence's length.  Returns (kmax, kmin)."""
    dev, kp, vp, ks, vs = cache._pointers()
    d = cache.device
    _need(block_table, "block_table", torch.int32, d, 2)
    _need(seq_lens, "seq_lens", torch.int32, d, 1)
    shp = (cache.num_blocks, cache.n_kv, cache.hd)
    if kmax is None:
        kmax = torch.full(shp, float("nan"), dtype=torch.float32, device=d)
    if kmin is None:
        kmin = torch.full(shp, float("nan"), dtype=torch.float32, device=d)
    for t, name in ((kmax, "kmax"), (kmin, "kmin")):
        _need(t, name, torch.float32, d, 3)
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} must be {shp}")
    if block_table.shape[0] != seq_lens.shape[0]:
        raise ValueError("block_table / seq_lens batch sizes disagree")
    with torch.cuda.device(dev):
        _check(lib.q8kv_quest_metadata(kmax.data_ptr(), kmin.data_ptr(), kp, ks, block_table.data_ptr(),
                                       seq_lens.data_ptr(), block_table.shape[1], cache.num_blocks,
                                       block_table.shape[0], cache.n_kv, cache.hd, cache.kv_bs,
                                       torch.cuda.current_stream(dev).cuda_stream))
    return kmax, kmin


def quest_select(q, cache, kmax, kmin, block_table, seq_lens, top_k, sel_table=None, sel_lens=None):
    """QUEST block selection: (sel_table int32 [batch][n_kv][top_k] kept
    physical blocks per kv head in logical order, -1 padded; sel_lens int32
    [batch] tokens they hold)."""
    dev = cache._pointers()[0]
    d = cache.device
    _need(q, "q", torch.float32, d, 3)
    _need(block_table, "block_table", torch.int32, d, 2)
    _need(seq_lens, "seq_lens", torch.int32, d, 1)
    _need(kmax, "kmax", torch.float32, d, 3)
    _need(kmin, "kmin", torch.float32, d, 3)
    batch, n_q, hd = q.shape
    if hd != cache.hd or block_table.shape[0] != batch or seq_lens.shape[0] != batch:
        raise ValueError("q / block_table / seq_lens / cache shapes disagree")
    if tuple(kmax.shape) != (cache.num_blocks, cache.n_kv, hd) or kmin.shape != kmax.shape:
        raise ValueError("kmax / kmin must be [num_blocks][n_kv][hd]")
    if sel_table is None:
        sel_table = torch.empty((batch, cache.n_kv, top_k), dtype=torch.int32, device=d)
    if sel_lens is None:
        sel_lens = torch.empty((batch,), dtype=torch.int32, device=d)
    _need(sel_table, "sel_table", torch.int32, d, 3)
    _need(sel_lens, "sel_lens", torch.int32, d, 1)
    if tuple(sel_table.shape) != (batch, cache.n_kv, top_k) or tuple(sel_lens.shape) != (batch,):
        raise ValueError("sel_table must be [batch][n_kv][top_k] and sel_lens [batch]")
    with torch.cuda.device(dev):
        _check(lib.q8kv_quest_select(sel_table.data_ptr(), sel_lens.data_ptr(), q.data_ptr(), kmax.data_ptr(),
                                     kmin.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
                                     block_table.shape[1], cache.num_blocks, batch, n_q, cache.n_kv, hd,
                                     cache.kv_bs, int(top_k), torch.cuda.current_stream(dev).cuda_stream))
    return sel_table, sel_lens


def decode_attn_heads(q, cache, head_table, seq_lens, scale, out=None, part_tokens=0):
    """decode_attn with one block list per kv head: head_table int32
    [batch][n_kv][max_blocks] (e.g. quest_select's sel_table), seq_lens int32
    [batch].  Returns out (fp32 [batch][n_q][hd])."""
    return _decode(lib.q8kv_decode_attn_heads, q, cache, head_table, seq_lens, scale, out, part_tokens, 3)


def plan(batch, n_q, n_kv, hd, kv_bs, max_blocks):
    """(tokens per partition, partitions of the longest sequence) of the
    automatic split plan."""
    pt, npart = ctypes.c_int(), ctypes.c_int()
    _check(lib.q8kv_plan(batch, n_q, n_kv, hd, kv_bs, max_blocks, ctypes.byref(pt), ctypes.byref(npart)))
    return pt.value, npart.value


def debug_stream_read(a, b):
    """Measurement export: one plain linear read of the device tensors a and b
    (contiguous, sizes multiples of 16 bytes) on the current stream."""
    for t in (a, b):
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
            raise ValueError("stream-read buffers must be contiguous device tensors")
    nb = lambda t: t.numel() * t.element_size()
    with torch.cuda.device(a.device):
        _check(lib.q8kv_debug_stream_read(a.data_ptr(), nb(a), b.data_ptr(), nb(b),
                                          torch.cuda.current_stream(a.device).cuda_stream))


def debug_load_probe(cache, item_pages, pattern, num_pages=None):
    """Issue the decode kernel's loads over cache's pools without its
    arithmetic (q8kv_debug_load_probe; pattern 0, 1 or 2)."""
    dev, kp, vp, ks, vs = cache._pointers()
    if num_pages is None:
        num_pages = cache.num_blocks * cache.n_kv // item_pages * item_pages
    _call(dev, lib.q8kv_debug_load_probe, (kp, vp, ks, vs, num_pages, cache.hp, cache.kv_bs, item_pages, pattern))


def release():
    _check(lib.q8kv_release())


def debug_set_wide(enable):
    """Test export: allow (True, the default) or forbid the 8-wave workgroups
    of static grids of at most one workgroup per CU."""
    _check(lib.q8kv_debug_set_wide(1 if enable else 0))


def debug_set_stage(enable):
    """Test export: use (True) or not (False, the default) the LDS-staged
    int8 static-grid kernels; same results, bit for bit."""
    _check(lib.q8kv_debug_set_stage(1 if enable else 0))


def debug_quantize_q(q):
    """Test export: the decode prologue's int8 query and per-32-block scales."""
    if q.dtype != torch.float32 or not q.is_cuda or not q.is_contiguous():
        raise ValueError("q must be a contiguous float32 device tensor")
    hd = q.shape[-1]
    rows = q.numel() // hd
    qi = torch.empty(q.shape, dtype=torch.int8, device=q.device)
    qsc = torch.empty(q.shape[:-1] + (hd // 32,), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        _check(lib.q8kv_debug_quantize_q(_ptr(qi), _ptr(qsc), _ptr(q), rows, hd, _stream(q.device)))
    return qi, qsc


def debug_block_dots(q, cache, block_table, seq_lens, max_tok):
    """Test export: int32 dots [batch][n_q][max_tok][hd/32] from the decode
    kernel's matrix-core scoring step (entries past seq_len stay zero)."""
    cache.validate()
    d = cache.device
    _need(q, "q", torch.float32, d, 3)
    _need(block_table, "block_table", torch.int32, d, 2)
    _need(seq_lens, "seq_lens", torch.int32, d, 1)
    batch, n_q, hd = q.shape
    dots = torch.zeros((batch, n_q, max_tok, hd // 32), dtype=torch.int32, device=d)
    with torch.cuda.device(d):
        _check(lib.q8kv_debug_block_dots(
            _ptr(dots), max_tok, _ptr(q), _ptr(cache.k_pages), _ptr(block_table), _ptr(seq_lens),
            block_table.shape[1], cache.num_blocks, batch, n_q, cache.n_kv, hd, cache.kv_bs,
            _stream(d)))
    return dots
