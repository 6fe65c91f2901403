"""GPU-side assembly for the parity tests: the same seeded fp32 sources the
oracle quantises on the host are quantised on the GPU by q8kv_append, then
decoded by q8kv_decode_attn.  Nothing here computes any part of the method."""
import sys

import numpy as np
import torch

import decode_attention_int8_amd as q8
from cases import POISON_INT8

DEV = torch.device("cuda", 0)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    return t if dtype is None else t.to(dtype)


def gpu_cache(c, poison=True, src_dtype=torch.float32, seqs=None):
    """Append every sequence's fp32 (or bf16) source rows into a device cache."""
    w = c.w
    cache = q8.PagedKVCache(c.num_blocks, w.n_kv, w.kv_bs, w.hd, device=DEV)
    cache.k_pages.fill_(POISON_INT8 if poison else 0)
    cache.v_pages.fill_(POISON_INT8 if poison else 0)
    cache.k_scale.fill_(float("nan") if poison else 0.0)
    cache.v_scale.fill_(float("nan") if poison else 0.0)
    for b in (range(w.batch) if seqs is None else seqs):
        if len(c.slots[b]) == 0:
            continue
        cache.append(to_dev(c.k_src[b], src_dtype), to_dev(c.v_src[b], src_dtype), to_dev(c.slots[b]))
    return cache


def dev_inputs(c):
    return to_dev(c.q), to_dev(c.table), to_dev(c.lens)


def decode(c, cache, part_tokens=0, lens=None):
    q, bt, sl = dev_inputs(c)
    if lens is not None:
        sl = to_dev(np.asarray(lens, np.int32))
    out = q8.decode_attn(q, cache, bt, sl, c.scale, part_tokens=part_tokens)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def chunk_offsets(hd, which):
    """Byte offset, inside a 16-row sub-tile of a device page, of element
    (row, column) -- the page byte order include/q8kv.h documents: 1 KB chunks
    of 64 lane slots x 16 bytes; K chunk c slot 16r+n holds row n, columns
    64c+16r..+16; V slot 16r+n holds rows 4r..4r+3 x columns BPL n..+BPL
    (BPL = hd/16) in (row, column) order, cut into 16-byte pieces, piece c in
    chunk c."""
    row = np.arange(16)[:, None]
    col = np.arange(hd)[None, :]
    if which == "k":
        return (col // 64) * 1024 + 16 * (16 * ((col % 64) // 16) + row) + col % 16
    bpl = hd // 16
    slot = 16 * (row // 4) + col // bpl
    qb = (row % 4) * bpl + col % bpl
    return (qb // 16) * 1024 + 16 * slot + qb % 16


def fp8_v_offsets(hd):
    """Byte offset, inside a 16-row sub-tile of an FP8 V page, of element
    (row, column), as include/q8kv.h defines it: slot 16r+n holds rows
    4r..4r+3 of columns 16s+n; dword s (those four rows in row order) lies in
    chunk s/4 at bytes 4(s%4)..."""
    row = np.arange(16)[:, None]
    col = np.arange(hd)[None, :]
    slot = 16 * (row // 4) + col % 16
    qb = 4 * (col // 16) + row % 4
    return (qb // 16) * 1024 + 16 * slot + qb % 16


def natural_fp8_pages(pages, which):
    """FP8 device pages [nb][n_kv][kv_bs][hd] in chunk order -> row-major rows
    (K uses the int8 K order)."""
    nb, n_kv, kv_bs, hd = pages.shape
    sub = pages.reshape(nb, n_kv, kv_bs // 16, 16 * hd)
    off = chunk_offsets(hd, "k") if which == "k" else fp8_v_offsets(hd)
    return sub[..., off.reshape(-1)].reshape(nb, n_kv, kv_bs, hd)


def q40_codes(pages, which):
    """q4_0 device pages [nb][n_kv][kv_bs][hd/2] (sub-tile nibble order) ->
    codes [nb][n_kv][kv_bs][hd] in row order, as include/q8kv.h defines the
    order: slot 16r+n owns hd/8 bytes; K byte 8c+i = row n, columns
    64c+16r+i (low nibble) and 64c+16r+8+i (high); V byte 4(s/2)+j = row
    4r+j, column 16s+n, even s low nibble, odd s high."""
    nb, n_kv, kv_bs, half = pages.shape
    hd = 2 * half
    sub = pages.reshape(nb, n_kv, kv_bs // 16, 16 * half)
    out = np.empty((nb, n_kv, kv_bs // 16, 16, hd), np.uint8)
    for row in range(16):
        for col in range(hd):
            if which == "k":
                r, n = (col % 64) // 16, row
                i = col % 16
                byte = (16 * r + n) * (hd // 8) + 8 * (col // 64) + (i % 8)
                hi = i >= 8
            else:
                r, n = row // 4, col % 16
                s_ = col // 16
                byte = (16 * r + n) * (hd // 8) + 4 * (s_ // 2) + row % 4
                hi = (s_ % 2) == 1
            b = sub[..., byte]
            out[:, :, :, row, col] = (b >> 4) if hi else (b & 15)
    return out.reshape(nb, n_kv, kv_bs, hd)


def natural_pages(pages, which):
    """Device pages [nb][n_kv][kv_bs][hp] in chunk order -> row-major rows
    (hp wide: a padded head's pad columns included)."""
    nb, n_kv, kv_bs, hd = pages.shape
    sub = pages.reshape(nb, n_kv, kv_bs // 16, 16 * hd)
    return sub[..., chunk_offsets(hd, which).reshape(-1)].reshape(nb, n_kv, kv_bs, hd)


def assert_cache_equal(host, dev, blocks=None):
    """Bitwise equality of pages (in row order) and scales (NaN == NaN for
    poisoned rows).  Pages wider than the head size hold zero codes in the
    pad columns of every written row (a row whose host scale is a number)
    and the pool's fill in the rest."""
    for f in ("k_pages", "v_pages", "k_scale", "v_scale"):
        a = getattr(host, f)
        b = getattr(dev, f).cpu().numpy()
        if f.endswith("pages"):
            b = natural_pages(b, f[0])
        if blocks is not None:
            a, b = a[blocks], b[blocks]
        if f.endswith("pages") and b.shape[-1] > a.shape[-1]:
            written = ~np.isnan(getattr(host, f[0] + "_scale"))
            if blocks is not None:
                written = written[blocks]
            pad = b[..., a.shape[-1]:]
            want = np.where(written[..., None], np.int8(0), a[..., :1])
            assert np.array_equal(pad, np.broadcast_to(want, pad.shape)), f + " pad columns"
            b = b[..., :a.shape[-1]]
        if a.dtype == np.float32:
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f
        else:
            assert np.array_equal(a, b), f
