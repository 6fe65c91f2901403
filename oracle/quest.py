"""QUEST block metadata and query-aware block selection -- TEST INFRASTRUCTURE ONLY.

Plain numpy definitions, used by tests, the smoke check and the benchmark's
CPU-baseline leg only; the product path never imports this module.

Metadata (page "CANN ops-transformer Quest Prefill Metadata" (xdnf.cn),
section on the experiment background): for every KV block of a sequence,
two hd-dimensional vectors -- the per-channel maximum and the per-channel
minimum over the block's tokens of the cached K rows.  Over the int8 cache
a K element is the fp32 product float(code) * k_scale of its row; a
sequence's last block only holds L - (nblk - 1) * kv_bs valid rows.  The
vectors are stored per physical block: kmax, kmin [num_blocks][n_kv][hd].

Selection (same page: at decode, a cheap match of the query against each
block's metadata picks the top-k blocks that take part in attention): the
block's bound for query head h is the largest dot product any vector inside
the block's channel-wise [min, max] box can have with q_h,
    U_h(j) = sum_c max(q_h[c] * kmax[j][c], q_h[c] * kmin[j][c]),
and a kv head's bound is the largest over the query heads that read it.
Readings (the page names the selection operator but does not define it):
  * the block holding the newest token is always kept (its tokens are the
    most recent and, mid-decode, its metadata is not final);
  * the other top_k - 1 blocks are those with the largest bounds, ties to
    the lower logical index;
  * a sequence of at most top_k blocks keeps all of them;
  * the selected blocks keep their logical order, so the selected tokens of
    every kv head form one sequence of (top_k - 1) * kv_bs + (rows of the
    last block) tokens -- the same length for every kv head.
Attention over the selection is the ordinary decode over that per-head
block list (oracle.decode, one kv head at a time).
"""
import numpy as np


def metadata(k_pages, k_scale, block_table, seq_lens, kv_bs):
    """(kmax, kmin) fp32 [num_blocks][n_kv][hd] for every block the table
    references below its sequence's length; other blocks stay NaN."""
    nb, n_kv, _, hd = k_pages.shape
    kmax = np.full((nb, n_kv, hd), np.nan, np.float32)
    kmin = np.full((nb, n_kv, hd), np.nan, np.float32)
    bt = np.asarray(block_table)
    for b in range(bt.shape[0]):
        L = int(seq_lens[b])
        for j in range(-(-max(L, 0) // kv_bs)):
            p = int(bt[b, j])
            rows = min(kv_bs, L - j * kv_bs)
            for kh in range(n_kv):
                k = k_pages[p, kh, :rows].astype(np.float32) * k_scale[p, kh, :rows, None]  # fp32 products
                kmax[p, kh] = k.max(axis=0)
                kmin[p, kh] = k.min(axis=0)
    return kmax, kmin


def bounds(q, kmax, kmin, block_table, seq_lens, n_kv, kv_bs):
    """U [batch][n_kv][max_blocks] float64: each block's bound (the largest
    over the kv head's query heads); -inf past the sequence's blocks."""
    q = np.asarray(q, np.float64)
    batch, n_q, hd = q.shape
    G = n_q // n_kv
    bt = np.asarray(block_table)
    U = np.full((batch, n_kv, bt.shape[1]), -np.inf)
    for b in range(batch):
        nblk = -(-max(int(seq_lens[b]), 0) // kv_bs)
        for kh in range(n_kv):
            for j in range(nblk):
                p = int(bt[b, j])
                mx, mn = kmax[p, kh].astype(np.float64), kmin[p, kh].astype(np.float64)
                U[b, kh, j] = max(np.maximum(q[b, h] * mx, q[b, h] * mn).sum() for h in range(kh * G, (kh + 1) * G))
    return U


def select(U, block_table, seq_lens, kv_bs, top_k):
    """(sel_logical [batch][n_kv][top_k] logical block indices, -1 padded;
    sel_table the matching physical blocks; sel_lens [batch] tokens the
    selection covers)."""
    batch, n_kv, _ = U.shape
    bt = np.asarray(block_table)
    sel = np.full((batch, n_kv, top_k), -1, np.int64)
    lens = np.zeros(batch, np.int32)
    for b in range(batch):
        L = max(int(seq_lens[b]), 0)
        nblk = -(-L // kv_bs)
        if nblk == 0:
            continue
        last_rows = L - (nblk - 1) * kv_bs
        for kh in range(n_kv):
            if nblk <= top_k:
                chosen = list(range(nblk))
            else:
                cand = sorted(range(nblk - 1), key=lambda j: (-U[b, kh, j], j))[:top_k - 1]
                chosen = sorted(cand) + [nblk - 1]
            sel[b, kh, :len(chosen)] = chosen
        lens[b] = (min(nblk, top_k) - 1) * kv_bs + last_rows
    table = np.where(sel >= 0, np.take_along_axis(np.broadcast_to(bt[:, None, :], (batch, n_kv, bt.shape[1])),
                                                  np.maximum(sel, 0), axis=2), -1).astype(np.int32)
    return sel, table, lens
