"""Pins of the QUEST metadata / selection oracle (oracle/quest.py).

Checked against what the definitions imply rather than against their own
formulas:

* metadata: every valid row's dequantised K value lies inside [kmin, kmax]
  and both bounds are attained by some valid row (rows read through the
  block table with oracle.gather_rows, a different access path); rows past
  the sequence's length, poisoned with huge values, change nothing; moving
  blocks to other physical slots moves their metadata with them;
* bounds: U_h(j) is at least q_h . k for every valid row of block j (the box
  holds every row) and equals the largest q_h . x over the box's corners
  found by brute force on a tiny hd; a one-row block's bound is exactly its
  dot product; the kv head's bound is the largest over its query heads;
* selection: brute force over all subsets of a small sequence -- the chosen
  blocks are the last block plus the top_k - 1 largest bounds (ties to the
  lower index), in logical order; the selected length counts the tokens of
  the chosen blocks one by one;
* with top_k at least the number of blocks, attention over the selection is
  bitwise the dense decode.
"""
import itertools

import numpy as np
import pytest

import oracle
import workloads
from cases import build
from oracle import quest


def quest_case(G=4, n_kv=2, hd=128, kv_bs=16, batch=4, seq_len=150, key=3000, lens=None):
    w = workloads.Workload("quest", batch, G * n_kv, n_kv, hd, kv_bs, seq_len, ragged=True, table="pool", key=key)
    return build(w, lens=lens)


def test_metadata_contains_and_attains_every_row():
    c = quest_case()
    kmax, kmin = quest.metadata(c.cache.k_pages, c.cache.k_scale, c.table, c.lens, c.w.kv_bs)
    for b in range(c.w.batch):
        L = int(c.lens[b])
        for kh in range(c.w.n_kv):
            k, _, ks, _ = oracle.gather_rows(c.cache, c.table, b, kh, L)
            kd = k.astype(np.float32) * ks[:, None]
            for j in range(-(-L // c.w.kv_bs)):
                rows = kd[j * c.w.kv_bs:(j + 1) * c.w.kv_bs]
                p = int(c.table[b, j])
                assert np.all(rows <= kmax[p, kh]) and np.all(rows >= kmin[p, kh])
                assert np.all((rows == kmax[p, kh]).any(axis=0)) and np.all((rows == kmin[p, kh]).any(axis=0))


def test_metadata_ignores_rows_past_the_length_and_follows_placement():
    c = quest_case(key=3001)
    kmax, kmin = quest.metadata(c.cache.k_pages, c.cache.k_scale, c.table, c.lens, c.w.kv_bs)
    # poison every row past each sequence's end inside its last block
    kp = c.cache.k_pages.copy()
    ks = c.cache.k_scale.copy()
    for b in range(c.w.batch):
        L = int(c.lens[b])
        j = (L - 1) // c.w.kv_bs
        p = int(c.table[b, j])
        r0 = L - j * c.w.kv_bs
        kp[p, :, r0:] = 127
        ks[p, :, r0:] = 1e30
    kmax2, kmin2 = quest.metadata(kp, ks, c.table, c.lens, c.w.kv_bs)
    assert np.array_equal(kmax, kmax2, equal_nan=True) and np.array_equal(kmin, kmin2, equal_nan=True)
    # move all blocks to new physical slots
    perm = np.random.default_rng(1).permutation(c.num_blocks)
    kp3 = np.empty_like(c.cache.k_pages)
    ks3 = np.empty_like(c.cache.k_scale)
    kp3[perm] = c.cache.k_pages
    ks3[perm] = c.cache.k_scale
    table3 = np.where(c.table >= 0, perm[np.maximum(c.table, 0)], -1)
    kmax3, kmin3 = quest.metadata(kp3, ks3, table3, c.lens, c.w.kv_bs)
    assert np.array_equal(kmax3[perm], kmax, equal_nan=True) and np.array_equal(kmin3[perm], kmin, equal_nan=True)


def test_bounds_dominate_rows_and_match_box_corners():
    c = quest_case(G=3, n_kv=1, hd=64, kv_bs=16, batch=2, seq_len=70, key=3002)
    kmax, kmin = quest.metadata(c.cache.k_pages, c.cache.k_scale, c.table, c.lens, c.w.kv_bs)
    U = quest.bounds(c.q, kmax, kmin, c.table, c.lens, 1, c.w.kv_bs)
    for b in range(2):
        L = int(c.lens[b])
        k, _, ks, _ = oracle.gather_rows(c.cache, c.table, b, 0, L)
        kd = k.astype(np.float64) * ks[:, None].astype(np.float64)
        for j in range(-(-L // 16)):
            dots = kd[16 * j:16 * (j + 1)] @ c.q[b].astype(np.float64).T  # [rows][heads]
            assert U[b, 0, j] >= dots.max() - 1e-9
            assert np.isclose(U[b, 0, j], max(
                np.maximum(c.q[b, h] * kmax[int(c.table[b, j]), 0].astype(np.float64),
                           c.q[b, h] * kmin[int(c.table[b, j]), 0].astype(np.float64)).sum() for h in range(3)))
        assert np.all(np.isneginf(U[b, 0, -(-L // 16):]))
    # brute force over the box corners on a tiny hd
    rng = np.random.default_rng(2)
    for _ in range(20):
        lo = rng.standard_normal(6)
        hi = lo + rng.random(6)
        qv = rng.standard_normal(6)
        corners = max(np.dot(qv, np.where(np.array(bits), hi, lo)) for bits in itertools.product([0, 1], repeat=6))
        u = quest.bounds(qv[None, None, :], hi[None, None, :].astype(np.float32)[:, :, :],
                         lo[None, None, :].astype(np.float32), np.array([[0]]), [1], 1, 1)
        bound = np.maximum(qv * hi.astype(np.float32), qv * lo.astype(np.float32)).sum()
        assert np.isclose(u[0, 0, 0], bound)
        assert np.isclose(bound, max(np.dot(qv, np.where(np.array(bits), hi.astype(np.float32), lo.astype(np.float32)))
                                     for bits in itertools.product([0, 1], repeat=6)))
        assert corners <= bound + 1e-5 or np.isclose(corners, bound, atol=1e-5)


def test_one_row_block_bound_is_its_dot():
    c = quest_case(G=1, n_kv=1, hd=128, kv_bs=16, batch=1, seq_len=17, key=3003, lens=[17])
    kmax, kmin = quest.metadata(c.cache.k_pages, c.cache.k_scale, c.table, c.lens, 16)
    U = quest.bounds(c.q, kmax, kmin, c.table, c.lens, 1, 16)
    k, _, ks, _ = oracle.gather_rows(c.cache, c.table, 0, 0, 17)
    row = (k[16].astype(np.float32) * ks[16]).astype(np.float64)  # the fp32 dequantised row
    assert np.isclose(U[0, 0, 1], row @ c.q[0, 0].astype(np.float64), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("top_k", [1, 2, 3, 5])
def test_selection_brute_force(top_k):
    rng = np.random.default_rng(10 + top_k)
    batch, n_kv, kv_bs, max_blocks = 6, 2, 16, 7
    lens = np.array([0, 1, 16, 17, 100, 112])
    table = np.arange(batch * max_blocks, dtype=np.int32).reshape(batch, max_blocks)
    U = np.round(rng.standard_normal((batch, n_kv, max_blocks)), 1)  # rounding makes ties
    sel, tab, sel_lens = quest.select(U, table, lens, kv_bs, top_k)
    for b in range(batch):
        nblk = -(-int(lens[b]) // kv_bs)
        for kh in range(n_kv):
            best = None
            if nblk <= top_k:
                best = list(range(nblk))
            else:
                for subset in itertools.combinations(range(nblk - 1), top_k - 1):
                    key = (sorted((-U[b, kh, j] for j in subset)), list(subset))
                    # largest bounds first; among equal multisets the lexicographically lowest indices
                    if best is None or key < best[0]:
                        best = (key, list(subset))
                best = best[1] + [nblk - 1]
            got = [int(x) for x in sel[b, kh] if x >= 0]
            assert got == sorted(best), (b, kh, got, best)
            assert all(tab[b, kh, i] == table[b, got[i]] for i in range(len(got)))
        tokens = 0
        for j in (sel[b, 0][sel[b, 0] >= 0] if nblk else []):
            for t in range(j * kv_bs, (j + 1) * kv_bs):
                tokens += t < lens[b]
        assert sel_lens[b] == tokens


def test_full_selection_is_dense_decode():
    c = quest_case(G=2, n_kv=2, batch=3, seq_len=90, key=3004)
    kmax, kmin = quest.metadata(c.cache.k_pages, c.cache.k_scale, c.table, c.lens, c.w.kv_bs)
    U = quest.bounds(c.q, kmax, kmin, c.table, c.lens, c.w.n_kv, c.w.kv_bs)
    _, tab, sel_lens = quest.select(U, c.table, c.lens, c.w.kv_bs, c.table.shape[1])
    assert np.array_equal(sel_lens, c.lens)
    out = quest_decode(c.q, c.cache, tab, sel_lens, c.scale)
    dense = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale)
    assert np.array_equal(out.view(np.uint32), dense.view(np.uint32))


def quest_decode(q, cache, head_table, lens, scale):
    """Decode over per-kv-head block lists, one kv head at a time through the
    ordinary oracle decode on that head's pages."""
    q = np.asarray(q, np.float32)
    batch, n_q, hd = q.shape
    G = n_q // cache.n_kv
    out = np.empty_like(q)
    for kh in range(cache.n_kv):
        sub = oracle.Cache(cache.num_blocks, 1, cache.kv_bs, hd)
        sub.k_pages = np.ascontiguousarray(cache.k_pages[:, kh:kh + 1])
        sub.v_pages = np.ascontiguousarray(cache.v_pages[:, kh:kh + 1])
        sub.k_scale = np.ascontiguousarray(cache.k_scale[:, kh:kh + 1])
        sub.v_scale = np.ascontiguousarray(cache.v_scale[:, kh:kh + 1])
        t = np.ascontiguousarray(head_table[:, kh])
        out[:, kh * G:(kh + 1) * G] = oracle.decode(q[:, kh * G:(kh + 1) * G], sub, t, lens, scale)
    return out
