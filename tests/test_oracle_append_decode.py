"""Pins of the oracle's fused append + decode step (``oracle.append_decode``).

The step stores each sequence's newest token into the paged cache and then
attends over the whole sequence, the new token included.  What pins it, other
than itself:

* the slot of the newest token against a brute-force walk of the block table
  (count positions page by page until position L - 1 is reached);
* the cache it leaves behind and the output it returns against a cache built
  the way every other test builds one -- every token of the sequence appended
  in order through the seeded slot lists of ``workloads`` -- and the decode of
  that cache (bit for bit: the same quantiser and recurrence on the same
  bytes);
* closed forms: a sequence whose only token is the new one returns that
  token's dequantised V row exactly, and a new token whose K row points along
  the query by a wide margin takes (almost) all the softmax weight.
"""
import numpy as np
import pytest

import oracle
import workloads
from cases import POISON_INT8, build


def brute_force_slot(table_row, L, kv_bs):
    """Walk the sequence's pages in order, counting positions, until the
    (L-1)-th is reached; -1 if the walk leaves the row or L <= 0."""
    if L <= 0:
        return -1
    pos = 0
    for blk in table_row:
        for row in range(kv_bs):
            if pos == L - 1:
                return int(blk) * kv_bs + row
            pos += 1
    return -1


def history_and_new(c):
    """A host cache holding tokens 0 .. L-2 of every sequence, and the new
    token's rows [batch][n_kv][hd] (zeros for empty sequences)."""
    w = c.w
    hist = oracle.Cache(c.num_blocks, w.n_kv, w.kv_bs, w.hd, fill_int8=POISON_INT8, fill_scale=np.nan)
    k_new = np.zeros((w.batch, w.n_kv, w.hd), np.float32)
    v_new = np.zeros_like(k_new)
    for b in range(w.batch):
        L = int(c.lens[b])
        if L <= 0:
            continue
        if L > 1:
            hist.append(c.k_src[b][:L - 1], c.v_src[b][:L - 1], c.slots[b][:L - 1])
        k_new[b] = c.k_src[b][L - 1]
        v_new[b] = c.v_src[b][L - 1]
    return hist, k_new, v_new


@pytest.mark.parametrize("kv_bs", [16, 32, 64, 256])
def test_new_slot_brute_force(kv_bs):
    rng = np.random.default_rng(70 + kv_bs)
    batch, max_blocks, num_blocks = 40, 6, 200
    table = np.full((batch, max_blocks), -1, np.int32)
    lens = rng.integers(-2, max_blocks * kv_bs + 1, size=batch).astype(np.int32)
    lens[:6] = [0, 1, kv_bs, kv_bs + 1, max_blocks * kv_bs, -1]
    perm = rng.permutation(num_blocks)
    used = 0
    for b in range(batch):
        nb = -(-max(int(lens[b]), 0) // kv_bs)
        table[b, :nb] = perm[used:used + nb] if used + nb <= num_blocks else rng.integers(0, num_blocks, nb)
        used += nb
    table[7, :] = num_blocks + 3          # entries outside the pool: skipped
    lens[7] = 5
    got = oracle.new_token_slots(table, lens, kv_bs, num_blocks)
    for b in range(batch):
        want = brute_force_slot(table[b], int(lens[b]), kv_bs)
        if want >= num_blocks * kv_bs:
            want = -1
        assert got[b] == want, (b, int(lens[b]))


@pytest.mark.parametrize("hd,G,kv_bs,batch,seq_len", [
    (128, 4, 16, 5, 70), (64, 1, 32, 3, 33), (256, 8, 64, 4, 130), (128, 2, 16, 6, 17),
])
def test_append_decode_equals_full_history(hd, G, kv_bs, batch, seq_len):
    w = workloads.Workload("fuse", batch, 2 * G, 2, hd, kv_bs, seq_len, ragged=True, table="pool",
                           key=600 + hd + G + kv_bs)
    lens = list(workloads.seq_lens(w))
    lens[0] = 1                     # the new token is the whole sequence
    lens[1] = kv_bs                 # newest token in the last row of a page
    if batch > 3:
        lens[2] = kv_bs + 1         # ... in the first row of a fresh page
    lens[-1] = 0                    # empty: nothing stored, zero row
    c = build(w, lens=lens)
    hist, k_new, v_new = history_and_new(c)
    for part_tokens in (0, 32):
        h = oracle.Cache(c.num_blocks, w.n_kv, kv_bs, hd)
        for f in ("k_pages", "v_pages", "k_scale", "v_scale"):
            setattr(h, f, getattr(hist, f).copy())
        got = oracle.append_decode(c.q, h, k_new, v_new, c.table, c.lens, c.scale, part_tokens=part_tokens)
        want = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, part_tokens=part_tokens)
        for f in ("k_pages", "v_pages"):
            assert np.array_equal(getattr(h, f), getattr(c.cache, f)), f
        for f in ("k_scale", "v_scale"):
            assert np.array_equal(getattr(h, f).view(np.uint32), getattr(c.cache, f).view(np.uint32)), f
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
        assert not got[-1].any()


def test_new_token_alone_returns_its_dequantised_v():
    w = workloads.Workload("fuse1", 3, 4, 2, 128, 16, 1, key=611)
    c = build(w, lens=[1, 1, 1])
    hist, k_new, v_new = history_and_new(c)
    out = oracle.append_decode(c.q, hist, k_new, v_new, c.table, c.lens, c.scale)
    vq, vs = oracle.quantize(v_new)            # [batch][n_kv][hd], [batch][n_kv]
    for b in range(3):
        for h in range(4):
            kh = h // 2
            want = (vq[b, kh].astype(np.float32) * vs[b, kh]).astype(np.float32)
            assert np.array_equal(out[b, h], want)


def test_dominant_new_token():
    """A new K row along the query with a wide score margin takes (almost)
    all the weight: the output is the new token's dequantised V row up to the
    other tokens' total weight, bounded by (L-1) e^-margin times max |V|."""
    w = workloads.Workload("fusedom", 2, 2, 1, 128, 16, 300, key=612)
    c = build(w)
    hist, k_new, v_new = history_and_new(c)
    for b in range(2):
        q = c.q[b, 0]
        k_new[b, 0] = 40.0 * q / np.linalg.norm(q)
    c.q[:, 1] = c.q[:, 0]
    out = oracle.append_decode(c.q, hist, k_new, v_new, c.table, c.lens, c.scale)
    vq, vs = oracle.quantize(v_new)
    for b in range(2):
        L = int(c.lens[b])
        k, v, ks, vs_h = oracle.gather_rows(hist, c.table, b, 0, L)
        qi, qsc = oracle.quantize_q(c.q[b, 0])
        s = ((k.astype(np.int64).reshape(L, 4, 32) * qi.astype(np.int64).reshape(4, 32)).sum(-1)
             @ qsc.astype(np.float64)) * ks * c.scale
        margin = s[-1] - s[:-1].max()
        assert margin > 10
        bound = (L - 1) * np.exp(-margin) * 2 * float(np.abs(v * vs_h[:, None]).max()) + 1e-6
        want = vq[b, 0].astype(np.float64) * vs[b, 0]
        assert np.abs(out[b, 0] - want).max() <= bound
