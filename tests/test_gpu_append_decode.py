"""GPU parity of the fused append + decode step (q8kv_append_decode_attn).

Each case starts from a device cache that holds tokens 0 .. L-2 of every
sequence (appended by q8kv_append from the seeded sources) and calls the
fused step with token L-1's K/V rows.  It checks:

* the cache afterwards against the oracle's (``oracle.append_decode`` on the
  host copy of the same history), bit for bit;
* the output against the oracle (fp32 and fp64 twins) within the decode
  tolerances;
* the output against the library's own two-launch path (q8kv_append at the
  same slots, then q8kv_decode_attn_split with the same partition length),
  bit for bit: the fused kernel patches the new row into its tile registers
  instead of reading it back, and must not change a single result bit.

Lengths are chosen so that the new token lands on every kind of position: the
first and last row of a 16-row sub-tile, of a 32-token tile, of a page and of
a partition, a sequence made of the new token alone, and an empty sequence.
"""
import numpy as np
import pytest
import torch

import decode_attention_int8_amd as q8
import oracle
import workloads
from cases import POISON_INT8, build
from gpu_cases import DEV, assert_cache_equal, say, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-4
TOL64 = 2e-5


def history(c, src_dtype=torch.float32):
    """Host and device caches with tokens 0 .. L-2 of each sequence, and the
    new rows [batch][n_kv][hd] (zeros for empty sequences)."""
    w = c.w
    host = oracle.Cache(c.num_blocks, w.n_kv, w.kv_bs, w.hd, fill_int8=POISON_INT8, fill_scale=np.nan)
    dev = q8.PagedKVCache(c.num_blocks, w.n_kv, w.kv_bs, w.hd, device=DEV)
    dev.k_pages.fill_(POISON_INT8)
    dev.v_pages.fill_(POISON_INT8)
    dev.k_scale.fill_(float("nan"))
    dev.v_scale.fill_(float("nan"))
    k_new = np.zeros((w.batch, w.n_kv, w.hd), np.float32)
    v_new = np.zeros_like(k_new)
    for b in range(w.batch):
        L = int(c.lens[b])
        if L <= 0:
            continue
        k, v = c.k_src[b], c.v_src[b]
        if src_dtype == torch.bfloat16:
            # the host side sees exactly the values the device widens
            k = torch.from_numpy(k).to(torch.bfloat16).float().numpy()
            v = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
        if L > 1:
            host.append(k[:L - 1], v[:L - 1], c.slots[b][:L - 1])
            dev.append(to_dev(k[:L - 1], src_dtype), to_dev(v[:L - 1], src_dtype), to_dev(c.slots[b][:L - 1]))
        k_new[b] = k[L - 1]
        v_new[b] = v[L - 1]
    return host, dev, k_new, v_new


def clone(dev):
    return q8.PagedKVCache.wrap(dev.k_pages.clone(), dev.v_pages.clone(), dev.k_scale.clone(), dev.v_scale.clone(),
                                hd=dev.hd)


def run_case(c, part_tokens=0, src_dtype=torch.float32, reps=1):
    host, dev, k_new, v_new = history(c, src_dtype)
    ref_dev = clone(dev)
    q, bt, sl = to_dev(c.q), to_dev(c.table), to_dev(c.lens)
    kn, vn = to_dev(k_new, src_dtype), to_dev(v_new, src_dtype)
    got = None
    for _ in range(reps):  # the step is idempotent: the same slot gets the same bytes
        got = q8.append_decode_attn(q, dev, kn, vn, bt, sl, c.scale, part_tokens=part_tokens)
        torch.cuda.synchronize()
    got = got.cpu().numpy()
    # the library's two-launch path on an identical copy of the history
    slots = oracle.new_token_slots(c.table, c.lens, c.w.kv_bs, c.num_blocks)
    ref_dev.append(kn, vn, to_dev(slots))
    two = q8.decode_attn(q, ref_dev, bt, sl, c.scale, part_tokens=part_tokens)
    torch.cuda.synchronize()
    two = two.cpu().numpy()
    want = oracle.append_decode(c.q, host, k_new, v_new, c.table, c.lens, c.scale, threads=8)
    want64 = oracle.decode(c.q, host, c.table, c.lens, c.scale, use_f64=True, threads=8)
    assert_cache_equal(host, dev)
    assert_cache_equal(host, ref_dev)
    assert np.array_equal(got.view(np.uint32), two.view(np.uint32)), "fused != append + decode"
    assert np.all(np.isfinite(got))
    err = float(np.abs(got - want).max())
    err64 = float(np.abs(got - want64).max())
    assert err <= TOL, f"max-abs error {err:.3g} > {TOL} (fp32 oracle)"
    assert err64 <= TOL64, f"max-abs error {err64:.3g} > {TOL64} (fp64 oracle)"
    for b in range(c.w.batch):
        if c.lens[b] <= 0:
            assert not got[b].any()
    return err


def edge_lens(batch, kv_bs, pt):
    """Lengths whose new token (position L-1) sits on sub-tile, tile, page and
    partition edges, plus L = 1 and L = 0."""
    cand = [1, 0, 16, 17, 32, 33, 31, kv_bs, kv_bs + 1, 2 * kv_bs, 129, 128]
    if pt:
        cand += [pt, pt + 1, 2 * pt, pt - 1]
    return [cand[i % len(cand)] + (i // len(cand)) * 64 for i in range(batch)]


@pytest.mark.parametrize("hd,G,kv_bs", [(64, 1, 16), (64, 8, 32), (128, 1, 16), (128, 4, 64),
                                        (128, 8, 16), (256, 2, 32), (256, 8, 128), (128, 5, 256),
                                        (128, 16, 16), (64, 10, 32),  # head groups: one of them stores the token
                                        (96, 8, 16), (160, 4, 32), (32, 2, 64)])  # padded pages
def test_append_decode_shapes(hd, G, kv_bs):
    batch = 14
    lens = edge_lens(batch, kv_bs, 0)
    w = workloads.Workload("fused", batch, 2 * G, 2, hd, kv_bs, max(lens), ragged=True, table="pool",
                           key=1000 + hd + G + kv_bs)
    c = build(w, lens=lens, with_cache=False)
    say(f"fused append+decode hd={hd} G={G} kv_bs={kv_bs} lens={lens}")
    run_case(c)


@pytest.mark.parametrize("pt", [32, 64, 96, 128])
def test_append_decode_split_and_merge(pt):
    """Split contexts: the new token falls in the last partition, whichever
    wave owns its tile; in-kernel merge (few partitions) and the combine
    kernel (many)."""
    lens = edge_lens(12, 16, pt)
    w = workloads.Workload("fusedsplit", 12, 8, 2, 128, 16, max(lens), ragged=True, table="pool",
                           key=1100 + pt)
    c = build(w, lens=lens, with_cache=False)
    say(f"fused split pt={pt} lens={lens}")
    run_case(c, part_tokens=pt, reps=2)


@pytest.mark.parametrize("hd", [128, 64, 256])
def test_append_decode_persistent_grid(hd):
    """More items than resident workgroups: the persistent grid's item order
    and its rolled tile loop, at every page width."""
    rng = np.random.default_rng(1200 + hd)
    lens = [int(x) for x in rng.integers(1, 700, size=64)]
    lens[:6] = [0, 1, 32, 33, 64, 65]
    w = workloads.Workload("fusedpersist", 64, 8, 2, hd, 16, 700, ragged=True, table="pool",
                           key=1200 + hd)
    c = build(w, lens=lens, with_cache=False)
    say(f"fused persistent tokens={sum(lens)}")
    run_case(c, part_tokens=32)


def test_append_decode_bf16_source():
    lens = edge_lens(8, 32, 0)
    w = workloads.Workload("fusedbf16", 8, 8, 2, 128, 32, max(lens), ragged=True, table="pool", key=1300)
    c = build(w, lens=lens, with_cache=False)
    run_case(c, src_dtype=torch.bfloat16)


def test_append_decode_steps_in_a_row():
    """Three decode steps: each call stores its token and the next step
    attends to it from memory."""
    w = workloads.Workload("fusedsteps", 4, 8, 2, 128, 16, 80, ragged=True, table="pool", key=1400)
    full = [50, 1, 31, 80]
    c = build(w, lens=full, with_cache=False)
    lens0 = [L - 3 for L in full]
    lens0[1] = 0
    host = oracle.Cache(c.num_blocks, w.n_kv, w.kv_bs, w.hd, fill_int8=POISON_INT8, fill_scale=np.nan)
    dev = q8.PagedKVCache(c.num_blocks, w.n_kv, w.kv_bs, w.hd, device=DEV)
    dev.k_pages.fill_(POISON_INT8)
    dev.v_pages.fill_(POISON_INT8)
    dev.k_scale.fill_(float("nan"))
    dev.v_scale.fill_(float("nan"))
    for b in range(4):
        if lens0[b] > 0:
            host.append(c.k_src[b][:lens0[b]], c.v_src[b][:lens0[b]], c.slots[b][:lens0[b]])
            dev.append(to_dev(c.k_src[b][:lens0[b]]), to_dev(c.v_src[b][:lens0[b]]), to_dev(c.slots[b][:lens0[b]]))
    q, bt = to_dev(c.q), to_dev(c.table)
    for step in range(3):
        lens = np.array([min(l0 + step + 1, f) if f > 0 else 0 for l0, f in zip(lens0, full)], np.int32)
        lens[1] = 1 if step == 0 else 0
        k_new = np.stack([c.k_src[b][max(lens[b] - 1, 0)] for b in range(4)])
        v_new = np.stack([c.v_src[b][max(lens[b] - 1, 0)] for b in range(4)])
        got = q8.append_decode_attn(q, dev, to_dev(k_new), to_dev(v_new), bt, to_dev(lens), c.scale)
        torch.cuda.synchronize()
        want = oracle.append_decode(c.q, host, k_new, v_new, c.table, lens, c.scale)
        assert_cache_equal(host, dev)
        assert float(np.abs(got.cpu().numpy() - want).max()) <= TOL


def test_append_decode_bad_entry_writes_nothing():
    """A new slot whose table entry lies outside the pool: NaN row for that
    sequence only, and the cache is left untouched."""
    lens = [40, 17, 33]
    w = workloads.Workload("fusedbad", 3, 4, 2, 128, 16, 40, ragged=True, table="pool", key=1500)
    c = build(w, lens=lens, with_cache=False)
    host, dev, k_new, v_new = history(c)
    c.table = c.table.copy()
    c.table[1, 1] = c.num_blocks + 5          # position 16 = the new token of sequence 1
    before = [t.clone() for t in (dev.k_pages, dev.v_pages, dev.k_scale, dev.v_scale)]
    slots = oracle.new_token_slots(c.table, c.lens, w.kv_bs, c.num_blocks)
    assert slots[1] == -1
    got = q8.append_decode_attn(to_dev(c.q), dev, to_dev(k_new), to_dev(v_new), to_dev(c.table),
                                to_dev(c.lens), c.scale).cpu().numpy()
    assert np.all(np.isnan(got[1]))
    assert np.all(np.isfinite(got[[0, 2]]))
    # only the other sequences' new rows changed
    host.append(k_new, v_new, slots)
    assert_cache_equal(host, dev)
    changed = [not torch.equal(a, b) for a, b in zip(before, (dev.k_pages, dev.v_pages, dev.k_scale, dev.v_scale))]
    assert all(changed)
