"""GPU parity at the five workloads' full sizes, in the launch configuration
the benchmark times (the default partition plan; static or persistent grid,
in-kernel merge or combine kernel as the shape decides), for the int8 codec
and the FP8 and q4_0 codecs, the fused append + decode and QUEST.

The whole workload is appended on the GPU and decoded in one call.  The
oracle then computes a sample of the outputs: a few sequences (the longest
and the shortest non-empty one, plus the first and last) and, of those, the
query heads of the first and the last kv head.  It runs on a host cache that
holds only the sampled rows of one kv head, addressed through the same block
table; the other sequences are given length 0 there.

At the same sizes the quantised cache and the integer scoring are checked
bit for bit on the sampled sequences: their device pages and scales (read
back through the page byte order the header defines) against the oracle's
quantisation of the same rows, and the decode kernel's int32 block dots
(q8kv_debug_block_dots, over each sampled sequence's whole length) against
the oracle's.

The fused step re-stores every sequence's newest token with its own values,
as the benchmark's fused leg does: the cache must come back unchanged and
the output must be the plain decode's, bit for bit.  QUEST runs as the
benchmark's leg does (top_k = ceil(max_blocks / 8)); on the sample its
metadata is compared bit for bit, its selection checked for validity against
fp64 bounds, and the decode over the selected blocks against the oracle.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import decode_attention_int8_amd as q8
import oracle
import workloads
from gpu_cases import DEV, natural_pages, say, to_dev
from oracle import fp8kv, q40, quest
from test_oracle_quest import quest_decode

pytestmark = pytest.mark.gpu

TOL = 2e-4    # GPU vs the fp32 oracle (int8 codec), or vs the fp64 definition (FP8, q4_0)
TOL64 = 2e-5  # int8 codec: GPU vs the oracle's fp64 twin

CODECS = {
    "q8": (q8.PagedKVCache, q8.decode_attn),
    "fp8": (q8.Fp8KVCache, q8.fp8_decode_attn),
    "q40": (q8.Q40KVCache, q8.q40_decode_attn),
}


def sample_seqs(lens):
    nz = [int(b) for b in np.flatnonzero(lens > 0)]
    pick = {nz[0], nz[-1], int(np.argmax(lens)), min(nz, key=lambda b: (int(lens[b]), b))}
    return sorted(pick)


_built = {}


def full_case(name):
    """Device caches of every codec holding the whole workload, the outputs
    of one decode call each, and the sampled sequences' source rows."""
    if name in _built:
        return _built[name]
    w = workloads.WORKLOADS[name]
    lens = workloads.seq_lens(w)
    table, nb = workloads.block_table(w, lens)
    seqs = sample_seqs(lens)
    caches = {}
    for codec, (cls, _) in CODECS.items():
        c = cls(nb, w.n_kv, w.kv_bs, w.hd, device=DEV)
        for t in (c.k_pages, c.v_pages, c.k_scale, c.v_scale):
            t.zero_()
        caches[codec] = c
    rows = {}
    k_last = np.zeros((w.batch, w.n_kv, w.hd), np.float32)
    v_last = np.zeros_like(k_last)
    say(f"full size {name}: {int(lens.sum())} tokens, sampled sequences {seqs}")
    with ThreadPoolExecutor(8) as ex:
        for c0 in range(0, w.batch, 8):
            bs = list(range(c0, min(c0 + 8, w.batch)))
            futs = {b: ex.submit(workloads.kv_rows, w, b, int(lens[b])) for b in bs}
            for b in bs:
                k, v = futs[b].result()
                if int(lens[b]) == 0:
                    continue
                k_last[b], v_last[b] = k[-1], v[-1]
                sm = workloads.slot_mapping(w, table, b, int(lens[b]))
                kd, vd, smd = to_dev(k), to_dev(v), to_dev(sm)
                for c in caches.values():
                    c.append(kd, vd, smd)
                if b in seqs:
                    rows[b] = (k, v, sm)
    q = workloads.query(w)
    scale = workloads.softmax_scale(w.hd)
    qd, td, ld = to_dev(q), to_dev(table), to_dev(lens)
    outs = {}
    # the sampled sequences' pages and scales, and the int32 block dots of a
    # decode over just those sequences (their table rows and lengths)
    c8 = caches["q8"]
    pages = {}
    for b in seqs:
        blocks = torch.from_numpy(table[b, :-(-int(lens[b]) // w.kv_bs)].astype(np.int64)).to(DEV)
        pages[b] = tuple(t.index_select(0, blocks).cpu().numpy() for t in (c8.k_pages, c8.v_pages, c8.k_scale, c8.v_scale))
    sub = np.array(seqs)
    max_tok = int(lens[sub].max())
    dots = q8.debug_block_dots(to_dev(q[sub]), c8, to_dev(table[sub]), to_dev(lens[sub]), max_tok).cpu().numpy()
    outs["bits"] = dict(pages=pages, dots=dots)
    for codec, (_, fn) in CODECS.items():
        outs[codec] = fn(qd, caches[codec], td, ld, scale).cpu().numpy()
    # the fused step, storing each sequence's newest token again
    c8 = caches["q8"]
    before = [t.clone() for t in (c8.k_pages, c8.v_pages, c8.k_scale, c8.v_scale)]
    outs["fused"] = q8.append_decode_attn(qd, c8, to_dev(k_last), to_dev(v_last), td, ld, scale).cpu().numpy()
    outs["fused_cache_same"] = all(torch.equal(a, b) for a, b in zip(before, (c8.k_pages, c8.v_pages, c8.k_scale, c8.v_scale)))
    del before
    # QUEST
    top_k = max(1, -(-w.max_blocks // 8))
    kmax, kmin = q8.quest_metadata(c8, td, ld)
    sel, sel_lens = q8.quest_select(qd, c8, kmax, kmin, td, ld, top_k)
    outs["quest"] = dict(kmax=kmax.cpu().numpy(), kmin=kmin.cpu().numpy(), sel=sel.cpu().numpy(),
                         sel_lens=sel_lens.cpu().numpy(), top_k=top_k,
                         out=q8.decode_attn_heads(qd, c8, sel, sel_lens, scale).cpu().numpy())
    torch.cuda.synchronize()
    del caches, c8, kmax, kmin, sel, sel_lens
    torch.cuda.empty_cache()
    _built.clear()  # keep one workload's state at a time
    _built[name] = (w, lens, table, nb, seqs, rows, q, scale, outs)
    return _built[name]


def sampled_reference(codec, w, lens, table, nb, seqs, rows, q, scale, kh):
    """Oracle outputs [batch][G][hd] of kv head kh for the sampled sequences."""
    G = w.n_q // w.n_kv
    host = {"q8": oracle.Cache, "fp8": fp8kv.Fp8Cache, "q40": q40.Q40Cache}[codec](nb, 1, w.kv_bs, w.hd)
    sl = np.zeros_like(lens)
    for b in seqs:
        k, v, sm = rows[b]
        host.append(k[:, kh:kh + 1], v[:, kh:kh + 1], sm)
        sl[b] = lens[b]
    qs = np.ascontiguousarray(q[:, kh * G:(kh + 1) * G])
    if codec == "q8":
        return (oracle.decode(qs, host, table, sl, scale, threads=8),
                oracle.decode(qs, host, table, sl, scale, use_f64=True, threads=8))
    ref = fp8kv.decode if codec == "fp8" else q40.decode
    return ref(qs, host, table, sl, scale), None


# one list ordered by workload, so each workload is built once
CHECKS = [(n, c) for n in workloads.ORDER for c in ["bits"] + list(CODECS) + ["fused", "quest"]]


@pytest.mark.parametrize("name,check", CHECKS)
def test_full_size(name, check):
    if check == "bits":
        full_size_bits(name)
    elif check == "fused":
        full_size_fused_append_decode(name)
    elif check == "quest":
        full_size_quest(name)
    else:
        full_size_sampled(name, check)


def full_size_sampled(name, codec):
    w, lens, table, nb, seqs, rows, q, scale, outs = full_case(name)
    got = outs[codec]
    G = w.n_q // w.n_kv
    assert np.all(np.isfinite(got))
    for kh in sorted({0, w.n_kv - 1}):
        say(f"  {name} {codec}: kv head {kh}, sequences {seqs}")
        want, want64 = sampled_reference(codec, w, lens, table, nb, seqs, rows, q, scale, kh)
        g = got[seqs][:, kh * G:(kh + 1) * G]
        err = float(np.abs(g - want[seqs]).max())
        assert err <= TOL, f"{name} {codec} kv head {kh}: max-abs error {err:.3g} > {TOL}"
        if want64 is not None:
            err64 = float(np.abs(g - want64[seqs]).max())
            assert err64 <= TOL64, f"{name} {codec} kv head {kh}: max-abs error {err64:.3g} vs fp64 > {TOL64}"
    # sequences of length 0 give zero rows
    for b in np.flatnonzero(lens == 0):
        assert not got[b].any()


def full_size_bits(name):
    """Pages, scales and int32 block dots of the sampled sequences, bit for
    bit.  The oracle quantises the sampled rows into a host pool of just
    their blocks (the same logical order, renumbered)."""
    w, lens, table, nb, seqs, rows, q, scale, outs = full_case(name)
    pages, dots = outs["bits"]["pages"], outs["bits"]["dots"]
    nblk = [-(-int(lens[b]) // w.kv_bs) for b in seqs]
    host = oracle.Cache(sum(nblk), w.n_kv, w.kv_bs, w.hd)
    sub_table = np.full((len(seqs), max(nblk)), -1, np.int32)
    first = 0
    for i, b in enumerate(seqs):
        sub_table[i, :nblk[i]] = np.arange(first, first + nblk[i], dtype=np.int32)
        k, v, _ = rows[b]
        t = np.arange(int(lens[b]))
        host.append(k, v, (sub_table[i, t // w.kv_bs] * w.kv_bs + t % w.kv_bs).astype(np.int32))
        first += nblk[i]
    first = 0
    for i, b in enumerate(seqs):
        say(f"  {name} bits: sequence {b}, {int(lens[b])} tokens")
        kp, vp, ks, vs = pages[b]
        sl = slice(first, first + nblk[i])
        assert np.array_equal(natural_pages(kp, "k"), host.k_pages[sl]), f"{name} seq {b}: K pages"
        assert np.array_equal(natural_pages(vp, "v"), host.v_pages[sl]), f"{name} seq {b}: V pages"
        assert np.array_equal(ks.view(np.uint32), host.k_scale[sl].view(np.uint32)), f"{name} seq {b}: K scales"
        assert np.array_equal(vs.view(np.uint32), host.v_scale[sl].view(np.uint32)), f"{name} seq {b}: V scales"
        first += nblk[i]
    sub = np.array(seqs)
    want = oracle.block_dots(q[sub], host, sub_table, lens[sub], dots.shape[2])
    assert np.array_equal(dots, want), f"{name}: int32 block dots differ"


def full_size_fused_append_decode(name):
    w, lens, table, nb, seqs, rows, q, scale, outs = full_case(name)
    say(f"  {name} fused append + decode")
    assert outs["fused_cache_same"], "re-storing the newest tokens changed the cache"
    assert np.array_equal(outs["fused"].view(np.uint32), outs["q8"].view(np.uint32))


def full_size_quest(name):
    w, lens, table, nb, seqs, rows, q, scale, outs = full_case(name)
    qs_ = outs["quest"]
    top_k, kmax, kmin, sel, sel_lens, got = (qs_[k] for k in ("top_k", "kmax", "kmin", "sel", "sel_lens", "out"))
    G = w.n_q // w.n_kv
    logical_len = np.minimum(-(-lens // w.kv_bs), top_k)
    assert np.array_equal(sel_lens, np.where(lens > 0, (logical_len - 1) * w.kv_bs + lens - (-(-lens // w.kv_bs) - 1) * w.kv_bs, 0))
    for kh in sorted({0, w.n_kv - 1}):
        say(f"  {name} quest: kv head {kh}, top_k {top_k}, sequences {seqs}")
        host = oracle.Cache(nb, 1, w.kv_bs, w.hd)
        sl = np.zeros_like(lens)
        for b in seqs:
            k, v, sm = rows[b]
            host.append(k[:, kh:kh + 1], v[:, kh:kh + 1], sm)
            sl[b] = lens[b]
        wmax, wmin = quest.metadata(host.k_pages, host.k_scale, table, sl, w.kv_bs)
        qs = np.ascontiguousarray(q[:, kh * G:(kh + 1) * G])
        U = quest.bounds(qs, wmax, wmin, table, sl, 1, w.kv_bs)
        for b in seqs:
            nblk = -(-int(lens[b]) // w.kv_bs)
            blocks = table[b, :nblk]
            assert np.array_equal(kmax[blocks, kh].view(np.uint32), wmax[blocks, 0].view(np.uint32))
            assert np.array_equal(kmin[blocks, kh].view(np.uint32), wmin[blocks, 0].view(np.uint32))
            logical = {int(p): j for j, p in enumerate(blocks)}
            row = sel[b, kh]
            kept = [logical[int(x)] for x in row if x >= 0]
            assert len(kept) == min(nblk, top_k) and np.all(row[len(kept):] == -1)
            assert kept == sorted(kept) and kept[-1] == nblk - 1
            if nblk > top_k > 1:
                chosen = set(kept[:-1])
                dropped = [j for j in range(nblk - 1) if j not in chosen]
                mag = max(np.abs(np.maximum(qs[b, g].astype(np.float64) * wmax[blocks[j], 0],
                                            qs[b, g].astype(np.float64) * wmin[blocks[j], 0])).sum()
                          for g in range(G) for j in range(nblk - 1))
                eps = mag * 2.0 ** -20
                assert min(U[b, 0, j] for j in chosen) >= max(U[b, 0, j] for j in dropped) - eps
        # decode over the GPU's own selection
        head_table = np.ascontiguousarray(sel[:, kh:kh + 1])
        want = quest_decode(qs, host, head_table, np.where(sl > 0, sel_lens, 0), scale)
        err = float(np.abs(got[seqs][:, kh * G:(kh + 1) * G] - want[seqs]).max())
        assert err <= TOL, f"{name} quest kv head {kh}: max-abs error {err:.3g} > {TOL}"
