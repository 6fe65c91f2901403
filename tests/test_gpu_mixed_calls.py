"""The library's per-stream state across mixed calls: the grow-only split
workspace, the persistent grid's work ticket, the in-kernel merge's arrival
counters and the QUEST bounds buffer must all be left ready for any next
call.  A sequence of calls of different shapes and entry points (static and
persistent grids, in-kernel and combine-kernel merges, a workspace that has
to grow, the fused step, both codecs, QUEST) is run once, checked against the
oracle, then run again in reverse order, on a second stream, on two streams
at once and after q8kv_release: every output must repeat bit for bit.
"""
import numpy as np
import pytest
import torch

import decode_attention_int8_amd as q8
import oracle
import workloads
from cases import build
from gpu_cases import DEV, gpu_cache, say, to_dev

pytestmark = pytest.mark.gpu


def case(key, batch, G, hd, kv_bs, seq_len, lens=None):
    w = workloads.Workload(f"mixed{key}", batch, 2 * G, 2, hd, kv_bs, seq_len, ragged=lens is None,
                           table="pool", key=key)
    return build(w, lens=lens)


def test_mixed_calls_repeat_bitwise():
    small = case(4100, 3, 4, 128, 16, 300)                        # static grid, in-kernel merges
    wide = case(4101, 64, 8, 128, 32, 1024)                       # persistent grid
    deep = case(4102, 2, 8, 64, 64, 9000, lens=[9000, 4500])      # combine kernel, large workspace
    caches = {id(c): gpu_cache(c) for c in (small, wide, deep)}

    def codec_cache(cls, c):
        cache = cls(c.num_blocks, c.w.n_kv, c.w.kv_bs, c.w.hd, device=DEV)
        for t in (cache.k_pages, cache.v_pages, cache.k_scale, cache.v_scale):
            t.zero_()
        for b in range(c.w.batch):
            if len(c.slots[b]):
                cache.append(to_dev(c.k_src[b]), to_dev(c.v_src[b]), to_dev(c.slots[b]))
        return cache

    fp8 = {id(c): codec_cache(q8.Fp8KVCache, c) for c in (small, deep)}
    q40 = {id(c): codec_cache(q8.Q40KVCache, c) for c in (small, deep)}

    def dev_in(c):
        return to_dev(c.q), to_dev(c.table), to_dev(c.lens)

    def plain(c, pt):
        q, bt, sl = dev_in(c)
        return q8.decode_attn(q, caches[id(c)], bt, sl, c.scale, part_tokens=pt)

    def codec(fn, store, c, pt):
        q, bt, sl = dev_in(c)
        return fn(q, store[id(c)], bt, sl, c.scale, part_tokens=pt)

    def quest(c):
        q, bt, sl = dev_in(c)
        cache = caches[id(c)]
        kmax, kmin = q8.quest_metadata(cache, bt, sl)
        sel, sel_lens = q8.quest_select(q, cache, kmax, kmin, bt, sl, 3)
        return q8.decode_attn_heads(q, cache, sel, sel_lens, c.scale)

    def fused(c):
        # store every sequence's newest token again with its own values
        q, bt, sl = dev_in(c)
        kn = np.zeros((c.w.batch, c.w.n_kv, c.w.hd), np.float32)
        vn = np.zeros_like(kn)
        for b in range(c.w.batch):
            if c.lens[b] > 0:
                kn[b], vn[b] = c.k_src[b][-1], c.v_src[b][-1]
        return q8.append_decode_attn(q, caches[id(c)], to_dev(kn), to_dev(vn), bt, sl, c.scale)

    calls = [
        ("small plain", lambda: plain(small, 0)),
        ("deep plain (combine)", lambda: plain(deep, 0)),
        ("wide plain (persistent)", lambda: plain(wide, 32)),
        ("small split 32", lambda: plain(small, 32)),
        ("deep split 64 (grows the workspace)", lambda: plain(deep, 64)),
        ("small fused", lambda: fused(small)),
        ("deep fp8 (combine)", lambda: codec(q8.fp8_decode_attn, fp8, deep, 0)),
        ("small q4_0 split 32", lambda: codec(q8.q40_decode_attn, q40, small, 32)),
        ("wide quest", lambda: quest(wide)),
        ("deep q4_0 split 64", lambda: codec(q8.q40_decode_attn, q40, deep, 64)),
        ("small fp8", lambda: codec(q8.fp8_decode_attn, fp8, small, 0)),
        ("deep quest", lambda: quest(deep)),
        ("wide plain again", lambda: plain(wide, 0)),
    ]
    first = {}
    for name, fn in calls:
        say(f"mixed: {name}")
        first[name] = fn().cpu().numpy()
    # the plain decodes against the oracle
    for name, c in (("small plain", small), ("deep plain (combine)", deep), ("wide plain (persistent)", wide)):
        want = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, threads=8)
        assert float(np.abs(first[name] - want).max()) <= 2e-4, name
    # the same calls in reverse order, then on a second stream
    for name, fn in reversed(calls):
        got = fn().cpu().numpy()
        assert np.array_equal(got.view(np.uint32), first[name].view(np.uint32)), name
    side = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(side):
        outs = {name: fn() for name, fn in calls}
    side.synchronize()
    for name in outs:
        assert np.array_equal(outs[name].cpu().numpy().view(np.uint32), first[name].view(np.uint32)), name
    # two streams at once, each with its own ticket, counters and workspace
    s1, s2 = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    torch.cuda.synchronize()
    conc = {}
    for _ in range(3):
        with torch.cuda.stream(s1):
            conc["wide plain (persistent)"] = plain(wide, 32)
            conc["deep plain (combine)"] = plain(deep, 0)
        with torch.cuda.stream(s2):
            conc["deep split 64 (grows the workspace)"] = plain(deep, 64)
            conc["small split 32"] = plain(small, 32)
        s1.synchronize()
        s2.synchronize()
        for name, t in conc.items():
            assert np.array_equal(t.cpu().numpy().view(np.uint32), first[name].view(np.uint32)), name
    q8.release()
    # and after the workspaces are released
    got = plain(deep, 64).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), first["deep split 64 (grows the workspace)"].view(np.uint32))
