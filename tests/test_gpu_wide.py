"""The decode kernel in its two workgroup sizes.  A static grid of at most
one workgroup per CU at hd 64 and 128 runs 8-wave workgroups; other grids
run 4-wave ones.  Each small case here fits such a grid, so it is decoded
once with the 8-wave kernel and once, after q8kv_debug_set_wide(0), with the
4-wave kernel, for every codec, the fused append + decode, and the three
merge paths (one partition, in-kernel merge, combine kernel).  Both outputs
are checked against the oracle of their codec.
"""
import numpy as np
import pytest

import decode_attention_int8_amd as q8
import oracle
from oracle import fp8kv, q40
from cases import build
from gpu_cases import DEV, gpu_cache, say, to_dev
import workloads

pytestmark = pytest.mark.gpu

TOL = 2e-4


def case(key, batch, G, hd, kv_bs, seq_len, lens=None):
    w = workloads.Workload(f"wide{key}", batch, 2 * G, 2, hd, kv_bs, seq_len, ragged=lens is None,
                           table="pool", key=key)
    return build(w, lens=lens)


def codec_cache(cls, c):
    cache = cls(c.num_blocks, c.w.n_kv, c.w.kv_bs, c.w.hd, device=DEV)
    for t in (cache.k_pages, cache.v_pages, cache.k_scale, cache.v_scale):
        t.zero_()
    for b in range(c.w.batch):
        if len(c.slots[b]):
            cache.append(to_dev(c.k_src[b]), to_dev(c.v_src[b]), to_dev(c.slots[b]))
    return cache


def both(fn):
    """fn() with 8-wave workgroups allowed, then forbidden."""
    try:
        q8.debug_set_wide(True)
        wide = fn().cpu().numpy()
        q8.debug_set_wide(False)
        narrow = fn().cpu().numpy()
    finally:
        q8.debug_set_wide(True)
    return wide, narrow


# (part_tokens, what it exercises)
SPLITS = [(0, "default plan"), (32, "in-kernel merge"), (None, "combine kernel")]


@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("pt,label", SPLITS)
def test_wide_and_narrow_match(hd, pt, label):
    if pt is None:
        # 2 x 4 heads x 40 partitions of 32 tokens: more states than the
        # in-kernel merge takes
        c = case(4200 + hd, 2, 4, hd, 32, 1280, lens=[1280, 700])
        pt = 32
    else:
        c = case(4210 + hd + pt, 3, 4, hd, 16, 300)
    say(f"wide vs narrow: hd {hd}, {label}, lens {list(c.lens)}")
    q, bt, sl = to_dev(c.q), to_dev(c.table), to_dev(c.lens)
    cache = gpu_cache(c)
    want = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, threads=8)
    wide, narrow = both(lambda: q8.decode_attn(q, cache, bt, sl, c.scale, part_tokens=pt))
    for name, got in (("wide", wide), ("narrow", narrow)):
        err = float(np.abs(got - want).max())
        assert err <= TOL, f"{name}: max-abs error {err:.3g} vs the oracle"
    # the fused step, re-storing each sequence's newest token
    kn = np.zeros((c.w.batch, c.w.n_kv, hd), np.float32)
    vn = np.zeros_like(kn)
    for b in range(c.w.batch):
        if c.lens[b] > 0:
            kn[b], vn[b] = c.k_src[b][-1], c.v_src[b][-1]
    fw, fn_ = both(lambda: q8.append_decode_attn(q, cache, to_dev(kn), to_dev(vn), bt, sl, c.scale,
                                                 part_tokens=pt))
    assert np.array_equal(fw.view(np.uint32), wide.view(np.uint32))
    assert np.array_equal(fn_.view(np.uint32), narrow.view(np.uint32))
    # the FP8 and q4_0 codecs against their fp64 oracles
    for cls, fn, host_cls, ref in ((q8.Fp8KVCache, q8.fp8_decode_attn, fp8kv.Fp8Cache, fp8kv.decode),
                                   (q8.Q40KVCache, q8.q40_decode_attn, q40.Q40Cache, q40.decode)):
        cc = codec_cache(cls, c)
        host = host_cls(c.num_blocks, c.w.n_kv, c.w.kv_bs, hd)
        for b in range(c.w.batch):
            if len(c.slots[b]):
                host.append(c.k_src[b], c.v_src[b], c.slots[b])
        want_c = ref(c.q, host, c.table, c.lens, c.scale)
        for name, got in zip(("wide", "narrow"), both(lambda: fn(q, cc, bt, sl, c.scale, part_tokens=pt))):
            err = float(np.abs(got - want_c).max())
            assert err <= TOL, f"{cls.__name__} {name}: max-abs error {err:.3g} vs the oracle"
    for b in np.flatnonzero(c.lens == 0):
        assert not wide[b].any() and not narrow[b].any()
