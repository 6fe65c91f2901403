"""GPU: q8kv_decode_attn_noalloc, the allocation-free decode entry, called
through the C ABI with raw pointers, gives q8kv_decode_attn_split's output
bit for bit on two calls in a row, the second with a smaller input (so the
scratch array holds the first call's states and counters when the second
starts).  The pairs cover the in-kernel merge of partition states, the
combine kernel (more than 64 states per group), the persistent grid (more
work items than resident workgroups, which takes work from the scratch's
ticket) with either merge, head groups above 8 query heads, and an unsplit
call.  The first call of each pair is also checked against the oracle.
"""
import numpy as np
import pytest
import torch

import decode_attention_int8_amd as q8
import oracle
import workloads
from cases import build
from gpu_cases import DEV, dev_inputs, gpu_cache, say

pytestmark = pytest.mark.gpu

TOL, TOL64 = 2e-4, 2e-5


def case(name, batch, G, n_kv, hd, kv_bs, lens, key):
    w = workloads.Workload(name, batch, G * n_kv, n_kv, hd, kv_bs, max(lens), ragged=True, table="pool",
                           spare_blocks=2, key=key)
    return build(w, lens=lens)


def call_noalloc(c, dev, pt):
    q, bt, sl = dev_inputs(c)
    out = torch.full_like(q, float("nan"))
    w = c.w
    rc = q8.lib.q8kv_decode_attn_noalloc(out.data_ptr(), q.data_ptr(), dev.k_pages.data_ptr(),
                                         dev.v_pages.data_ptr(), dev.k_scale.data_ptr(), dev.v_scale.data_ptr(),
                                         bt.data_ptr(), sl.data_ptr(), bt.shape[1], dev.num_blocks, w.batch,
                                         w.n_q, w.n_kv, w.hd, w.kv_bs, c.scale, pt,
                                         torch.cuda.current_stream(DEV).cuda_stream)
    assert rc == q8.Q8KV_OK, q8.last_error()
    torch.cuda.synchronize()
    return out.cpu().numpy()


def call_split(c, dev, pt):
    q, bt, sl = dev_inputs(c)
    out = q8.decode_attn(q, dev, bt, sl, c.scale, part_tokens=pt)
    torch.cuda.synchronize()
    return out.cpu().numpy()


rng = np.random.default_rng(4242)
PAIRS = {
    # in-kernel merge (np * G <= 64), then a smaller batch
    "fused_merge": ((6, 8, 2, 128, 64, [400, 333, 64, 0, 129, 257], 64),
                    (3, 8, 2, 128, 64, [170, 5, 96], 64)),
    # combine kernel: 256 partitions of 32 tokens, then fewer and shorter
    "combine": ((2, 8, 2, 128, 32, [256 * 32, 5000], 32),
                (1, 8, 2, 128, 32, [3000], 32)),
    # persistent grid: 64 sequences x 2 kv heads x up to 32 partitions
    "persistent": ((64, 4, 2, 128, 32, [int(x) for x in rng.integers(1, 1025, size=64)], 32),
                   (40, 4, 2, 128, 32, [int(x) for x in rng.integers(1, 700, size=40)], 32)),
    # persistent grid with the in-kernel merge: 128 x 4 x 8 items, 64 states
    # per group, arrival counters in the scratch
    "persistent_merge": ((128, 8, 4, 128, 64, [int(x) for x in rng.integers(1, 1025, size=128)], 128),
                         (50, 8, 4, 128, 64, [int(x) for x in rng.integers(1, 1025, size=50)], 128)),
    # 16 query heads per kv head (two head groups), automatic plan
    "head_groups": ((4, 16, 2, 128, 64, [4000, 100, 2500, 1], 0),
                    (2, 16, 2, 128, 64, [900, 64], 0)),
    # hd 64 and 256, then an unsplit call (one partition)
    "hd_mix": ((3, 4, 2, 256, 64, [1500, 700, 64], 64),
               (2, 2, 3, 64, 16, [40, 17], 64)),
    # padded pages (hd 160 and 96), in-kernel merge then combine kernel
    "hd_pad": ((3, 8, 2, 160, 32, [900, 300, 33], 64),
               (2, 4, 2, 96, 16, [3000, 17], 32)),
}


@pytest.mark.parametrize("name", list(PAIRS))
def test_noalloc_matches_split_twice(name):
    for i, (batch, G, n_kv, hd, kv_bs, lens, pt) in enumerate(PAIRS[name]):
        say(f"no-alloc {name} call {i + 1}: batch {batch} G {G} n_kv {n_kv} hd {hd} kv_bs {kv_bs} "
            f"part_tokens {pt} tokens {sum(lens)}")
        c = case(f"na_{name}_{i}", batch, G, n_kv, hd, kv_bs, lens, 7000 + 10 * i + len(name))
        dev = gpu_cache(c)
        got = call_noalloc(c, dev, pt)
        want = call_split(c, dev, pt)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{name} call {i + 1}"
        if i == 0:
            ref = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, threads=8)
            ref64 = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, use_f64=True, threads=8)
            assert float(np.abs(got - ref).max()) <= TOL
            assert float(np.abs(got - ref64).max()) <= TOL64


def test_noalloc_repeated_calls_stay_exact():
    """Ten calls in a row on the persistent shape: the counters the scratch
    keeps between calls never leak into a result."""
    batch, G, n_kv, hd, kv_bs, lens, pt = PAIRS["persistent"][0]
    c = case("na_repeat", batch, G, n_kv, hd, kv_bs, lens, 7777)
    dev = gpu_cache(c)
    want = call_split(c, dev, pt)
    for k in range(10):
        got = call_noalloc(c, dev, pt)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"call {k + 1}"


def test_noalloc_binding():
    batch, G, n_kv, hd, kv_bs, lens, pt = PAIRS["fused_merge"][0]
    c = case("na_bind", batch, G, n_kv, hd, kv_bs, lens, 7100)
    dev = gpu_cache(c)
    q, bt, sl = dev_inputs(c)
    out = torch.empty_like(q)
    q8.decode_attn_noalloc(q, dev, bt, sl, c.scale, out, part_tokens=pt)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), call_split(c, dev, pt).view(np.uint32))
