"""The LDS-staged variant of the int8 decode kernels (q8kv_debug_set_stage).

With staging on, static grids at hd 64 and 128 load their tiles straight
into a per-wave LDS ring (two tiles in flight per wave) and read each tile
into registers only to compute it.  The arithmetic is the default kernels',
so every output must match them bit for bit: plain decode over the merge
paths (one partition, in-kernel merge, combine kernel), 4- and 8-wave
workgroups, lengths on tile and partition edges, and the fused append +
decode (output and cache).  Grids of more than two workgroups per CU run the
persistent kernel while staging is on; one case covers that switch.  Each
staged output is also checked against the oracle.
"""
import numpy as np
import pytest
import torch

import decode_attention_int8_amd as q8
import oracle
import workloads
from cases import build
from gpu_cases import DEV, decode, gpu_cache, say, to_dev

pytestmark = pytest.mark.gpu

TOL, TOL64 = 2e-4, 2e-5


def staged_and_default(fn):
    try:
        q8.debug_set_stage(True)
        a = fn()
        q8.debug_set_stage(False)
        b = fn()
    finally:
        q8.debug_set_stage(False)
    return a, b


def check_oracle(c, got, pt):
    want = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, part_tokens=0, threads=8)
    want64 = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, use_f64=True, threads=8)
    assert float(np.abs(got - want).max()) <= TOL
    assert float(np.abs(got - want64).max()) <= TOL64


CASES = [
    # (hd, G, kv_bs, lens, part_tokens, wide allowed)
    (128, 8, 16, [1, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 300], 0, True),
    (128, 8, 16, [1, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 300], 0, False),
    (128, 4, 64, [700, 1, 0, 257, 512, 96], 32, False),     # in-kernel merge
    (128, 8, 32, [40 * 32, 23 * 32 + 5], 32, False),       # combine kernel
    (64, 1, 16, [1, 0, 16, 17, 32, 33, 31, 129, 128, 65, 64], 0, True),
    (64, 8, 128, [1000, 513, 2], 64, False),
    (128, 16, 64, [2000, 77], 0, False),                   # two head groups per kv head
    (96, 8, 16, [1, 16, 17, 33, 129, 300], 0, True),       # padded pages
    (32, 4, 32, [700, 1, 0, 257], 32, False),
]


@pytest.mark.parametrize("hd,G,kv_bs,lens,pt,wide", CASES)
def test_staged_decode_bitwise(hd, G, kv_bs, lens, pt, wide):
    w = workloads.Workload("stage", len(lens), 2 * G, 2, hd, kv_bs, max(lens), ragged=True, table="pool",
                           spare_blocks=2, key=3000 + hd + G + kv_bs + pt)
    c = build(w, lens=lens)
    say(f"staged decode hd={hd} G={G} kv_bs={kv_bs} pt={pt} wide={wide} lens={lens}")
    dev = gpu_cache(c)
    try:
        q8.debug_set_wide(wide)
        got, ref = staged_and_default(lambda: decode(c, dev, part_tokens=pt))
    finally:
        q8.debug_set_wide(True)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    check_oracle(c, got, pt)


@pytest.mark.parametrize("hd,G,kv_bs", [(128, 8, 16), (64, 1, 16), (128, 4, 64)])
def test_staged_fused_append_bitwise(hd, G, kv_bs):
    lens = [1, 0, 16, 17, 32, 33, 31, kv_bs, kv_bs + 1, 2 * kv_bs, 129, 128, 65, 64]
    w = workloads.Workload("stagefused", len(lens), 2 * G, 2, hd, kv_bs, max(lens), ragged=True, table="pool",
                           key=3100 + hd + G + kv_bs)
    c = build(w, lens=lens)
    say(f"staged fused append hd={hd} G={G} kv_bs={kv_bs}")
    k_new = np.stack([c.k_src[b][-1] if c.lens[b] > 0 else np.zeros((w.n_kv, hd), np.float32)
                      for b in range(w.batch)])
    v_new = np.stack([c.v_src[b][-1] if c.lens[b] > 0 else np.zeros((w.n_kv, hd), np.float32)
                      for b in range(w.batch)])
    q, bt, sl = to_dev(c.q), to_dev(c.table), to_dev(c.lens)
    caches = []

    def step():
        dev = gpu_cache(c)  # every token already stored: the step re-stores the newest
        out = q8.append_decode_attn(q, dev, to_dev(k_new), to_dev(v_new), bt, sl, c.scale)
        torch.cuda.synchronize()
        caches.append(dev)
        return out.cpu().numpy()

    got, ref = staged_and_default(step)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    for f in ("k_pages", "v_pages", "k_scale", "v_scale"):
        a, b = getattr(caches[0], f), getattr(caches[1], f)
        assert torch.equal(a.view(torch.int8) if a.dtype == torch.float32 else a,
                           b.view(torch.int8) if b.dtype == torch.float32 else b), f
    check_oracle(c, got, 0)


def test_staged_switches_large_static_grids_to_persistent():
    """600 items (more than two per CU on a 256-CU device, fewer than the
    persistent grid's residency) run the persistent kernel when staging is
    on: same bits."""
    lens = [2048] * 75
    w = workloads.Workload("stagebig", 75, 8, 1, 128, 64, 2048, ragged=False, table="perm", key=3200)
    c = build(w, lens=lens)
    say("staged switch to the persistent grid (75 x 8 partitions)")
    dev = gpu_cache(c)
    got, ref = staged_and_default(lambda: decode(c, dev, part_tokens=256))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    check_oracle(c, got, 256)
