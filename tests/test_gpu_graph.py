"""GPU: q8kv_decode_attn_noalloc captured in a HIP graph (through
torch.cuda.graph) and replayed.  The entry allocates nothing and clears its
scratch counters with a kernel rather than a memset node, so it can be
captured once library state is set up (one eager call on the device).
Every replay, with eager decode calls and synchronisations between the
replays, must give the eager call's output bit for bit: on the in-kernel
merge, the combine kernel and the persistent grid."""
import numpy as np
import pytest
import torch

import decode_attention_int8_amd as q8
import workloads
from cases import build
from gpu_cases import DEV, dev_inputs, gpu_cache, say

pytestmark = pytest.mark.gpu

rng = np.random.default_rng(5150)
CASES = {
    # (batch, G, n_kv, hd, kv_bs, lens, part_tokens)
    "in_kernel_merge": (6, 8, 2, 128, 64, [400, 333, 64, 0, 129, 257], 64),
    "combine": (2, 8, 2, 128, 32, [256 * 32, 5000], 32),
    "persistent": (64, 4, 2, 128, 32, [int(x) for x in rng.integers(1, 1025, size=64)], 32),
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_decode_replays_from_a_graph(name):
    batch, G, n_kv, hd, kv_bs, lens, pt = CASES[name]
    w = workloads.Workload("graph_" + name, batch, G * n_kv, n_kv, hd, kv_bs, max(lens), ragged=True, table="pool",
                           key=5150 + len(name))
    c = build(w, lens=lens, with_cache=False)
    say(f"graph replay {name}: batch {batch} G {G} part_tokens {pt}")
    dev = gpu_cache(c)
    q, bt, sl = dev_inputs(c)
    want = torch.empty_like(q)
    q8.decode_attn_noalloc(q, dev, bt, sl, c.scale, want, part_tokens=pt)  # sets up the library's state
    torch.cuda.synchronize()
    out = torch.full_like(q, float("nan"))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q8.decode_attn_noalloc(q, dev, bt, sl, c.scale, out, part_tokens=pt)
    torch.cuda.synchronize()
    ref = want.cpu().numpy()
    for k in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"replay {k + 1}"
        # eager work between replays (the workspace path, not the scratch)
        eager = q8.decode_attn(q, dev, bt, sl, c.scale, part_tokens=pt)
        torch.cuda.synchronize()
        assert np.array_equal(eager.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    del g
