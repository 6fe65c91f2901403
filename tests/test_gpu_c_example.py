"""GPU: the plain C caller (decode_attention_int8_amd/csrc/q8kv_example.c)
builds a cache with q8kv_append and decodes with q8kv_decode_attn through the
C ABI alone, in a process of its own with no Python or torch.  Its output
is checked against the oracle on the same seeded inputs (2e-4 against the
fp32 oracle, 2e-5 against its fp64 twin), at hd 128 and at a padded head
size."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import workloads
from cases import build
from gpu_cases import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXAMPLE = os.path.join(ROOT, "decode_attention_int8_amd", "q8kv_example")
TOL, TOL64 = 2e-4, 2e-5


def write_inputs(path, c):
    w = c.w
    n_tokens = sum(len(s) for s in c.slots)
    hdr = np.array([w.batch, w.n_q, w.n_kv, w.hd, w.kv_bs, c.num_blocks, c.table.shape[1], n_tokens], np.int32)
    k = np.concatenate([k for k in c.k_src if len(k)]).astype(np.float32)
    v = np.concatenate([v for v in c.v_src if len(v)]).astype(np.float32)
    slots = np.concatenate([s for s in c.slots if len(s)]).astype(np.int32)
    with open(path, "wb") as f:
        for a in (hdr, np.array([c.scale], np.float32), c.q.astype(np.float32), c.table.astype(np.int32),
                  c.lens.astype(np.int32), k, v, slots):
            f.write(np.ascontiguousarray(a).tobytes())


@pytest.mark.parametrize("hd,G,kv_bs", [(128, 8, 16), (96, 4, 64)])
def test_c_caller_matches_the_oracle(hd, G, kv_bs):
    if not os.path.exists(EXAMPLE):
        pytest.fail("q8kv_example is not built (decode_attention_int8_amd/build.py)")
    lens = [300, 1, 0, 129, 2 * kv_bs + 3]
    w = workloads.Workload("cexample", len(lens), 2 * G, 2, hd, kv_bs, max(lens), ragged=True, table="pool",
                           key=3600 + hd)
    c = build(w, lens=lens, poison=False)
    say(f"C caller hd={hd} G={G} kv_bs={kv_bs}")
    with tempfile.TemporaryDirectory() as d:
        inp, outp = os.path.join(d, "in.bin"), os.path.join(d, "out.bin")
        write_inputs(inp, c)
        r = subprocess.run([EXAMPLE, inp, outp], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        got = np.fromfile(outp, np.float32).reshape(c.q.shape)
    want = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, threads=8)
    want64 = oracle.decode(c.q, c.cache, c.table, c.lens, c.scale, use_f64=True, threads=8)
    assert float(np.abs(got - want).max()) <= TOL
    assert float(np.abs(got - want64).max()) <= TOL64
    assert not got[2].any()  # the empty sequence
