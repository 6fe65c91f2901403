"""CPU checks of the benchmark's contract and its byte accounting.

* bench.py refuses more than one GPU with exit status 2 and a message, before
  it touches the GPU;
* the algorithmic bytes behind roofline.achieved: per (token, kv head) 2 hd
  code bytes and two fp32 scales for the int8 codec, plus q and out (fp32),
  the used block-table entries and seq_lens -- checked against the figures
  written out by hand for the fixed-length workloads (tiny: 512 tokens x 1
  kv head x 264 B = 135,168 B of KV, + 2 x 512 B of q / out + 32 x 4 B of
  table + 4 B of lengths = 136,324 B; and the 7B-like, GQA-batch and 128K
  workloads likewise), and the FP8 / q4_0 codecs' per-row byte counts;
* the CPU-baseline leg returns the reported fields on a short sample.
"""
import os
import subprocess
import sys

import numpy as np
import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "4"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name,kv,total", [
    ("tiny", 135_168, 136_324),
    ("mha7b", 34_603_008, 34_636_804),
    ("gqa_batch", 276_824_064, 277_381_184),
    ("long_gqa", 138_412_032, 138_452_996),
])
def test_algorithmic_bytes(name, kv, total):
    w = workloads.WORKLOADS[name]
    lens = workloads.seq_lens(w)
    assert workloads.kv_bytes(w, lens) == kv
    assert workloads.step_bytes(w, lens) == total


def test_codec_bytes_per_row():
    w = workloads.WORKLOADS["mha7b"]
    lens = np.array([1])
    per = w.n_kv
    # FP8: 2 x 128 E4M3 codes + one scale byte per 64 elements of K and of V
    assert workloads.fp8_kv_bytes(w, lens) == per * (256 + 4)
    # q4_0: 2 x 64 bytes of 4-bit codes + one fp16 scale per 32 elements of K and of V
    assert workloads.q40_kv_bytes(w, lens) == per * (128 + 16)
    base = workloads.step_bytes(w, lens) - workloads.kv_bytes(w, lens)
    assert workloads.step_bytes(w, lens, codec="fp8") == base + workloads.fp8_kv_bytes(w, lens)
    assert workloads.step_bytes(w, lens, codec="q40") == base + workloads.q40_kv_bytes(w, lens)


def test_cpu_baseline_leg_fields():
    sys.path.insert(0, ROOT)
    import bench
    import oracle
    w = workloads.WORKLOADS["tiny"]
    lens = workloads.seq_lens(w)
    table, nb = workloads.block_table(w, lens)
    g = dict(lens=lens, table=table, nb=nb)
    host = oracle.Cache(nb, w.n_kv, w.kv_bs, w.hd)
    for b in range(w.batch):
        k, v = workloads.kv_rows(w, b, int(lens[b]))
        host.append(k, v, workloads.slot_mapping(w, table, b, int(lens[b])))
    q = workloads.query(w)
    scale = workloads.softmax_scale(w.hd)

    def out_fn(sl):  # the oracle stands in for the GPU here
        return oracle.decode(q, host, table, sl, scale)

    cpu, parity = bench.cpu_baseline(w, g, out_fn, 0.2)
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s" and cpu["value"] > 0
    assert cpu["cores"] >= 1 and cpu["sample_seconds"] >= 0.2 and "whole step" in cpu["sample"]
    assert parity["ok"] and parity["max_abs_err_vs_oracle"] == 0.0 and parity["ok_f64"]
    # the single-threaded pass, bitwise equal to the OpenMP one, and the host
    st = cpu["single_thread"]
    assert st["cores"] == 1 and st["value"] > 0 and st["bitwise_equal_to_parallel"]
    assert cpu["host_nproc"] >= 1 and isinstance(cpu["cpu_model"], str)


def test_bench_defaults_name_the_gated_workloads():
    """The headline is the ragged batch (the largest workload) and the 128K
    step is timed in the same run."""
    sys.path.insert(0, ROOT)
    import bench
    old = sys.argv
    sys.argv = ["bench.py"]
    try:
        args = bench.parse()
    finally:
        sys.argv = old
    assert args.workload == "ragged" and "long_gqa" in args.also.split(",")


def test_timeline_edits_apply_to_the_kernel_source():
    """bench.py --timeline stamps a copy of the kernel source at fixed
    points; each must still occur exactly once."""
    sys.path.insert(0, ROOT)
    import bench
    src = open(os.path.join(ROOT, "decode_attention_int8_amd", "csrc", "q8kv.hip")).read()
    out = bench.timeline_source(src)
    assert out.count("STAMP(") == 4 and "q8kv_timeline_read" in out


def test_item_timeline_edits_apply_to_the_kernel_source():
    """bench.py --item-timeline stamps a copy of the kernel source at fixed
    points; each must still occur exactly once."""
    sys.path.insert(0, ROOT)
    import bench
    src = open(os.path.join(ROOT, "decode_attention_int8_amd", "csrc", "q8kv.hip")).read()
    out = bench.items_source(src)
    assert out.count("ISTAMP(") == 6 and "q8kv_items_read" in out
