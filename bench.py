#!/usr/bin/env python3
"""Benchmark: q8-KV single-query decode attention on one MI355X.

One step = one q8kv_decode_attn call over one batch of the workload (Q
quantise, page walk, int8 scoring, online softmax, P.V, split combine); the
KV cache is appended (quantised) beforehand and is resident in HBM when the
timed region starts.  Cold-cache timing: the step rotates over R copies of
the page pool so that R copies span >= 1 GB (four times the MI355X's 256 MB
last-level cache), so each step reads its KV from HBM.

Prints ONE JSON line: value = KV GB/s (int8 K and V rows plus their fp32
scales, per step, divided by the step time), plus us/step, the roofline of
the decode launch (algorithmic bytes / mean launch time, from HIP events on
the launch stream around the timed launches, against 8 TB/s; traffic = HBM
bytes per launch from the committed counter summary when it matches the
kernel source), the per-call distribution (events around each call of a
second pass: median, min, p90), a plain linear read of the same K+V pools in
one launch (the streaming ceiling the decode is compared with), the CPU
oracle timed on a bounded sample of the same workload, and sampled parity
against that oracle and its fp64 twin.  A last leg times the fused step
that also stores each sequence's new token (q8kv_append_decode_attn) against
the same work as two launches (q8kv_append, then q8kv_decode_attn), and
others the same step over the FP8 codec (q8kv_fp8_decode_attn) and the
q4_0 codec (q8kv_q40_decode_attn), each with a sampled parity check against
its oracle, and a QUEST leg (block metadata, top-k block selection, decode
over the kept blocks).
"""
import argparse
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "q8-KV decode attention µs/step + KV GB/s (% of HBM peak), 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    # a short step needs ~1000 untimed steps (~15 ms) before the clocks settle;
    # 100 steps after 10 read ~3% slow on the 7B-like workload
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=1000)
    p.add_argument("--workload", default="mha7b", choices=workloads.ORDER)
    p.add_argument("--cold-bytes", type=float, default=1.0e9,
                   help="bytes the rotated cache copies must span (0: warm, one copy)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline and parity sample")
    p.add_argument("--no-fused", action="store_true", help="skip the fused append + decode leg")
    p.add_argument("--no-fp8", action="store_true", help="skip the FP8-codec leg")
    p.add_argument("--no-q40", action="store_true", help="skip the q4_0-codec leg")
    p.add_argument("--no-quest", action="store_true", help="skip the QUEST metadata / selection leg")
    p.add_argument("--part-tokens", type=int, default=0, help="override the split plan (0: automatic)")
    p.add_argument("--copy-mb", type=float, default=0.0,
                   help="after timing, run one device-to-device copy of this many MiB (a known-size "
                        "kernel that scales hardware byte counters)")
    return p.parse_args()


CODECS = ("fp8", "q40")


def codec_api(name):
    """(cache class, decode call, algorithmic KV bytes) of a KV codec."""
    import decode_attention_int8_amd as q8
    return {"fp8": (q8.Fp8KVCache, q8.fp8_decode_attn, workloads.fp8_kv_bytes),
            "q40": (q8.Q40KVCache, q8.q40_decode_attn, workloads.q40_kv_bytes)}[name]


def cold_copies(cache, wrap, kv_bytes, copies_bytes, dev):
    """The cache plus clones, so that the copies span copies_bytes of
    algorithmic KV (bounded by 80% of free memory and 256 copies)."""
    import torch
    R = 1 if copies_bytes <= 0 else max(1, math.ceil(copies_bytes / kv_bytes))
    free, _ = torch.cuda.mem_get_info(dev)
    pool_bytes = sum(t.numel() * t.element_size() for t in (cache.k_pages, cache.v_pages, cache.k_scale, cache.v_scale))
    R = max(1, min(R, int(0.8 * free // max(pool_bytes, 1)) + 1, 256))
    return [cache] + [wrap(cache.k_pages.clone(), cache.v_pages.clone(), cache.k_scale.clone(), cache.v_scale.clone())
                      for _ in range(R - 1)]


def build_gpu(w, dev, copies_bytes, codecs=CODECS):
    import torch
    import decode_attention_int8_amd as q8
    lens = workloads.seq_lens(w)
    table, nb = workloads.block_table(w, lens)
    cache = q8.PagedKVCache(nb, w.n_kv, w.kv_bs, w.hd, device=dev)
    others = {}
    for name in codecs:
        others[name] = codec_api(name)[0](nb, w.n_kv, w.kv_bs, w.hd, device=dev)
    for c in [cache] + list(others.values()):
        for t in (c.k_pages, c.v_pages, c.k_scale, c.v_scale):
            t.zero_()
    t0 = time.time()
    # each sequence's newest rows, which the fused-append leg stores again
    k_last = np.zeros((w.batch, w.n_kv, w.hd), np.float32)
    v_last = np.zeros_like(k_last)
    with ThreadPoolExecutor(8) as ex:
        chunk = 8
        for c0 in range(0, w.batch, chunk):
            bs = list(range(c0, min(c0 + chunk, w.batch)))
            futs = {b: ex.submit(workloads.kv_rows, w, b, int(lens[b])) for b in bs}
            for b in bs:
                k, v = futs[b].result()
                if int(lens[b]) > 0:
                    k_last[b], v_last[b] = k[-1], v[-1]
                sm = workloads.slot_mapping(w, table, b, int(lens[b]))
                kd, vd, smd = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev), torch.from_numpy(sm).to(dev)
                cache.append(kd, vd, smd)
                for c in others.values():
                    c.append(kd, vd, smd)
    torch.cuda.synchronize()
    log(f"appended {int(lens.sum())} tokens x {w.n_kv} kv heads in {time.time() - t0:.1f}s")
    caches = cold_copies(cache, q8.PagedKVCache.wrap, workloads.kv_bytes(w, lens), copies_bytes, dev)
    codec_caches = {name: cold_copies(c, codec_api(name)[0].wrap, codec_api(name)[2](w, lens), copies_bytes, dev)
                    for name, c in others.items()}
    q = torch.from_numpy(workloads.query(w)).to(dev)
    return dict(lens=lens, table=table, nb=nb, caches=caches, codec=codec_caches, q=q, k_last=k_last, v_last=v_last,
                table_d=torch.from_numpy(table).to(dev), lens_d=torch.from_numpy(lens).to(dev))


def time_gpu(w, g, steps, warmup, part_tokens):
    import torch
    import decode_attention_int8_amd as q8
    scale = workloads.softmax_scale(w.hd)
    R = len(g["caches"])
    out = torch.empty_like(g["q"])

    def step(i):
        q8.decode_attn(g["q"], g["caches"][i % R], g["table_d"], g["lens_d"], scale, out=out,
                       part_tokens=part_tokens)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # HIP events on the launch stream bracket the K back-to-back launches of
    # the timed region; their mean is the per-launch (= per-step) duration
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    loop_ms = e0.elapsed_time(e1) / steps
    # the per-call distribution: events around every call of a second pass
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    calls = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    per_call = {"median": round(float(np.median(calls)), 3), "min": round(float(calls.min()), 3),
                "p90": round(float(np.percentile(calls, 90)), 3)}
    return loop_ms, per_call, out


def time_append_decode(w, g, steps, warmup, part_tokens):
    """The fused step (q8kv_append_decode_attn: store each sequence's new
    token at position L-1, then attend over 0..L-1) against the same work as
    two launches (q8kv_append at those slots, then q8kv_decode_attn), both
    rotated over the cold copies.  The new rows are the rows each sequence's
    newest token already holds, so the cache bytes do not change.  Returns a
    dict of per-step times in us."""
    import torch
    import decode_attention_int8_amd as q8
    scale = workloads.softmax_scale(w.hd)
    R = len(g["caches"])
    dev = g["q"].device
    k_new = torch.from_numpy(g["k_last"]).to(dev)
    v_new = torch.from_numpy(g["v_last"]).to(dev)
    lens, table = g["lens"], g["table"]
    slots = np.array([int(table[b, (L - 1) // w.kv_bs]) * w.kv_bs + (L - 1) % w.kv_bs if L > 0 else -1
                      for b, L in enumerate(lens.tolist())], np.int32)
    slots_d = torch.from_numpy(slots).to(dev)
    out = torch.empty_like(g["q"])
    stream = torch.cuda.current_stream()

    def fused(i):
        q8.append_decode_attn(g["q"], g["caches"][i % R], k_new, v_new, g["table_d"], g["lens_d"], scale,
                              out=out, part_tokens=part_tokens)

    def append(i):
        g["caches"][i % R].append(k_new, v_new, slots_d)

    def two(i):
        append(i)
        q8.decode_attn(g["q"], g["caches"][i % R], g["table_d"], g["lens_d"], scale, out=out,
                       part_tokens=part_tokens)

    def timed(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    res = {"fused_us": timed(fused), "two_launch_us": timed(two), "append_us": timed(append)}
    return {k: round(v, 3) for k, v in res.items()}


def time_codec(w, g, name, steps, warmup, part_tokens):
    """The same decode step over another KV codec (FP8 or q4_0), rotated over
    its own cold copies.  Returns us per step."""
    import torch
    decode = codec_api(name)[1]
    scale = workloads.softmax_scale(w.hd)
    caches = g["codec"][name]
    R = len(caches)
    out = torch.empty_like(g["q"])

    def step(i):
        decode(g["q"], caches[i % R], g["table_d"], g["lens_d"], scale, out=out, part_tokens=part_tokens)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def codec_parity(w, g, name, max_seqs=2, max_tokens=16384):
    """Max-abs difference of a codec's decode against its oracle (fp64
    definition) on a bounded sample of the workload's sequences: the sampled
    sequences' rows are re-quantised on the host by the oracle."""
    import torch
    from oracle import fp8kv, q40
    host_cls, ref = {"fp8": (fp8kv.Fp8Cache, fp8kv.decode), "q40": (q40.Q40Cache, q40.decode)}[name]
    lens = g["lens"]
    seqs, tot = [], 0
    sample_lens = np.zeros_like(lens)
    for b in np.argsort(lens, kind="stable"):
        if len(seqs) >= max_seqs or (seqs and tot + lens[b] > max_tokens):
            break
        # a sequence longer than the whole budget is sampled as its prefix
        sample_lens[b] = min(int(lens[b]), max_tokens)
        seqs.append(int(b))
        tot += int(sample_lens[b])
    scale = workloads.softmax_scale(w.hd)
    out = codec_api(name)[1](g["q"], g["codec"][name][0], g["table_d"],
                             torch.from_numpy(sample_lens).to(g["q"].device), scale).cpu().numpy()
    host = host_cls(g["nb"], w.n_kv, w.kv_bs, w.hd)
    for b in seqs:
        n = int(sample_lens[b])
        k, v = workloads.kv_rows(w, b, int(lens[b]))
        host.append(k[:n], v[:n], workloads.slot_mapping(w, g["table"], b, n))
    want = ref(workloads.query(w), host, g["table"], sample_lens, scale)
    return {"max_abs_err_vs_oracle_f64": float(np.abs(out[seqs] - want[seqs]).max()),
            "sample": f"{len(seqs)} sequences, {tot} tokens"}


def time_quest(w, g, steps, warmup, top_k):
    """QUEST legs on the int8 cache: the metadata pass over every referenced
    block (a prefill-time op), and one decode step that selects top_k blocks
    per kv head (bounds + top-k kernels) and attends over them
    (q8kv_decode_attn_heads), against the dense step.  Timed with events
    around back-to-back calls on caches[0] (the metadata and the selection
    are small beside the cache)."""
    import torch
    import decode_attention_int8_amd as q8
    scale = workloads.softmax_scale(w.hd)
    cache = g["caches"][0]
    q, bt, sl = g["q"], g["table_d"], g["lens_d"]
    kmax, kmin = q8.quest_metadata(cache, bt, sl)
    sel, sel_lens = q8.quest_select(q, cache, kmax, kmin, bt, sl, top_k)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    R = len(g["caches"])
    meta_us = timed(lambda i: q8.quest_metadata(g["caches"][i % R], bt, sl, kmax, kmin), max(steps // 4, 5))
    select_us = timed(lambda i: q8.quest_select(q, cache, kmax, kmin, bt, sl, top_k, sel, sel_lens), steps)
    sparse_us = timed(lambda i: q8.decode_attn_heads(q, g["caches"][i % R], sel, sel_lens, scale, out=out), steps)
    step_us = timed(lambda i: (q8.quest_select(q, g["caches"][i % R], kmax, kmin, bt, sl, top_k, sel, sel_lens),
                               q8.decode_attn_heads(q, g["caches"][i % R], sel, sel_lens, scale, out=out)), steps)
    lens = g["lens"]
    nblk = [-(-int(L) // w.kv_bs) for L in lens]
    meta_bytes = sum(nblk) * w.n_kv * (w.kv_bs * (w.hd + 4) + 2 * w.hd * 4)
    kept_tokens = int(sel_lens.sum().item()) * w.n_kv
    sparse_bytes = kept_tokens * (2 * w.hd + 8) + 2 * w.batch * w.n_q * w.hd * 4
    return {"top_k": top_k, "kept_tokens_per_kv_head": int(sel_lens.sum().item()),
            "metadata_us": round(meta_us, 3), "metadata_bytes": meta_bytes,
            "metadata_gbs": round(meta_bytes / (meta_us * 1e-6) / 1e9, 1),
            "select_us": round(select_us, 3), "sparse_decode_us": round(sparse_us, 3),
            "sparse_decode_gbs": round(sparse_bytes / (sparse_us * 1e-6) / 1e9, 1),
            "quest_step_us": round(step_us, 3)}


def time_stream_read(g, steps):
    """A plain linear read of the same page pools (K and V) in one launch per
    step, rotated like the decode steps: the streaming ceiling the decode is
    compared with.  Returns (us per read, bytes per read)."""
    import torch
    import decode_attention_int8_amd as q8
    R = len(g["caches"])
    pairs = [(c.k_pages, c.v_pages) for c in g["caches"]]
    nbytes = sum(t.numel() * t.element_size() for t in pairs[0])
    for i in range(3):
        q8.debug_stream_read(*pairs[i % R])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        q8.debug_stream_read(*pairs[i % R])
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps, nbytes


def profiled_traffic(w, key=None):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(key or w.name)
    if not rec:
        return None
    src = b"".join(open(os.path.join(ROOT, f), "rb").read()
                   for f in ("decode_attention_int8_amd/csrc/q8kv.hip", "include/q8kv.h"))
    if hashlib.sha256(src).hexdigest() != rec["source_sha256"]:
        return None
    return rec["traffic_bytes"]


def cpu_baseline(w, g, gpu_out_fn, seconds):
    """Time the oracle (OpenMP over (b, h), all usable host cores, at most 16)
    on a bounded sample of the workload: whole steps repeated for about
    `seconds` when a step is short, else the longest sequences (truncated if
    need be) up to that budget, scaled to a whole step by the token fraction.
    Also compares the GPU's outputs with the oracle's on that sample."""
    import oracle
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    lens, table = g["lens"], g["table"]
    scale = workloads.softmax_scale(w.hd)
    q = workloads.query(w)
    tokens_total = int(lens.sum())
    host = oracle.Cache(g["nb"], w.n_kv, w.kv_bs, w.hd)
    srcs = {}

    def add(b):
        if b not in srcs:
            k, v = workloads.kv_rows(w, b, int(lens[b]))
            host.append(k, v, workloads.slot_mapping(w, table, b, int(lens[b])))
            srcs[b] = (k, v)

    order = [int(b) for b in np.argsort(-lens, kind="stable")]
    add(order[0])
    probe = np.zeros_like(lens)
    probe[order[0]] = min(int(lens[order[0]]), 4096)
    oracle.decode(q, host, table, probe, scale, threads=threads)  # warm: threads, first touches
    t = time.perf_counter()
    oracle.decode(q, host, table, probe, scale, threads=threads)
    sec_per_tok = (time.perf_counter() - t) / int(probe[order[0]])
    budget = max(1, int(seconds / max(sec_per_tok, 1e-12)))
    sl = np.zeros_like(lens)
    acc = 0
    for b in order:
        if acc >= budget:
            break
        take = min(int(lens[b]), budget - acc)
        if take > 0:
            add(b)
            sl[b] = take
            acc += take
    seqs = [b for b in order if sl[b] > 0]
    whole = acc == tokens_total
    # a whole step that is short repeats until the time budget is spent
    reps = 0
    t = time.perf_counter()
    while True:
        want = oracle.decode(q, host, table, sl, scale, threads=threads)
        reps += 1
        secs = time.perf_counter() - t
        if not whole or secs >= seconds:
            break
    step_s = secs / reps / (acc / tokens_total)
    kvb = workloads.kv_bytes(w, lens)
    got = gpu_out_fn(sl)
    err = float(np.abs(got[seqs] - want[seqs]).max())
    want64 = oracle.decode(q, host, table, sl, scale, use_f64=True, threads=threads)
    err64 = float(np.abs(got[seqs] - want64[seqs]).max())
    oracle_drift = float(np.abs(want[seqs] - want64[seqs]).max())
    # q8 vs unquantised fp32 KV on a few heads of the sample
    q8err, rel = [], []
    b = seqs[0]
    Lb = int(sl[b])
    kb, vb = srcs[b]
    for h in range(0, w.n_q, max(1, w.n_q // 4)):
        ex = oracle.exact_f64(q[b, h], kb[:Lb, h // w.group], vb[:Lb, h // w.group], scale)
        q8err.append(np.abs(want[b, h] - ex).max())
        rel.append(np.linalg.norm(want[b, h] - ex) / np.linalg.norm(ex))
    if whole:
        sample = f"the whole step ({tokens_total} tokens, all {w.n_q} heads) repeated {reps} times"
    else:
        sample = (f"{len(seqs)} of {w.batch} sequences, {acc} of {tokens_total} tokens "
                  f"({100.0 * acc / tokens_total:.2f}%), all {w.n_q} heads; time scaled by the token fraction")
    cpu = {"value": round(kvb / step_s / 1e9, 4), "unit": "GB/s", "us_per_step": round(step_s * 1e6, 1),
           "cores": threads, "kind": "oracle", "sample": sample, "sample_seconds": round(secs, 2)}
    parity = {"max_abs_err_vs_oracle": err, "tol": 2e-4, "ok": bool(err <= 2e-4),
              "max_abs_err_vs_oracle_f64": err64, "oracle_f32_vs_f64": oracle_drift,
              "checked": f"{len(seqs)} sequences x {w.n_q} heads (the CPU sample)",
              "q8_vs_fp32kv_max_abs": float(max(q8err)), "q8_vs_fp32kv_rel_l2": float(max(rel))}
    return cpu, parity


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import decode_attention_int8_amd as q8
    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    log(f"workload {w.name}: batch {w.batch}, heads {w.n_q}/{w.n_kv}, hd {w.hd}, kv_bs {w.kv_bs}, "
        f"seq_len {'U{1..%d}' % w.seq_len if w.ragged else w.seq_len}")
    codecs = tuple(c for c in CODECS if not (c == "fp8" and args.no_fp8) and not (c == "q40" and args.no_q40))
    g = build_gpu(w, dev, args.cold_bytes, codecs)
    lens = g["lens"]
    kvb = workloads.kv_bytes(w, lens)
    algo = workloads.step_bytes(w, lens)
    pt, npart = q8.plan(w.batch, w.n_q, w.n_kv, w.hd, w.kv_bs, w.max_blocks)
    if args.part_tokens:
        pt, npart = args.part_tokens, -(-w.max_blocks * w.kv_bs // args.part_tokens)
    log(f"KV bytes/step {kvb / 1e6:.2f} MB, {len(g['caches'])} rotated copies, plan {pt} tokens x {npart} partitions")
    loop_ms, per_call, _ = time_gpu(w, g, args.steps, args.warmup, args.part_tokens)
    log(f"step {loop_ms * 1e3:.2f} us (per call: median {per_call['median']}, min {per_call['min']}, "
        f"p90 {per_call['p90']} us)")
    read_us, read_bytes = time_stream_read(g, args.steps)
    read_gbs = read_bytes / (read_us * 1e-6) / 1e9
    log(f"streaming read of the K+V pools: {read_us:.2f} us, {read_gbs:.0f} GB/s")
    kv_gbs = kvb / (loop_ms * 1e-3) / 1e9
    achieved = algo / (loop_ms * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": round(kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(loop_ms, 5),
        "us_per_step": round(loop_ms * 1e3, 3),
        "hbm_frac": round(kv_gbs / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q, "n_kv_heads": w.n_kv,
                   "hd": w.hd, "kv_bs": w.kv_bs,
                   "seq_len": ("U{1..%d}" % w.seq_len) if w.ragged else w.seq_len,
                   "tokens": int(lens.sum()), "kv_bytes_per_step": kvb, "algorithmic_bytes_per_step": algo,
                   "part_tokens": pt, "n_parts": npart, "cold_cache_copies": len(g["caches"])},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(w),
                     "algorithmic_bytes": algo, "launch_us": round(loop_ms * 1e3, 3)},
        "per_call_us": per_call,
        "stream_read_ceiling": {"gbs": round(read_gbs, 1), "bytes": read_bytes, "us": round(read_us, 3),
                                "frac_of_peak": round(read_gbs / HBM_PEAK_GBS, 4),
                                "decode_frac_of_ceiling": round(achieved / read_gbs, 4)},
        "cpu_baseline": None,
    }
    for name in codecs:
        c_us = time_codec(w, g, name, args.steps, args.warmup, args.part_tokens)
        c_algo = workloads.step_bytes(w, lens, codec=name)
        rec[name] = {"us_per_step": round(c_us, 3), "kv_bytes_per_step": codec_api(name)[2](w, lens),
                     "algorithmic_bytes": c_algo,
                     "achieved_gbs": round(c_algo / (c_us * 1e-6) / 1e9, 2),
                     "frac": round(c_algo / (c_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic(w, f"{w.name}:{name}"),
                     "cold_cache_copies": len(g["codec"][name])}
        log(f"{name} codec: {c_us:.2f} us/step, {rec[name]['achieved_gbs']:.0f} GB/s")
    if not args.no_quest:
        top_k = max(1, -(-w.max_blocks // 8))
        qs = time_quest(w, g, args.steps, args.warmup, top_k)
        qs["dense_us"] = round(loop_ms * 1e3, 3)
        log(f"quest: metadata {qs['metadata_us']} us ({qs['metadata_gbs']} GB/s), select {qs['select_us']} us, "
            f"sparse decode {qs['sparse_decode_us']} us, step {qs['quest_step_us']} us vs dense {qs['dense_us']} us")
        rec["quest"] = qs
    if not args.no_fused:
        fa = time_append_decode(w, g, args.steps, args.warmup, args.part_tokens)
        new_bytes = w.batch * w.n_kv * (2 * w.hd * 4 + 2 * (w.hd + 4))
        fa["algorithmic_bytes"] = algo + new_bytes
        fa["gbs"] = round((algo + new_bytes) / (fa["fused_us"] * 1e-6) / 1e9, 2)
        fa["saved_us"] = round(fa["two_launch_us"] - fa["fused_us"], 3)
        fa["traffic"] = profiled_traffic(w, f"{w.name}:append_decode")
        log(f"append+decode: fused {fa['fused_us']} us, append then decode {fa['two_launch_us']} us "
            f"(append alone {fa['append_us']} us)")
        rec["append_decode"] = fa
    if args.copy_mb > 0:
        n = int(args.copy_mb * 2 ** 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read, {n} bytes written")
        del src, dst
    if not args.no_cpu:
        scale = workloads.softmax_scale(w.hd)

        def gpu_out(sample_lens):
            o = q8.decode_attn(g["q"], g["caches"][0], g["table_d"],
                               torch.from_numpy(np.ascontiguousarray(sample_lens)).to(dev), scale)
            torch.cuda.synchronize()
            return o.cpu().numpy()

        cpu, parity = cpu_baseline(w, g, gpu_out, args.cpu_seconds)
        rec["cpu_baseline"] = cpu
        rec["parity"] = parity
        for name in codecs:
            rec[name]["parity"] = codec_parity(w, g, name)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
