#!/usr/bin/env python3
"""Benchmark: q8-KV single-query decode attention on one MI355X.

One step = one q8kv_decode_attn call over one batch of the workload (Q
quantise, page walk, int8 scoring, online softmax, P.V, split merge); the
KV cache is appended (quantised) beforehand and is resident in HBM when the
timed region starts.  Cold-cache timing: the step rotates over R copies of
the page pool so that R copies span >= 1 GB (four times the MI355X's 256 MB
last-level cache), so each step reads its KV from HBM.

The headline workload is the ragged batch (64 sequences of U{1..32768}
tokens, 64/8 heads), the largest of the five; the 128K-token long-context
step (32/4 heads) is timed in the same run and reported under
"workloads".  Prints ONE JSON line: value = KV GB/s (int8 K and V rows plus
their fp32 scales, per step, divided by the step time), plus us/step, the
roofline of the decode launch (algorithmic bytes / mean launch time, from
HIP events on the launch stream around the timed launches, against 8 TB/s;
traffic = HBM bytes per launch from the committed counter summary when it
matches the kernel source), the per-call distribution (events around each
call of a second pass: median, min, p90), a plain linear read of the same
K+V pools in one launch (the streaming ceiling the decode is compared
with), the CPU oracle timed on a bounded sample of the same workload
(OpenMP over (sequence, head) and single-threaded), and sampled parity
against that oracle and its fp64 twin.  Further legs time the fused step
that also stores each sequence's new token (q8kv_append_decode_attn)
against the same work as two launches (q8kv_append, then
q8kv_decode_attn), the same step over the FP8 codec
(q8kv_fp8_decode_attn) and the q4_0 codec (q8kv_q40_decode_attn), each
with a sampled parity check against its oracle, and QUEST (block metadata,
top-k block selection, decode over the kept blocks).
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
    p.add_argument("--workload", default="ragged", choices=workloads.ORDER)
    p.add_argument("--also", default="long_gqa",
                   help="comma-separated further workloads timed in the same run ('' for none)")
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
    p.add_argument("--load-probe", action="store_true",
                   help="also time the decode kernel's loads alone in three load orders (q8kv_debug_load_probe)")
    p.add_argument("--item-timeline", action="store_true",
                   help="per-item phases of the decode kernel (prologue, tile loop, end, gaps) from a stamped "
                        "copy of the library")
    p.add_argument("--timeline", action="store_true",
                   help="instead of the benchmark: build a copy of the library whose decode kernel "
                        "stamps each workgroup's start, end of streaming and CU, and report the "
                        "timeline of one call after idle and of the last of 30 back-to-back calls")
    p.add_argument("--stage", action="store_true",
                   help="time the LDS-staged variant of the int8 static-grid kernels (same results; "
                        "not the default kernels)")
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
    # (at least 200 calls, so that the quantiles mean something)
    n = max(steps, 200)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
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


LOAD_PATTERNS = {0: "page layout (1 KB operand chunks) + scale loads",
                 1: "page layout, no scale loads",
                 2: "row-major pages read into the same operands + scale loads"}


def time_load_probe(w, g, steps, part_tokens):
    """The decode kernel's loads without its arithmetic over the same pools
    (q8kv_debug_load_probe), one item per partition of the plan, for each
    load pattern: us per launch and the rate of the bytes it loads."""
    import torch
    import decode_attention_int8_amd as q8
    caches = g["caches"]
    item_pages = max(part_tokens // w.kv_bs, -(-128 // w.kv_bs))
    num_pages = caches[0].num_blocks * w.n_kv // item_pages * item_pages
    stream = torch.cuda.current_stream()
    res = {"item_pages": item_pages, "num_pages": num_pages, "patterns": {}}
    for pat, what in LOAD_PATTERNS.items():
        for i in range(3):
            q8.debug_load_probe(caches[i % len(caches)], item_pages, pat, num_pages)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            q8.debug_load_probe(caches[i % len(caches)], item_pages, pat, num_pages)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        nbytes = num_pages * w.kv_bs * (2 * w.hd + (0 if pat == 1 else 8))
        res["patterns"][str(pat)] = {"what": what, "us": round(us, 3), "bytes": nbytes,
                                     "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}
        log(f"load probe {pat} ({what}): {us:.2f} us, {nbytes / (us * 1e-6) / 1e9:.0f} GB/s")
    return res


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


def cpu_model():
    """The host CPU's model string (Linux /proc/cpuinfo), or ''."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def oracle_threads():
    """OpenMP threads of the oracle's parallel pass: every core this process
    may run on, at most 16 (the host share of one GPU on the benchmark
    machines, whatever the machine's own core count)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def host_cache_for(w, g, seqs_lens, host=None, srcs=None):
    """An oracle host cache holding the given sequences' first L tokens
    (dict b -> L), quantised on the host from the same seeded rows (added to
    `host` when given; sequences already in `srcs` are kept)."""
    import oracle
    if host is None:
        host, srcs = oracle.Cache(g["nb"], w.n_kv, w.kv_bs, w.hd), {}
    for b, L in seqs_lens.items():
        if b in srcs and len(srcs[b][0]) >= L:
            continue
        k, v = workloads.kv_rows(w, b, int(g["lens"][b]))
        host.append(k[:L], v[:L], workloads.slot_mapping(w, g["table"], b, L))
        srcs[b] = (k[:L], v[:L])
    return host, srcs


def cpu_baseline(w, g, gpu_out_fn, seconds):
    """Time the oracle on bounded samples of the workload, with OpenMP over
    (sequence, head) on the host share of cores and single-threaded: whole
    steps repeated for about `seconds` when a step is short, else the
    longest sequences (truncated if need be) up to that budget, scaled to a
    whole step by the token fraction.  The two passes must agree bit for bit.
    Also compares the GPU's outputs on the parallel pass's sample with the
    oracle and its fp64 twin."""
    import oracle
    threads = oracle_threads()
    lens, table = g["lens"], g["table"]
    scale = workloads.softmax_scale(w.hd)
    q = workloads.query(w)
    tokens_total = int(lens.sum())
    order = [int(b) for b in np.argsort(-lens, kind="stable")]

    def sample(budget_tokens):
        sl = np.zeros_like(lens)
        acc = 0
        for b in order:
            if acc >= budget_tokens:
                break
            take = min(int(lens[b]), budget_tokens - acc)
            if take > 0:
                sl[b] = take
                acc += take
        return sl, acc

    # rate probe on the longest sequence (first 4096 tokens)
    probe = np.zeros_like(lens)
    probe[order[0]] = min(int(lens[order[0]]), 4096)
    host, srcs = host_cache_for(w, g, {order[0]: int(lens[order[0]])})
    oracle.decode(q, host, table, probe, scale, threads=threads)  # warm: threads, first touches
    t = time.perf_counter()
    oracle.decode(q, host, table, probe, scale, threads=threads)
    sec_per_tok = (time.perf_counter() - t) / int(probe[order[0]])
    sl, acc = sample(max(1, int(seconds / max(sec_per_tok, 1e-12))))
    host, srcs = host_cache_for(w, g, {int(b): int(lens[b]) for b in np.flatnonzero(sl)}, host, srcs)
    seqs = [b for b in order if sl[b] > 0]
    whole = acc == tokens_total

    def timed(sl_, nthreads, min_seconds):
        reps = 0
        t0 = time.perf_counter()
        while True:
            out_ = oracle.decode(q, host, table, sl_, scale, threads=nthreads)
            reps += 1
            secs_ = time.perf_counter() - t0
            if secs_ >= min_seconds:
                break
        return out_, secs_, reps

    want, secs, reps = timed(sl, threads, seconds if whole else 0.0)
    step_s = secs / reps / (acc / tokens_total)
    kvb = workloads.kv_bytes(w, lens)
    # single-threaded pass: a sample sized for about half the budget
    st_budget = max(1, int(0.5 * seconds / max(sec_per_tok * threads, 1e-12)))
    sl1, acc1 = sample(min(st_budget, acc))
    want1, secs1, reps1 = timed(sl1, 1, 0.5 * seconds if acc1 == tokens_total else 0.0)
    par1 = oracle.decode(q, host, table, sl1, scale, threads=threads)
    same = bool(np.array_equal(want1.view(np.uint32), par1.view(np.uint32)))
    step1_s = secs1 / reps1 / (acc1 / tokens_total)
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

    def describe(sl_, acc_, reps_):
        if acc_ == tokens_total:
            return f"the whole step ({tokens_total} tokens, all {w.n_q} heads) repeated {reps_} times"
        n = int(np.count_nonzero(sl_))
        return (f"{n} of {w.batch} sequences, {acc_} of {tokens_total} tokens "
                f"({100.0 * acc_ / tokens_total:.2f}%), all {w.n_q} heads; time scaled by the token fraction")

    cpu = {"value": round(kvb / step_s / 1e9, 4), "unit": "GB/s", "us_per_step": round(step_s * 1e6, 1),
           "cores": threads, "kind": "oracle", "sample": describe(sl, acc, reps),
           "sample_seconds": round(secs, 2),
           "single_thread": {"value": round(kvb / step1_s / 1e9, 4), "unit": "GB/s",
                             "us_per_step": round(step1_s * 1e6, 1), "cores": 1,
                             "sample": describe(sl1, acc1, reps1), "sample_seconds": round(secs1, 2),
                             "bitwise_equal_to_parallel": same},
           "host_nproc": os.cpu_count(), "host_affinity": len(os.sched_getaffinity(0)),
           "cpu_model": cpu_model()}
    parity = {"max_abs_err_vs_oracle": err, "tol": TOL, "ok": bool(err <= TOL),
              "max_abs_err_vs_oracle_f64": err64, "tol_f64": TOL64, "ok_f64": bool(err64 <= TOL64),
              "oracle_f32_vs_f64": oracle_drift,
              "checked": f"{len(seqs)} sequences x {w.n_q} heads (the CPU sample)",
              "q8_vs_fp32kv_max_abs": float(max(q8err)), "q8_vs_fp32kv_rel_l2": float(max(rel))}
    return cpu, parity


# GPU vs the fp32 oracle (the stated bar) and vs its fp64 twin (the tighter
# check: the fp32 oracle itself drifts by up to ~1.8e-4 on long peaked contexts)
TOL, TOL64 = 2e-4, 2e-5


def full_parity(w, g, out, max_seqs=2):
    """Parity of the timed launch's own output (the full sequences, the
    default plan) against the oracle and its fp64 twin, on up to max_seqs
    sequences (the longest first), every query head."""
    import oracle
    lens = g["lens"]
    order = [int(b) for b in np.argsort(-lens, kind="stable") if lens[b] > 0][:max_seqs]
    host, _ = host_cache_for(w, g, {b: int(lens[b]) for b in order})
    sl = np.zeros_like(lens)
    sl[order] = lens[order]
    scale = workloads.softmax_scale(w.hd)
    q = workloads.query(w)
    threads = oracle_threads()
    want = oracle.decode(q, host, g["table"], sl, scale, threads=threads)
    want64 = oracle.decode(q, host, g["table"], sl, scale, use_f64=True, threads=threads)
    got = out.cpu().numpy()
    err = float(np.abs(got[order] - want[order]).max())
    err64 = float(np.abs(got[order] - want64[order]).max())
    return {"max_abs_err_vs_oracle": err, "tol": TOL, "ok": bool(err <= TOL),
            "max_abs_err_vs_oracle_f64": err64, "tol_f64": TOL64, "ok_f64": bool(err64 <= TOL64),
            "checked": f"{len(order)} sequences ({int(sl.sum())} tokens) x {w.n_q} heads, "
                       f"the timed launch's output"}


def decode_record(w, g, args):
    """Time the int8 decode step of a built workload; the roofline, the
    per-call distribution and the streaming-read ceiling."""
    import decode_attention_int8_amd as q8
    lens = g["lens"]
    kvb = workloads.kv_bytes(w, lens)
    algo = workloads.step_bytes(w, lens)
    pt, npart = q8.plan(w.batch, w.n_q, w.n_kv, w.hd, w.kv_bs, w.max_blocks)
    if args.part_tokens:
        pt, npart = args.part_tokens, -(-w.max_blocks * w.kv_bs // args.part_tokens)
    log(f"{w.name}: KV bytes/step {kvb / 1e6:.2f} MB, {len(g['caches'])} rotated copies, "
        f"plan {pt} tokens x {npart} partitions")
    loop_ms, per_call, out = time_gpu(w, g, args.steps, args.warmup, args.part_tokens)
    log(f"{w.name}: step {loop_ms * 1e3:.2f} us (per call: median {per_call['median']}, min {per_call['min']}, "
        f"p90 {per_call['p90']} us)")
    read_us, read_bytes = time_stream_read(g, args.steps)
    read_gbs = read_bytes / (read_us * 1e-6) / 1e9
    log(f"{w.name}: streaming read of the K+V pools: {read_us:.2f} us, {read_gbs:.0f} GB/s")
    kv_gbs = kvb / (loop_ms * 1e-3) / 1e9
    achieved = algo / (loop_ms * 1e-3) / 1e9
    config = {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q, "n_kv_heads": w.n_kv,
              "hd": w.hd, "kv_bs": w.kv_bs,
              "seq_len": ("U{1..%d}" % w.seq_len) if w.ragged else w.seq_len,
              "tokens": int(lens.sum()), "kv_bytes_per_step": kvb, "algorithmic_bytes_per_step": algo,
              "part_tokens": pt, "n_parts": npart, "cold_cache_copies": len(g["caches"])}
    if args.stage:
        config["kernel_variant"] = "lds_staged"
    rec = {"us_per_step": round(loop_ms * 1e3, 3), "kv_gbs": round(kv_gbs, 2),
           "hbm_frac": round(kv_gbs / HBM_PEAK_GBS, 4), "config": config,
           "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(w),
                        "algorithmic_bytes": algo, "launch_us": round(loop_ms * 1e3, 3)},
           "per_call_us": per_call,
           "stream_read_ceiling": {"gbs": round(read_gbs, 1), "bytes": read_bytes, "us": round(read_us, 3),
                                   "frac_of_peak": round(read_gbs / HBM_PEAK_GBS, 4),
                                   "decode_frac_of_ceiling": round(achieved / read_gbs, 4)}}
    return rec, loop_ms, out


# Per-workgroup wall-clock stamps (s_memrealtime, 100 MHz) for --timeline:
# inserted into a copy of the kernel source at these points, each of which
# must occur exactly once (tests/test_bench_contract.py checks that).
TIMELINE_EDITS = [
    ("struct DecodeArgs {",
     "__device__ unsigned long long g_stamp[4096 * 8];\n"
     "#define STAMP(k, val) do { if (threadIdx.x == 0 && blockIdx.x < 4096) "
     "g_stamp[blockIdx.x * 8 + (k)] = (val); } while (0)\n"
     "struct DecodeArgs {"),
    ("    const int tid = threadIdx.x;\n    const int lane = tid & (kWave - 1);\n"
     "    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);\n    const int G = a.group;",
     "    STAMP(0, __builtin_amdgcn_s_memrealtime());\n"
     "    const int tid = threadIdx.x;\n    const int lane = tid & (kWave - 1);\n"
     "    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);\n    const int G = a.group;"),
    ("        const bool any_bad = __syncthreads_or(bad);",
     "        const bool any_bad = __syncthreads_or(bad);\n"
     "        STAMP(1, __builtin_amdgcn_s_memrealtime());\n"
     "        STAMP(2, (unsigned long long)__smid());"),
    ('extern "C" {\n',
     'extern "C" {\n'
     "int q8kv_timeline_read(unsigned long long* host, int n) {\n"
     "    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_stamp), sizeof(unsigned long long) * (size_t)n, 0,"
     " hipMemcpyDeviceToHost);\n}\n"
     "int q8kv_timeline_clear() {\n"
     "    static unsigned long long z[4096 * 8];\n"
     "    return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_stamp), z, sizeof(z), 0, hipMemcpyHostToDevice);\n}\n"),
]


# Per-item wall-clock stamps for --item-timeline: the start of each of a
# workgroup's first eight items, the end of its query prologue, the end of
# its tile loop and the end of its merge, plus the item's number.
ITEM_EDITS = [
    ("struct DecodeArgs {",
     "__device__ unsigned long long g_items[4096 * 8 * 6];\n"
     "#define ISTAMP(p, val) do { if (threadIdx.x == 0 && blockIdx.x < 4096 && kst < 8) "
     "g_items[(blockIdx.x * 8 + kst) * 6 + (p)] = (val); } while (0)\n"
     "struct DecodeArgs {"),
    ("    int item = blockIdx.x;\n", "    int item = blockIdx.x;\n    int kst = 0;\n"),
    ("        int itid = tid;\n",
     "        int itid = tid;\n        ISTAMP(0, __builtin_amdgcn_s_memrealtime());\n"
     "        ISTAMP(5, (unsigned long long)item);\n"),
    ("        } else {\n            __syncthreads();\n        }\n        // static grids: the tail wave quantises",
     "        } else {\n            __syncthreads();\n        }\n        ISTAMP(1, __builtin_amdgcn_s_memrealtime());\n"
     "        // static grids: the tail wave quantises"),
    ("        const bool any_bad = __syncthreads_or(bad);\n",
     "        const bool any_bad = __syncthreads_or(bad);\n        ISTAMP(2, __builtin_amdgcn_s_memrealtime());\n"),
    ("        // next item (the barrier also keeps LDS from being reused too early)\n",
     "        ISTAMP(3, __builtin_amdgcn_s_memrealtime());\n        ++kst;\n"
     "        // next item (the barrier also keeps LDS from being reused too early)\n"),
    ('extern "C" {\n',
     'extern "C" {\n'
     "int q8kv_items_read(unsigned long long* host, int n) {\n"
     "    return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_items), sizeof(unsigned long long) * (size_t)n, 0,"
     " hipMemcpyDeviceToHost);\n}\n"
     "int q8kv_items_clear() {\n"
     "    static unsigned long long z[4096 * 8 * 6];\n"
     "    return (int)hipMemcpyToSymbol(HIP_SYMBOL(g_items), z, sizeof(z), 0, hipMemcpyHostToDevice);\n}\n"),
]


def stamped_source(src, edits):
    for a, b in edits:
        if src.count(a) != 1:
            raise RuntimeError(f"stamp anchor not found exactly once: {a[:40]!r}")
        src = src.replace(a, b)
    return src


def timeline_source(src):
    return stamped_source(src, TIMELINE_EDITS)


def items_source(src):
    return stamped_source(src, ITEM_EDITS)


def stamped_library(make_source):
    """Build a copy of the library from make_source(kernel source) in a
    temporary directory and make the binding call it; returns its handle."""
    import ctypes
    import importlib.util
    import subprocess
    import tempfile
    import decode_attention_int8_amd as q8
    spec = importlib.util.spec_from_file_location("_q8kv_build_tl", os.path.join(ROOT, "decode_attention_int8_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    d = tempfile.mkdtemp(prefix="q8kv_stamped_")
    srcp, libp = os.path.join(d, "q8kv_stamped.hip"), os.path.join(d, "libq8kv_stamped.so")
    open(srcp, "w").write(make_source(open(b.SRC).read()))
    log("building the stamped library copy")
    subprocess.run([b.HIPCC] + b.FLAGS + [srcp, "-o", libp], check=True, capture_output=True)
    q8.LIB_PATH = libp
    q8.lib = q8._load()
    return ctypes.CDLL(libp)


def run_items(w, args):
    """Per-item phases of the decode kernel from the stamped library copy:
    for the last of 30 back-to-back calls, each item's query prologue, tile
    loop and end (wave merge, state store, merge) and each workgroup's gap
    between items, with the share of all workgroup time each takes."""
    import ctypes
    import torch
    import decode_attention_int8_amd as q8
    T = stamped_library(items_source)
    g = build_gpu(w, torch.device("cuda", 0), args.cold_bytes, codecs=())
    scale = workloads.softmax_scale(w.hd)
    out = torch.empty_like(g["q"])
    R = len(g["caches"])

    def call(i):
        q8.decode_attn(g["q"], g["caches"][i % R], g["table_d"], g["lens_d"], scale, out=out,
                       part_tokens=args.part_tokens)

    for i in range(50):
        call(i)
    torch.cuda.synchronize()
    if T.q8kv_items_clear() != 0:
        raise RuntimeError("stamp clear failed")
    torch.cuda.synchronize()
    for i in range(30):
        call(i)
    torch.cuda.synchronize()
    n = 4096 * 8 * 6
    st = np.zeros(n, np.uint64)
    if T.q8kv_items_read(st.ctypes.data_as(ctypes.c_void_p), n) != 0:
        raise RuntimeError("stamp read failed")
    st = st.reshape(4096, 8, 6).astype(np.int64)
    # slot 0 of a workgroup holds its first item of the last call; a later
    # slot belongs to that call when it starts after the previous item ended
    # and its four stamps are in order (the persistent loop stamps the start
    # of the check that finds no item left, then leaves)
    items = {}
    for wg in range(4096):
        if st[wg, 0, 0] <= 0:
            continue
        lst = []
        for k in range(8):
            s_ = st[wg, k]
            ok = s_[0] <= s_[1] <= s_[2] <= s_[3] and (k == 0 or s_[0] >= lst[-1][3])
            if not ok:
                break
            lst.append(s_[:4])
        items[wg] = np.array(lst)
    t0 = min(v[0, 0] for v in items.values())
    ph = np.concatenate([np.diff(v, axis=1) for v in items.values()]) / 100.0
    gaps = np.concatenate([(v[1:, 0] - v[:-1, 3]) for v in items.values() if len(v) > 1] or [np.zeros(0)]) / 100.0
    ends = np.array([v[-1, 3] - t0 for v in items.values()]) / 100.0
    starts = np.array([v[0, 0] - t0 for v in items.values()]) / 100.0
    span = float(ends.max())
    total = span * len(items)
    q = lambda x, p: round(float(np.percentile(x, p)), 2) if len(x) else None
    dist = lambda x: {"min": q(x, 0), "median": q(x, 50), "p90": q(x, 90), "max": q(x, 100)}
    return {"workgroups": len(items), "items": int(len(ph)), "span_us": round(span, 2),
            "items_per_workgroup": np.bincount([len(v) for v in items.values()]).tolist(),
            "prologue_us": dist(ph[:, 0]), "tile_loop_us": dist(ph[:, 1]), "end_us": dist(ph[:, 2]),
            "gap_us": dist(gaps), "workgroup_end_us": dist(ends),
            "share_of_workgroup_time": {
                "before_first_item": round(float(starts.sum()) / total, 4),
                "prologue": round(float(ph[:, 0].sum()) / total, 4),
                "tile_loop": round(float(ph[:, 1].sum()) / total, 4),
                "end": round(float(ph[:, 2].sum()) / total, 4),
                "gaps": round(float(gaps.sum()) / total, 4),
                "idle_after_last_item": round(float((span - ends).sum()) / total, 4)}}


def run_timeline(w, args):
    """Build the stamped copy of the library, run the workload's decode, and
    return the per-workgroup timeline (µs from the first workgroup's start)."""
    import ctypes
    import torch
    import decode_attention_int8_amd as q8
    T = stamped_library(timeline_source)
    g = build_gpu(w, torch.device("cuda", 0), args.cold_bytes, codecs=())
    scale = workloads.softmax_scale(w.hd)
    out = torch.empty_like(g["q"])
    R = len(g["caches"])
    state = {"i": 0}

    def call():
        q8.decode_attn(g["q"], g["caches"][state["i"] % R], g["table_d"], g["lens_d"], scale, out=out,
                       part_tokens=args.part_tokens)
        state["i"] += 1

    def read():
        st = np.zeros(4096 * 8, np.uint64)
        if T.q8kv_timeline_read(st.ctypes.data_as(ctypes.c_void_p), 4096 * 8) != 0:
            raise RuntimeError("stamp read failed")
        st = st.reshape(4096, 8).astype(np.int64)
        s_ = st[st[:, 0] > 0]
        t0 = s_[:, 0].min()
        start, end = (s_[:, 0] - t0) / 100.0, (s_[:, 1] - t0) / 100.0
        xcd = s_[:, 2] >> 6
        q = lambda x, p: round(float(np.percentile(x, p)), 2)
        return {"workgroups": int(len(s_)),
                "start_us": {"median": q(start, 50), "max": q(start, 100)},
                "stream_end_us": {"min": q(end, 0), "median": q(end, 50), "p90": q(end, 90), "max": q(end, 100)},
                "duration_us": {"median": q(end - start, 50), "max": q(end - start, 100)},
                "by_cu_group": {int(x): {"workgroups": int((xcd == x).sum()), "start_median": q(start[xcd == x], 50),
                                         "end_median": q(end[xcd == x], 50), "end_max": q(end[xcd == x], 100)}
                                for x in np.unique(xcd)}}

    for _ in range(50):
        call()
    torch.cuda.synchronize()
    res = {}
    for mode, n in (("after_idle", 1), ("back_to_back_last_of_30", 30)):
        if T.q8kv_timeline_clear() != 0:
            raise RuntimeError("stamp clear failed")
        torch.cuda.synchronize()
        for _ in range(n):
            call()
        torch.cuda.synchronize()
        res[mode] = read()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import decode_attention_int8_amd as q8
    q8.debug_set_stage(args.stage)
    w = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    if args.item_timeline:
        print(json.dumps({"items": run_items(w, args), "workload": w.name,
                          "note": "µs; one workgroup's items of the last of 30 back-to-back calls (its first eight)"}),
              flush=True)
        return
    if args.timeline:
        print(json.dumps({"timeline": run_timeline(w, args), "workload": w.name,
                          "note": "µs from the first workgroup's start; stream_end = after the tile loop, "
                                  "before the wave merge; CU groups are __smid() >> 6"}), flush=True)
        return
    log(f"workload {w.name}: batch {w.batch}, heads {w.n_q}/{w.n_kv}, hd {w.hd}, kv_bs {w.kv_bs}, "
        f"seq_len {'U{1..%d}' % w.seq_len if w.ragged else w.seq_len}")
    codecs = tuple(c for c in CODECS if not (c == "fp8" and args.no_fp8) and not (c == "q40" and args.no_q40))
    g = build_gpu(w, dev, args.cold_bytes, codecs)
    lens = g["lens"]
    algo = workloads.step_bytes(w, lens)
    head, loop_ms, _ = decode_record(w, g, args)
    probe = time_load_probe(w, g, args.steps, head["config"]["part_tokens"]) if args.load_probe else None
    rec = {
        "metric": METRIC,
        "value": head["kv_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(loop_ms, 5),
        "us_per_step": head["us_per_step"],
        "hbm_frac": head["hbm_frac"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "per_call_us": head["per_call_us"],
        "stream_read_ceiling": head["stream_read_ceiling"],
        "cpu_baseline": None,
    }
    if probe:
        rec["load_probe"] = probe
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
        log(f"cpu baseline: {cpu['us_per_step']} us/step on {cpu['cores']} threads, "
            f"{cpu['single_thread']['us_per_step']} us/step on one; parity {parity['max_abs_err_vs_oracle']:.3g} "
            f"(fp64 {parity['max_abs_err_vs_oracle_f64']:.3g})")
        for name in codecs:
            rec[name]["parity"] = codec_parity(w, g, name)
    # further workloads, each with its own record
    also = [x for x in args.also.split(",") if x and x != w.name]
    if also:
        del g
        torch.cuda.empty_cache()
        rec["workloads"] = {}
        for name in also:
            wx = workloads.WORKLOADS[name]
            gx = build_gpu(wx, dev, args.cold_bytes, codecs=())
            rx, _, out = decode_record(wx, gx, args)
            if not args.no_cpu:
                rx["parity"] = full_parity(wx, gx, out)
                log(f"{name}: parity {rx['parity']['max_abs_err_vs_oracle']:.3g} "
                    f"(fp64 {rx['parity']['max_abs_err_vs_oracle_f64']:.3g})")
            rec["workloads"][name] = rx
            del gx
            torch.cuda.empty_cache()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
