#!/usr/bin/env python3
"""Decode-step benchmark on one MI355X: quantize-append + split-K decode attention.

A step is one pass of the whole hot path on one batch: each sequence appends one new
token (fused Hadamard rotation + INT4 group quantization into the cache), then every
sequence runs GQA decode attention over its full quantized context (split-K kernel +
combine). By default the step is one kvq_decode_step call, whose split-K launch does the
append first in the unit that reads the new token; --unfused makes it the two calls
kvq_quantize_append + kvq_decode_attention (windows, value token groups, pruning and
the reference kernel always take separate calls). Inputs are seeded synthetic tensors
resident in HBM before timing starts.

Prints one JSON line. `value` is effective KV GB/s of the whole step (algorithmic
bytes / step time); `roofline` covers the dominant kernel (the split-K decode), timed
with HIP events the library records on its stream at the start and end of every launch
(as part of the launch itself). Before the W warmup
steps the step runs untimed for --settle-s seconds (default 0.25): the GPU's clocks
need some 50-100 ms of sustained load to settle.

  python bench.py [--steps K] [--warmup W] [--workload h1] [--gpus 1] [--window S,R] [--eager] [--unfused]

The timed step is the median of --repeats (5) timed replays of the K steps captured in one
HIP graph (after untimed replays for --settle-s seconds, at least one);
the eager host-launched K steps run first, and their per-launch events time the split
kernel for the roofline. --eager reports the host-launched step time instead.

With --window S,R the first S and last R tokens of every sequence stay in bf16
windows (InnerQ, Abstract): a step appends through the windows (the token leaving the
recent window is quantized into the cache) and decodes over windows and cache together.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn µs/step + effective KV GB/s (% HBM peak) at INT4, 32K ctx"
HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (the library records them; torch.cuda.Event only times
    events torch itself recorded)."""

    def __init__(self, n: int):
        import ctypes

        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e)

    def pair(self, i: int):
        return self.ev[2 * i].value, self.ev[2 * i + 1].value

    def elapsed_ms(self, i: int) -> float:
        f = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(f), self.ev[2 * i], self.ev[2 * i + 1]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in ("decode_mfma.h", "decode_mfma.hip", "decode_paged.hip", "kvq_device.h"):
        with open(os.path.join(ROOT, "bit_kv_cache_quantize_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profile_key(args) -> str:
    """Name of a run's split-kernel configuration: the workload and every option that
    changes what that kernel reads or how it runs (h1, h1_prune2, h1_window32x128, ...)."""
    key = args.workload
    if args.prune:
        key += f"_prune{args.prune}"
    if args.window:
        key += "_window" + args.window.replace(",", "x")
    if args.vgroup:
        key += "_vgroup"
    if args.hybrid:
        key += "_hybrid"
    if args.hadamard_block >= 0:
        key += f"_hb{args.hadamard_block}"
    if args.page_size >= 0:
        key += f"_p{args.page_size}"
    if args.num_splits:
        key += f"_splits{args.num_splits}"
    if args.unfused:
        key += "_unfused"
    return key


def traffic_from_profile(key: str):
    """HBM bytes per split-kernel launch from committed rocprofv3 counter runs of the same
    configuration (profile_key), or None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"decode_split_{key}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def host_threads() -> int:
    """Host threads for the oracle's multi-thread timing: the CPUs this process may run
    on, at most 16 (one GPU's share of a multi-GPU host) and at most OMP_NUM_THREADS
    when that is set."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, min(n, 16))


def host_description() -> dict:
    """CPU model (from /proc/cpuinfo) and core counts of the host the oracle ran on."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": aff}


def measure_stream_ceiling(kvq, dev, gib: int, reps: int = 10) -> dict:
    """Read bandwidth of this GPU for the decode kernel's load shape (kvq_stream_read: one
    16-byte load per lane, whole cache lines per wave instruction) over a `gib` GiB buffer,
    plain and non-temporal, at 2, 4 and 8 workgroups of 256 threads per CU; mean of `reps`
    hipEvent-timed launches per setting after one untimed launch. `ceiling` is the best."""
    import torch

    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)  # written once, so every page is resident
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    ev = HipEvents(reps)
    res = {}
    try:
        for nt in (1, 0):
            for wpc in (2, 4, 8):
                kvq.stream_read(buf, bool(nt), wpc, sink)
                for i in range(reps):
                    kvq.stream_read(buf, bool(nt), wpc, sink, events=ev.pair(i))
                torch.cuda.synchronize()
                ms = sum(ev.elapsed_ms(i) for i in range(reps)) / reps
                res[f"{'nontemporal' if nt else 'plain'}_wg{wpc}"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    finally:
        ev.close()
        del buf
    best = max(res.values())
    return {"ceiling": best, "unit": "GB/s", "bytes": nbytes, "settings": res,
            "best_setting": max(res, key=res.get), "frac_of_peak": round(best / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="h1")
    ap.add_argument("--reference", action="store_true", help="time the plain-VALU decode kernel instead")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--settle-s", type=float, default=0.25,
                    help="seconds of untimed steps before the warmup steps (the clocks settle under load)")
    ap.add_argument("--cpu-sample-seqs", type=int, default=2,
                    help="sequences in the oracle's one-thread timed sample (the multi-thread sample runs one "
                         "sequence per host thread)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-repeats", type=int, default=3,
                    help="runs of the oracle's timed sample; the CPU baseline is their median")
    ap.add_argument("--parity-seqs", type=int, default=2, help="sequences checked against the oracle")
    ap.add_argument("--window", default="", help="S,R: bf16 sink and recent windows of S and R tokens")
    ap.add_argument("--hybrid", action="store_true", help="hybrid symmetric/asymmetric groups (quant_mode 1)")
    ap.add_argument("--hadamard-block", type=int, default=-1,
                    help="override the workload's rotation block (0 = no rotation), e.g. to time rotation on/off")
    ap.add_argument("--page-size", type=int, default=-1,
                    help="override the workload's page size (tokens, a multiple of 16; 0 = one page per sequence), "
                         "e.g. to time a contiguous workload on paged caches")
    ap.add_argument("--vgroup", action="store_true",
                    help="values grouped along tokens (v_grouping 1) with a bf16 residual of one group")
    ap.add_argument("--prune", type=int, default=0,
                    help="query-channel pruning: key chunks kept per (sequence, kv head), of bits * head_dim / 128")
    ap.add_argument("--no-stream-probe", action="store_true", help="skip the read-stream ceiling measurement")
    ap.add_argument("--unfused", action="store_true",
                    help="append and decode as two calls (default: kvq_decode_step where the cache allows it)")
    ap.add_argument("--eager", action="store_true",
                    help="time the steps as host launches (default: the K steps replayed from one HIP graph)")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed replays of the K-step graph; the step time is their median")
    ap.add_argument("--stream-gib", type=int, default=4, help="GiB read by the read-stream probe")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="run one plain elementwise copy (torch.neg, fp32) of this many MiB before timing, "
                         "so hardware byte counters can be scaled against a kernel of known traffic")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this benchmark runs on exactly one GPU; --gpus must be 1 (the split-K decode would "
              "shard by batch, kv head or sequence range across GPUs, which is not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_kv_cache_quantize_amd as kvq
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.get(args.workload)
    if args.hadamard_block >= 0:
        w = w.with_(hadamard_block=args.hadamard_block)
    if args.page_size >= 0:
        w = w.with_(page_size=args.page_size)
    if w.ragged is not None:
        lens = wl.seq_lens(w)
    else:
        lens = torch.full((w.batch,), w.context, dtype=torch.int32)
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    # the step appends token T-1 of every sequence (its slot is rewritten each step, so
    # every step does the work of a real decode step at context T)
    geo = wl.geometry(w, extra_tokens=0, lens=lens)
    win_S, win_R = (int(x) for x in args.window.split(",")) if args.window else (0, 0)
    windowed = bool(args.window)
    residual = args.vgroup  # a window with sink 0 whose ring holds the incomplete last group
    if residual:
        if windowed:
            sys.exit("bench.py: --vgroup brings its own residual window")
        win_S, win_R, windowed = 0, w.group_size, True
    maxlen = int(lens.max())
    # the fused step covers plain caches: no windows, value token groups or pruning, the matrix kernel
    fused = not (args.unfused or windowed or args.prune or args.reference)
    t0 = time.time()
    cache = kvq.KVCache.allocate(d, Hkv, w.bits, w.group_size, w.hadamard_block, geo.page_size, geo.num_pages,
                                 device=dev, quant_mode=1 if args.hybrid else 0, v_grouping=1 if args.vgroup else 0)
    log(f"[bench] {w.name}: cache {cache.nbytes / 1e9:.2f} GB, B={B} Hq={Hq} Hkv={Hkv} T<= {maxlen}")
    window = kvq.KVWindow.allocate(cache, win_S, win_R, B, device=dev, residual=int(residual)) if windowed else None
    for b in range(B):
        T = int(lens[b])
        k, v = wl.keys(w, b, 0, T, device=dev), wl.values(w, b, 0, T, device=dev)
        if not windowed:
            kvq.quantize_append(cache, k, v, geo.slots(b, 0, T).to(dev))
        elif residual:
            # state before the step's token T-1: whole groups quantized, the rest in the ring
            done = (T - 1) - (T - 1) % win_R
            if done:
                kvq.quantize_append(cache, k[:done].contiguous(), v[:done].contiguous(), geo.slots(b, 0, done).to(dev))
            for t in range(done, T - 1):
                window.k[b, t % win_R] = k[t]
                window.v[b, t % win_R] = v[t]
        else:
            # state before the step's token T-1: sink rows, the ring holding T-1-R..T-2,
            # and the tokens between quantized
            lo, hi = win_S, T - 1 - win_R
            if hi > lo:
                kvq.quantize_append(cache, k[lo:hi].contiguous(), v[lo:hi].contiguous(),
                                    geo.slots(b, lo, hi - lo).to(dev))
            for t in list(range(min(win_S, T - 1))) + list(range(max(win_S, T - 1 - win_R), T - 1)):
                window.k[b, window.row(t)] = k[t]
                window.v[b, window.row(t)] = v[t]
        del k, v
    torch.cuda.synchronize()
    log(f"[bench] cache built in {time.time() - t0:.1f}s")

    # KV bytes of one layer exceed the 256 MB Infinity Cache by far for the 32K workloads;
    # smaller ones cycle through enough distinct copies to defeat it.
    ring = max(1, math.ceil(1.0e9 / cache.nbytes)) if cache.nbytes < 1.0e9 else 1
    caches = [cache]
    windows = [window]
    for _ in range(ring - 1):
        caches.append(cache.clone())
        windows.append(kvq.KVWindow(win_S, win_R, B, window.k.clone(), window.v.clone(), int(residual))
                       if windowed else None)

    n_inputs = 4
    qs = [wl.queries(w, step=s, device=dev) for s in range(n_inputs)]
    news = [wl.new_tokens(w, step=s, device=dev) for s in range(n_inputs)]
    last_slots = torch.stack([geo.slots(b, int(lens[b]) - 1, 1)[0] for b in range(B)]).to(dev)
    bt = geo.block_table.to(dev)
    lens_d = lens.to(dev)
    if windowed:
        ws_bytes = kvq.decode_window_workspace_bytes(cache, window, B, Hq, maxlen, args.num_splits)
        num_splits = kvq.decode_num_splits(cache, B, Hq, max(maxlen - win_S - win_R, 0), args.num_splits)
        seqs_d = torch.arange(B, dtype=torch.int32, device=dev)
        pos_d = (lens - 1).to(dev)
        # the evicted token's slot, or with a residual the first slot of the group the
        # step's token completes
        first = (lambda T: T - win_R) if residual else (lambda T: T - 1 - win_R)
        evict_d = torch.stack([geo.slots(b, max(first(int(lens[b])), 0), 1)[0] for b in range(B)]).to(dev)
    else:
        ws_bytes = kvq.decode_workspace_bytes(cache, B, Hq, maxlen, args.num_splits)
        num_splits = kvq.decode_num_splits(cache, B, Hq, maxlen, args.num_splits)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    if args.prune and (windowed or args.reference):
        sys.exit("bench.py: --prune runs the matrix kernel without windows")
    chunk_mask = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)

    if args.calibration_copy_mb > 0:
        n = args.calibration_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)  # reads and writes exactly n*4 bytes
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy: {args.calibration_copy_mb} MiB read + written")

    hip_events = HipEvents(args.steps)

    applied0 = []  # input indices of the steps applied to caches[0], in order

    def step(i: int, events=None):
        c = caches[i % ring]
        kn, vn = news[i % n_inputs]
        if i % ring == 0:
            applied0.append(i % n_inputs)
        if windowed:
            kvq.window_append(c, windows[i % ring], kn, vn, seqs_d, pos_d, evict_d)
            kvq.decode_attention_window(c, windows[i % ring], qs[i % n_inputs], bt, lens_d, maxlen,
                                        num_splits=args.num_splits, workspace=ws, out=out, events=events)
            return
        if fused:
            kvq.decode_step(c, kn, vn, qs[i % n_inputs], bt, lens_d, maxlen, num_splits=args.num_splits,
                            workspace=ws, out=out, events=events)
            return
        kvq.quantize_append(c, kn, vn, last_slots)
        if args.prune:
            kvq.decode_attention_pruned(c, qs[i % n_inputs], bt, lens_d, maxlen, args.prune,
                                        num_splits=args.num_splits, chunk_mask=chunk_mask, workspace=ws, out=out,
                                        events=events)
            return
        kvq.decode_attention(c, qs[i % n_inputs], bt, lens_d, maxlen, num_splits=args.num_splits, workspace=ws,
                             out=out, events=events, reference=args.reference)

    # The GPU needs some 50-100 ms of sustained load before its clocks settle: untimed
    # steps for settle_s seconds (checked every 20 steps), then the warmup steps.
    n_settle = 0
    t_settle = time.perf_counter()
    while args.settle_s > 0:
        for _ in range(20):
            step(n_settle)
            n_settle += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t_settle >= args.settle_s:
            break
    for i in range(args.warmup):
        step(n_settle + i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(n_settle + args.warmup + i, events=None if args.reference else hip_events.pair(i))
    end.record()
    total_steps = n_settle + args.warmup + args.steps
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    split_ms = None
    if not args.reference:
        split_ms = float(np.mean([hip_events.elapsed_ms(i) for i in range(args.steps)]))
    hip_events.close()

    # The same K steps replayed from one HIP graph: the three kernels of a step then run
    # back to back without host launches between them (short steps are otherwise paced by
    # the host). The graph is replayed untimed (see below), then timed --repeats times;
    # the last replayed step's output must equal the eager step's bit for bit. The split
    # kernel's event-timed launches above give the roofline either way.
    graph = None
    if not args.eager and not windowed and not args.reference:
        base = total_steps
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for j in range(min(args.steps, 8)):
                step(base + j)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for j in range(args.steps):
                step(base + j)
        # the capture leaves the GPU idle long enough for its clocks to drop: untimed
        # replays for settle_s seconds (at least one) before the timed ones; a short K
        # (20 steps of h1 are ~9 ms) would otherwise be timed on unsettled clocks
        n_untimed = 0
        t_settle = time.perf_counter()
        while True:
            g.replay()
            n_untimed += 1
            torch.cuda.synchronize()
            if time.perf_counter() - t_settle >= args.settle_s:
                break
        # the timed replay, repeated: the step is the median of the repeats
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = []
        for _ in range(max(1, args.repeats)):
            g0.record()
            g.replay()
            g1.record()
            torch.cuda.synchronize()
            reps.append(g0.elapsed_time(g1) / args.steps)
        graph_ms = float(np.median(reps))
        replayed = out.clone()
        step(base + args.steps - 1)
        torch.cuda.synchronize()
        graph = {"us_per_step": round(graph_ms * 1e3, 2), "steps": args.steps,
                 "matches_eager": bool(torch.equal(replayed, out)), "us_per_step_eager": round(ms * 1e3, 2),
                 "untimed_replays": n_untimed, "repeats_us_per_step": [round(r * 1e3, 2) for r in reps]}
        if not graph["matches_eager"]:
            sys.exit("bench.py: the graph-replayed step differs from the eager step")
        ms = graph_ms
        total_steps = base + args.steps
        del g

    # algorithmic bytes (what the method must move; no re-reads, no partials)
    per_tok_head = wl.kv_bytes_per_token_head(d, w.bits, w.group_size)
    kv_bytes = int(lens.to(torch.int64).sum()) * Hkv * per_tok_head
    q_bytes = B * Hq * d * 2
    out_bytes = B * Hq * d * 4
    append_bytes = B * Hkv * (2 * d * 2 + per_tok_head)
    n_chunks = d * w.bits // 128
    if args.prune:
        # pruned key chunks are not read: per token and kv head the K codes shrink to
        # keep / n_chunks of a row
        kv_bytes -= int(lens.to(torch.int64).sum()) * Hkv * (d * w.bits // 8) * (n_chunks - args.prune) // n_chunks
    if residual:
        # the residual holds T % G tokens at decode time; the append writes the token and,
        # when it completes a group, reads the G ring rows and writes their quantized form
        n_win = sum(int(T) % win_R for T in lens)
        split_kv_bytes = (int(lens.to(torch.int64).sum()) - n_win) * Hkv * per_tok_head
        kv_bytes = split_kv_bytes + n_win * Hkv * 2 * d * 2
        completing = sum(1 for T in lens if int(T) % win_R == 0)
        append_bytes = B * Hkv * 2 * (2 * d * 2) + completing * Hkv * win_R * (2 * d * 2 + per_tok_head)
    elif windowed:
        # window tokens are read as bf16 K and V rows; the append reads the new token,
        # writes it to the ring, reads the evicted row and writes its quantized form
        n_win = sum(min(win_S, int(T)) + min(win_R, max(int(T) - win_S, 0)) for T in lens)
        split_kv_bytes = (int(lens.to(torch.int64).sum()) - n_win) * Hkv * per_tok_head
        kv_bytes = split_kv_bytes + n_win * Hkv * 2 * d * 2
        append_bytes = B * Hkv * (3 * 2 * d * 2 + per_tok_head)
    step_bytes = kv_bytes + q_bytes + out_bytes + append_bytes
    # the split kernel reads the quantized span only (window tokens go to the window kernel);
    # a fused step's split kernel also does the append
    split_bytes = (split_kv_bytes if windowed else kv_bytes) + q_bytes + (append_bytes if fused else 0)
    value = step_bytes / (ms * 1e-3) / 1e9

    roofline = None
    if split_ms is not None:
        achieved = split_bytes / (split_ms * 1e-3) / 1e9
        traffic = traffic_from_profile(profile_key(args))
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": "decode_split", "profile_key": profile_key(args),
                    "algorithmic_bytes_per_launch": split_bytes,
                    "avg_launch_us": round(split_ms * 1e3, 2)}

    # ---- read-stream ceiling of this GPU, measured in the same process ----
    stream = None
    if not args.no_stream_probe:
        stream = measure_stream_ceiling(kvq, dev, args.stream_gib)
        if roofline is not None:
            roofline["stream_ceiling"] = stream["ceiling"]
            roofline["pct_of_stream"] = round(100.0 * roofline["achieved"] / stream["ceiling"], 2)

    # ---- parity on sampled sequences (the oracle recomputes them from the same bytes) ----
    parity = None
    cpu = None
    if windowed:
        args.no_cpu_baseline = True  # the CPU baseline is the default (window-free) workload's
    want_oracle = args.parity_seqs > 0 or not args.no_cpu_baseline
    if want_oracle:
        import concurrent.futures as cf

        import oracle

        # the last timed step's inputs
        i_last = total_steps - 1
        kn, vn = news[i_last % n_inputs]
        q_last = qs[i_last % n_inputs]
        applied0.append(i_last % n_inputs)
        if windowed:
            kvq.window_append(caches[0], windows[0], kn, vn, seqs_d, pos_d, evict_d)
            kvq.decode_attention_window(caches[0], windows[0], q_last, bt, lens_d, maxlen,
                                        num_splits=args.num_splits, workspace=ws, out=out)
        elif args.prune:
            kvq.quantize_append(caches[0], kn, vn, last_slots)
            kvq.decode_attention_pruned(caches[0], q_last, bt, lens_d, maxlen, args.prune,
                                        num_splits=args.num_splits, chunk_mask=chunk_mask, workspace=ws, out=out)
        elif fused:
            kvq.decode_step(caches[0], kn, vn, q_last, bt, lens_d, maxlen, num_splits=args.num_splits,
                            workspace=ws, out=out)
        else:
            kvq.quantize_append(caches[0], kn, vn, last_slots)
            kvq.decode_attention(caches[0], q_last, bt, lens_d, maxlen, num_splits=args.num_splits, workspace=ws,
                                 out=out, reference=args.reference)
        torch.cuda.synchronize()
        mask_h = chunk_mask.cpu().numpy()
        out_h = out.cpu().numpy().astype(np.float64)
        worst = 0.0

        if windowed:
            seqs = [int(s) for s in np.linspace(0, B - 1, num=min(args.parity_seqs, B)).round()]
            for b in seqs:
                T = int(lens[b])
                unit = w.group_size if args.vgroup else 16  # pages hold whole value token groups
                P = int(math.ceil(T / unit) * unit)
                ref = oracle.Cache(d, Hkv, w.bits, w.group_size, w.hadamard_block, P, 1,
                                   quant_mode=cache.quant_mode, v_grouping=cache.v_grouping)
                k = wl.keys(w, b, 0, T, device=dev)
                v = wl.values(w, b, 0, T, device=dev)
                # prefill state, then the last two steps applied to this cache: each step
                # rewrites the same ring row and evicted slot (or completed group), so they
                # fix the final state
                rw = oracle.Window(d, Hkv, win_S, win_R, 1, residual=int(residual))
                if residual:
                    done = (T - 1) - (T - 1) % win_R
                    if done:
                        ref.append(wl.bf16_bits(k[:done]), wl.bf16_bits(v[:done]), np.arange(done))
                    win_tokens = list(range(done, T - 1))
                else:
                    lo, hi = win_S, T - 1 - win_R
                    if hi > lo:
                        ref.append(wl.bf16_bits(k[lo:hi]), wl.bf16_bits(v[lo:hi]), np.arange(lo, hi))
                    win_tokens = list(range(min(win_S, T - 1))) + list(range(max(win_S, T - 1 - win_R), T - 1))
                for t in win_tokens:
                    rw.k[0, window.row(t)] = wl.bf16_bits(k[t])
                    rw.v[0, window.row(t)] = wl.bf16_bits(v[t])
                ev = max(T - win_R, 0) if residual else max(T - 1 - win_R, 0)
                for j in applied0[-2:]:
                    kj, vj = news[j]
                    rw.append(ref, wl.bf16_bits(kj[b:b + 1]), wl.bf16_bits(vj[b:b + 1]), np.zeros(1, np.int32),
                              np.array([T - 1], np.int32), np.array([ev], np.int64))
                o = rw.decode(ref, wl.bf16_bits(q_last[b:b + 1]), np.zeros((1, 1), np.int32),
                              np.array([T], np.int32))
                worst = max(worst, float(np.max(np.abs(o[0] - out_h[b]))))
                del k, v
            parity = {"max_abs_err": worst, "tolerance": 2e-3, "sequences": seqs, "ok": worst <= 2e-3}
        else:
            # Oracle caches of single sequences (contiguous layout), built in host threads:
            # the oracle is C behind ctypes, which releases the GIL during each call.
            n_thr = host_threads()
            n1 = max(args.parity_seqs, 0 if args.no_cpu_baseline else args.cpu_sample_seqs)
            seqs1 = [int(s) for s in np.linspace(0, B - 1, num=min(max(n1, 1), B)).round()]
            seqsN = [] if args.no_cpu_baseline or n_thr < 2 else \
                [int(s) for s in np.linspace(0, B - 1, num=min(n_thr, B)).round()]
            jobs = seqs1 + [seqsN[i % len(seqsN)] for i in range(n_thr)] if seqsN else list(seqs1)
            rows = {}
            for b in sorted(set(jobs)):
                T = int(lens[b])
                # the same draw of T tokens the GPU cache was built from (slot T - 1 is then
                # rewritten by the step's token)
                k = wl.keys(w, b, 0, T, device=dev)
                v = wl.values(w, b, 0, T, device=dev)
                rows[b] = (wl.bf16_bits(k[:T - 1]), wl.bf16_bits(v[:T - 1]))
                del k, v

            def build_one(b):
                T = int(lens[b])
                ref = oracle.Cache(d, Hkv, w.bits, w.group_size, w.hadamard_block, int(math.ceil(T / 16) * 16), 1,
                                   quant_mode=cache.quant_mode, v_grouping=cache.v_grouping)
                ref.append(rows[b][0], rows[b][1], np.arange(T - 1))
                return ref

            tb = time.perf_counter()
            with cf.ThreadPoolExecutor(max_workers=max(n_thr, 1)) as ex:
                refs = list(ex.map(build_one, jobs))
            t_build = time.perf_counter() - tb
            rows.clear()
            kn_h, vn_h, q_h = wl.bf16_bits(kn), wl.bf16_bits(vn), wl.bf16_bits(q_last)

            def oracle_step(i):
                """One decode step of sequence jobs[i] on its own oracle cache: append the
                step's token, then fp64 decode of every query head of the sequence."""
                b = jobs[i]
                ref, T = refs[i], int(lens[b])
                ref.append(kn_h[b:b + 1], vn_h[b:b + 1], np.array([T - 1]))
                one = (np.zeros((1, 1), np.int32), np.array([T], np.int32))
                if args.prune:  # the oracle takes the kernel's choice of kept chunks
                    return ref.decode_pruned(q_h[b:b + 1], *one, mask_h[b:b + 1])[0]
                return ref.decode(q_h[b:b + 1], *one)[0]

            def step_bytes_of(b):
                return int(lens[b]) * Hkv * per_tok_head + Hq * d * 6 + Hkv * (2 * d * 2 + per_tok_head)

            # each timing is the median of cpu_repeats runs of the same steps (a repeat
            # appends the same token to the same slot again, then decodes)
            n_rep = 1 if args.no_cpu_baseline else max(1, args.cpu_repeats)
            # one thread, the first len(seqs1) jobs in turn
            reps1 = []
            for _ in range(n_rep):
                ts = time.perf_counter()
                outs1 = [oracle_step(i) for i in range(len(seqs1))]
                reps1.append(time.perf_counter() - ts)
            t1 = float(np.median(reps1))
            checked = list(zip(seqs1, outs1))
            # n_thr threads, one job each, all started together
            tN, outsN, repsN = None, [], []
            if seqsN:
                idx = list(range(len(seqs1), len(jobs)))
                for _ in range(n_rep):
                    ts = time.perf_counter()
                    with cf.ThreadPoolExecutor(max_workers=n_thr) as ex:
                        outsN = list(ex.map(oracle_step, idx))
                    repsN.append(time.perf_counter() - ts)
                tN = float(np.median(repsN))
                checked += list(zip(jobs[len(seqs1):], outsN))
            for b, o in checked:
                worst = max(worst, float(np.max(np.abs(o - out_h[b]))))
            if args.parity_seqs > 0:
                parity = {"max_abs_err": worst, "tolerance": 2e-3, "sequences": sorted({b for b, _ in checked}),
                          "ok": worst <= 2e-3}
            if not args.no_cpu_baseline:
                T0 = int(lens[seqs1[0]])
                bytes1 = sum(step_bytes_of(b) for b in seqs1)
                one = {"value": round(bytes1 / t1 / 1e9, 6), "unit": "GB/s", "threads": 1,
                       "sample": f"{len(seqs1)} sequences one after another, {t1:.1f}s (median of "
                                 f"{n_rep}: {', '.join(f'{x:.2f}' for x in reps1)} s)"}
                cpu = {"value": one["value"], "unit": "GB/s", "cores": 1, "kind": "oracle",
                       "sample": f"{len(seqs1)} of {B} sequences ({Hkv} kv heads, {Hq} q heads, T={T0}): oracle "
                                 f"append of the step's token + fp64 decode of every query head, one after another; "
                                 f"{t1:.1f}s timed, cache build {t_build:.1f}s untimed",
                       "threads_1": one}
                if tN is not None:
                    bytesN = sum(step_bytes_of(b) for b in jobs[len(seqs1):])
                    cpu.update({"value": round(bytesN / tN / 1e9, 6), "cores": n_thr,
                                "sample": f"{n_thr} sequence steps ({len(set(seqsN))} distinct of {B}; {Hkv} kv "
                                          f"heads, {Hq} q heads, T={T0}) on {n_thr} host threads at once, each the "
                                          f"unmodified oracle (append of the step's token + fp64 decode of every "
                                          f"query head) on its own sequence; {tN:.1f}s timed (median of {n_rep}: "
                                          f"{', '.join(f'{x:.2f}' for x in repsN)} s), cache build "
                                          f"{t_build:.1f}s untimed"})
                cpu.update(host_description())

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "us_per_step": round(ms * 1e3, 2),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"int{w.bits}-kv/bf16-qkv/f32-accum",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V with key outlier channels; no weights or datasets)",
        "config": {"workload": w.name, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": d,
                   "context": maxlen, "bits": w.bits, "group_size": w.group_size,
                   "hadamard_block": w.hadamard_block, "page_size": geo.page_size, "num_splits": num_splits,
                   # automatic split count with more than one sequence: one partition length for
                   # the batch, planned on the device from seq_lens (num_splits = the count for a
                   # max_seq_len sequence of a uniform batch)
                   "partitions": "balanced" if (args.num_splits == 0 and B > 1 and not args.reference)
                   else "fixed",
                   "kernel": "reference" if args.reference else "mfma", "layer_ring": ring,
                   # fused: kvq_decode_step (the append inside the split-K launch)
                   "step": "fused" if fused else "append+decode",
                   "settle_steps": n_settle,
                   "step_bytes": step_bytes, "quant_mode": cache.quant_mode, "v_grouping": cache.v_grouping,
                   **({"keep_chunks": args.prune, "chunks": n_chunks,
                       "kv_bits_capacity": round(per_tok_head * 8 / (2 * d), 4),
                       "kv_bits_bandwidth": round(kv_bytes * 8 / (2 * d * Hkv * int(lens.to(torch.int64).sum())), 4)}
                      if args.prune else {}),
                   **({"window_sink": win_S, "window_recent": win_R, "residual": int(residual)} if windowed else {})},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "stream": stream,
        "graph": graph,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
