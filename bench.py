#!/usr/bin/env python3
"""Benchmark of the hybrid-head sparse decode step on one MI355X.

A step is one pass of every layer of the workload (attention of retrieval and sparse
heads, argsTopK of the retrieval heads, S hand-over) for one decode token, with all
inputs already resident in HBM. Prints ONE JSON line (rank 0).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Metric: effective HBM GB/s of the step = algorithmic bytes / step time, where the
algorithmic bytes of a layer are
  sum over (b, KV group g): 2*N_b*d*2 if g serves a retrieval head, else
                            |union of the group's S rows|*2*d*2
  + Q and O (B*Hq*d*2 each) + S reads of sparse heads and S writes of retrieval
  heads (k_b*4 each).
The roofline object is for the attention kernel (the dominant kernel; it also merges
the splits and, unless a layer has too many retrieval rows, selects S): its algorithmic
bytes (KV + Q + O) per launch over its average launch duration, timed with HIP events
on the launch stream inside the timed steps, at the edges of the runs of layers whose
call is that one launch (no events between those layers). copy_gbs (a device copy, read + write bytes per second) and
read_gbs (a read-only reduction) are practical denominators beside the 8 TB/s figure.
With the default 32K workload the 128K workload runs too and is reported under "also".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, vendor figure


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b_32k")
    ap.add_argument("--split", type=int, default=0, help="rows per split = 256<<(v-1), 0 = auto")
    ap.add_argument("--waves", type=int, default=0, help="attention waves per workgroup: 1 = 4, 2 = 8, 0 = auto")
    ap.add_argument("--kv", choices=("bf16", "fp8"), default="bf16",
                    help="KV cache format: bf16, or 8-bit E4M3 codes (unit scales)")
    ap.add_argument("--block-select", action="store_true",
                    help="retrieval heads keep 64-token blocks by block maximum (HySparse form)")
    ap.add_argument("--swa-window", type=int, default=0,
                    help="HySparse: sparse layers add a gated sliding-window branch over their own "
                         "cache of this many tokens (workloads whose sparse layers share the first "
                         "layer's cache)")
    ap.add_argument("--page-size", type=int, default=0,
                    help="paged KV: rows per page (power of two, 16..4096); 0 = contiguous")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--also", default="auto",
                    help="further workloads (comma list) reported in the same line; auto = the 128K "
                         "configuration with the default 32K run; none = no further workload")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-kernel-pass", action="store_true", help="omit the roofline object")
    ap.add_argument("--layers-detail", action="store_true", help="print per-layer times to stderr")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration under rocprofv3)")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn rocprofv3 FETCH_SIZE/WRITE_SIZE counter files into the traffic summary")
    ap.add_argument("--counter-commands", default="", help="commands that produced the counter files")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="mean k_attention duration from a rocprofv3 kernel trace, over all dispatches "
                         "and over those not followed by a selection launch (the bench's timed ones)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layer_bytes(w, l, S_in, d, kv_elem=2):
    """Algorithmic bytes of layer l given S^{l} (dict {(b,h): indices}) -> (attention, total).
    kv_elem: bytes per K/V element (2 for bf16, 1 for E4M3 codes)."""
    B, Hq, Hkv = w.batch, w.num_q_heads, w.num_kv_heads
    G = Hq // Hkv
    mask = w.retrieval_masks[l]
    kv = 0
    for b in range(B):
        n = w.seq_lens[b]
        for g in range(Hkv):
            heads = range(g * G, (g + 1) * G)
            if any(mask >> h & 1 for h in heads):
                kv += 2 * n * d * kv_elem
            else:
                u = np.unique(np.concatenate([S_in[(b, h)] for h in heads]))
                kv += int(u.size) * 2 * d * kv_elem
    qo = 2 * B * Hq * d * 2
    s_io = 0
    for b in range(B):
        kb = min(w.k_per_seq[b], w.seq_lens[b])
        for h in range(Hq):
            s_io += kb * 4
    return kv + qo, kv + qo + s_io


# the attention kernel's translation unit: its source and the headers it includes
ATTN_SOURCES = [os.path.join(ROOT, "hybrid_head_sparse_retrieval_amd", "csrc", f)
                for f in ("ld_attention.hip", "ld_device.h", "ld_internal.h")]
COPY_BYTES = 1 << 30


def source_hash(paths=ATTN_SOURCES):
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"k_attention_{workload}_traffic.json")


def copy_calibration():
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copied {COPY_BYTES} bytes 3 times")


def paged_inputs(torch, w, inputs, page):
    """The same layers with K/V moved into pools of `page`-row pages in a seeded random
    order: (q, k_pool, v_pool, block_table, page) per layer."""
    offs = w.kv_offsets()
    B = w.batch
    npp = [(int(offs[b + 1] - offs[b]) + page - 1) // page for b in range(B)]
    pps, total = max(npp), sum(npp)
    rng = np.random.default_rng(12345)
    out, cache = [], {}
    for l, (q, kc, vc) in enumerate(inputs):
        key = (kc.data_ptr(), vc.data_ptr())
        if key not in cache:
            perm = rng.permutation(total)
            Hkv, T, d = kc.shape
            kp = torch.zeros((Hkv, total * page, d), dtype=kc.dtype, device=kc.device)
            vp = torch.zeros_like(kp)
            bt = np.zeros((B, pps), dtype=np.int32)
            j = 0
            for b in range(B):
                for i in range(npp[b]):
                    pid = int(perm[j]); j += 1
                    bt[b, i] = pid
                    r0 = int(offs[b]) + i * page
                    r1 = min(int(offs[b + 1]), r0 + page)
                    kp[:, pid * page: pid * page + r1 - r0] = kc[:, r0:r1]
                    vp[:, pid * page: pid * page + r1 - r0] = vc[:, r0:r1]
            cache[key] = (kp, vp, torch.as_tensor(bt, device=kc.device))
        kp, vp, bt = cache[key]
        out.append((q, kp, vp, bt, page))
    return out


def copy_bandwidth(torch, reps=5):
    """Device-to-device copy of COPY_BYTES, read plus write bytes per second (GB/s): the
    practical bandwidth of a plain stream, reported beside the 8 TB/s figure."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2.0 * COPY_BYTES / (ms * 1e-3) / 1e9


READ_BYTES = 4 << 30


def read_bandwidth(torch, reps=5):
    """A read-only stream: the sum of READ_BYTES of fp64 zeros (a reduction that writes a
    few bytes; the fastest of torch's reductions measured on this device), bytes read per
    second (GB/s): a practical ceiling of a read-dominated kernel, beside the 8 TB/s."""
    x = torch.zeros(READ_BYTES // 8, dtype=torch.float64, device="cuda")
    for _ in range(2):
        x.sum()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        x.sum()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del x
    return READ_BYTES / (ms * 1e-3) / 1e9


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _counter_per_dispatch(csv_path, name_part, counter):
    """Mean value per dispatch of `counter` over dispatches whose kernel name holds
    name_part; for the attention kernel, only dispatches not followed by a selection
    launch (the launches the bench's roofline times)."""
    import csv
    vals, names = {}, {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            key = int(r["Dispatch_Id"])
            names[key] = r["Kernel_Name"]
            if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    ids = sorted(names)
    nxt = {a: names[b] for a, b in zip(ids, ids[1:])}
    if name_part == "k_attention":
        vals = {key: v for key, v in vals.items() if "k_sel" not in nxt.get(key, "")}
    return (sum(vals.values()) / len(vals), len(vals)) if vals else (None, 0)


def summarize_counters(args):
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.summarize_counters
    fk, nd = _counter_per_dispatch(fetch_csv, "k_attention", "FETCH_SIZE")
    wk, _ = _counter_per_dispatch(write_csv, "k_attention", "WRITE_SIZE")
    cf, _ = _counter_per_dispatch(cfetch_csv, "copy", "FETCH_SIZE")
    cw, _ = _counter_per_dispatch(cwrite_csv, "copy", "WRITE_SIZE")
    f_factor = cf * 1024.0 / COPY_BYTES      # counter KiB of a known-size copy over its bytes
    w_factor = cw * 1024.0 / COPY_BYTES
    fetch_b = fk * 1024.0 / f_factor
    write_b = wk * 1024.0 / w_factor
    out = {"kernel": "k_attention", "workload": args.workload, "dispatches": nd,
           "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
           "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1), "copy_bytes": COPY_BYTES,
           "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
           "traffic_bytes_per_launch": int(fetch_b + write_b),
           "fetch_bytes_per_launch": int(fetch_b), "write_bytes_per_launch": int(write_b),
           "source_sha256_16": source_hash(), "commands": args.counter_commands}
    os.makedirs(os.path.dirname(traffic_path(args.workload)), exist_ok=True)
    with open(traffic_path(args.workload), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def load_traffic(workload):
    """Measured HBM bytes per attention launch, or None when absent or taken on other code."""
    try:
        with open(traffic_path(workload)) as f:
            t = json.load(f)
    except OSError:
        return None
    return t["traffic_bytes_per_launch"] if t.get("source_sha256_16") == source_hash() else None


def summarize_trace(path):
    import csv
    with open(path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    alone, before_sel = [], []
    for i, r in enumerate(rows):
        if "k_attention" not in r["Kernel_Name"]:
            continue
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        nxt = rows[i + 1]["Kernel_Name"] if i + 1 < len(rows) else ""
        (before_sel if "k_sel" in nxt else alone).append(us)
    out = {"kernel": "k_attention", "dispatches": len(alone) + len(before_sel),
           "avg_us_all": round(float(np.mean(alone + before_sel)), 2) if alone or before_sel else None,
           "dispatches_alone": len(alone), "avg_us_alone": round(float(np.mean(alone)), 2) if alone else None,
           "dispatches_before_selection": len(before_sel),
           "avg_us_before_selection": round(float(np.mean(before_sel)), 2) if before_sel else None}
    print(json.dumps(out))


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)
    import torch
    import hybrid_head_sparse_retrieval_amd as ld
    from hybrid_head_sparse_retrieval_amd.step import DecodeStep
    import workloads as wl

    ld.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload in TSA_WORKLOADS:
        tsa_bench(args, torch, ld, dev)
        return
    if args.workload in PREFILL_WORKLOADS:
        prefill_bench(args, torch, ld, dev)
        return
    result = decode_bench(args, torch, ld, DecodeStep, wl, dev, args.workload, not args.no_cpu_baseline)
    also = default_also(args) if args.also == "auto" else [x for x in args.also.split(",") if x and x != "none"]
    if also:
        # further workloads of the same metric, run after the first one (its inputs freed),
        # with the same steps; only their headline figures are kept here
        result["also"] = {}
        for name in also:
            r = decode_bench(args, torch, ld, DecodeStep, wl, dev, name, False)
            result["also"][name] = {key: r[key] for key in ALSO_KEYS if key in r}
    print(json.dumps(result), flush=True)


# headline figures of the further workloads in the one JSON line
ALSO_KEYS = ("value", "unit", "ms_per_step", "us_per_layer", "pct_of_hbm_peak", "pct_of_read",
             "us_layer0", "us_layers_with_retrieval", "us_layers_sparse_only", "algorithmic_bytes_per_step",
             "roofline", "config")


def default_also(args):
    """The 128K configuration of the same metric rides along with the default 32K run
    (plain launch shape, bf16 contiguous KV, token selection)."""
    plain = (args.kv == "bf16" and not args.page_size and not args.block_select and not args.swa_window
             and not args.split and not args.waves)
    return ["qwen3_8b_128k"] if args.workload == "llama3_8b_32k" and plain else []


def decode_bench(args, torch, ld, DecodeStep, wl, dev, name, cpu_leg):
    """Time one decode-step workload; returns its result object."""
    w = wl.get_workload(name)
    L, d = w.layers, w.head_dim
    log(f"[bench] workload {w.name}: B={w.batch} L={L} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"d={d} N={w.seq_lens if w.batch > 1 else w.seq_lens[0]} k={w.k_per_seq if w.batch > 1 else w.k_per_seq[0]}")

    # ---- inputs resident in HBM
    t0 = time.time()
    inputs = []
    for l in range(L):
        x = wl.make_layer_inputs(w, l, device=dev)
        if w.shared_kv_from_layer0 and l > 0:
            inputs.append((x.q, inputs[0][1], inputs[0][2]))
        else:
            inputs.append((x.q, x.k, x.v))
    torch.cuda.synchronize()
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s "
        f"({sum(t.numel() * 2 for t in (inputs[0][1], inputs[0][2])) * w.kv_layers() / 1e9:.2f} GB KV)")

    logical = inputs
    kv_elem = 2
    if args.kv == "fp8":
        # E4M3 codes of the same draws (round to nearest even); the oracle leg keeps bf16
        cache = {}
        q8 = []
        for (q, kc, vc) in inputs:
            key = (kc.data_ptr(), vc.data_ptr())
            if key not in cache:
                cache[key] = (kc.float().to(torch.float8_e4m3fn).view(torch.uint8),
                              vc.float().to(torch.float8_e4m3fn).view(torch.uint8))
            q8.append((q,) + cache[key])
        inputs, kv_elem = q8, 1
        log("[bench] KV cache as E4M3 codes (unit scales)")
    if args.page_size:
        inputs = paged_inputs(torch, w, inputs, args.page_size)
        log(f"[bench] paged KV: {args.page_size}-row pages in a shuffled pool")

    split_flag = ld.flag_split_rows(args.split) | ld.flag_waves(args.waves)
    if args.block_select:
        if any(k % 64 for k in w.k_per_seq) or any(n % 64 for n in w.seq_lens) or w.batch > 1:
            log("[bench] --block-select needs one sequence with k and N multiples of 64")
            sys.exit(2)
        split_flag |= ld.FLAG_BLOCK_SELECT
    windows = None
    W = args.swa_window
    if W:
        if not w.shared_kv_from_layer0 or w.ragged_csr or not 1 <= W <= 4096 \
                or any(w.retrieval_masks[1:]):
            log("[bench] --swa-window needs a workload whose later layers are sparse layers on the "
                "first layer's cache, dense S and 1 <= W <= 4096")
            sys.exit(2)
        windows = [None]
        gen = torch.Generator(device="cpu")
        for l in range(1, L):
            gen.manual_seed(wl.stream_seed("window", w.name, l))
            kw = torch.randn((w.num_kv_heads, w.batch * W, d), generator=gen).to(torch.bfloat16).to(dev)
            vw = torch.randn((w.num_kv_heads, w.batch * W, d), generator=gen).to(torch.bfloat16).to(dev)
            gate = torch.randn((w.batch, w.num_q_heads), generator=gen).to(dev)
            windows.append((kw, vw, gate))
        log(f"[bench] sparse layers add a {W}-token window branch and a sigmoid gate")
    step = DecodeStep(w.batch, w.num_q_heads, w.num_kv_heads, d, w.seq_lens, w.k_per_seq,
                      w.retrieval_masks, csr=w.ragged_csr, device=dev, split_flag=split_flag,
                      window_len=W)

    # ---- accounting pass (untimed): S before every layer -> algorithmic bytes
    attn_bytes, total_bytes = [], []
    for l in range(L):
        S_in = step.s_rows() if l > 0 else None
        q, kc, vc = inputs[l][:3]
        win = windows[l] if windows else None
        if len(inputs[l]) > 3:
            step.layer(l, q, kc, vc, block_table=inputs[l][3], page_size=inputs[l][4], window=win)
        else:
            step.layer(l, q, kc, vc, window=win)
        a, t = layer_bytes(w, l, S_in, d, kv_elem) if l > 0 else layer_bytes(w, l, None, d, kv_elem)
        if win is not None:   # the window cache and the gate
            extra = 2 * w.num_kv_heads * w.batch * W * d * 2 + w.batch * w.num_q_heads * 4
            a, t = a + extra, t + extra
        attn_bytes.append(a)
        total_bytes.append(t)
    torch.cuda.synchronize()
    step_bytes = float(sum(total_bytes))
    log(f"[bench] algorithmic bytes/step {step_bytes / 1e9:.3f} GB")

    # ---- which layer calls are exactly one attention launch (merge and selection inside
    # it): the roofline times those launches inside the timed steps
    plans = []
    for l in range(L):
        q, kc, vc = inputs[l][:3]
        win = windows[l] if windows else None
        extra = {"block_table": inputs[l][3], "page_size": inputs[l][4]} if len(inputs[l]) > 3 else {}
        plans.append(step.plan(l, q, kc, vc, window=win, **extra))
    single = [l for l in range(L) if plans[l] is not None and plans[l]["launches"] == 1]
    # runs [a, b) of consecutive single-launch layers: an event before a and one before b
    runs, l = [], 0
    while l < L:
        if l in single:
            a = l
            while l < L and l in single:
                l += 1
            runs.append((a, l))
        else:
            l += 1

    # ---- warmup + timed steps (events between steps, on the launch stream)
    for _ in range(args.warmup):
        step.run(inputs, windows=windows)
    torch.cuda.synchronize()
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    # per step, events at the edges of the single-launch runs (none between their layers;
    # an edge at layer 0 or L reuses the step events)
    rev = []
    for i in range(args.steps):
        ev = [None] * (L + 1)
        for a, b in runs:
            for e in (a, b):
                if e not in (0, L) and ev[e] is None:
                    ev[e] = torch.cuda.Event(enable_timing=True)
        rev.append(ev)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    sev[0].record()
    for i in range(args.steps):
        step.run(inputs, windows=windows, events=rev[i])
        sev[i + 1].record()
    torch.cuda.synchronize()

    def edge(i, e):
        return sev[i] if e == 0 else (sev[i + 1] if e == L else rev[i][e])
    single_ms = sum(edge(i, a).elapsed_time(edge(i, b)) for i in range(args.steps) for a, b in runs)
    wall = time.perf_counter() - wall0
    per_step = np.array([sev[i].elapsed_time(sev[i + 1]) for i in range(args.steps)])
    ms_step = sev[0].elapsed_time(sev[-1]) / args.steps
    log(f"[bench] {args.steps} steps: {ms_step * 1e3:.1f} us/step (wall {wall / args.steps * 1e6:.1f} us/step; "
        f"p10 {np.percentile(per_step, 10) * 1e3:.1f}, p50 {np.median(per_step) * 1e3:.1f}, "
        f"p90 {np.percentile(per_step, 90) * 1e3:.1f} us)")

    # ---- the same step captured once in a HIP graph and replayed
    ms_graph = None
    try:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            step.run(inputs, windows=windows)           # eager pass on the capture stream first
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=cap):
                step.run(inputs, windows=windows)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        gev0, gev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gev0.record()
        for _ in range(args.steps):
            g.replay()
        gev1.record()
        torch.cuda.synchronize()
        ms_graph = gev0.elapsed_time(gev1) / args.steps
        log(f"[bench] graph replay: {ms_graph * 1e3:.1f} us/step")
        del g
    except Exception as e:  # capture is a secondary figure; report and go on
        log(f"[bench] graph capture unavailable: {e}")

    # ---- per-layer times inside full steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(L + 1)]
    reps = 5

    pre = torch.cuda.Event(enable_timing=True)
    spans = []
    for rep in range(reps + 1):
        # a GPU-side wait while the host queues the step, so no layer waits for the host;
        # the first pass is a warm-up (its first layer has been seen to take tens of ms)
        pre.record()
        torch.cuda._sleep(4_000_000)
        step.run(inputs, events=evs, windows=windows)
        torch.cuda.synchronize()
        span = np.array([evs[l].elapsed_time(evs[l + 1]) for l in range(L)]) * 1e3
        if args.layers_detail:
            log(f"[bench] per-layer pass {rep}: wait {pre.elapsed_time(evs[0]):.3f} ms, "
                f"layer 0 {span[0]:.1f} us, layer 1 {span[1]:.1f} us")
        if rep > 0:
            spans.append(span)
    per_layer = np.median(np.array(spans), axis=0)
    if args.layers_detail:
        for l in range(L):
            log(f"  layer {l:2d} mask={w.retrieval_masks[l]:#x} {per_layer[l]:8.1f} us "
                f"{total_bytes[l] / per_layer[l] / 1e3:8.1f} GB/s")

    # ---- roofline of the attention launch: the layers whose call is that one launch run
    # back to back inside the timed steps, bracketed by the events above, so their mean
    # span is the launch's duration as the device runs it in a step (the next launch's
    # dispatch overlaps the previous one's end)
    roof = None
    if not args.no_kernel_pass and single:
        avg_us = single_ms * 1e3 / (args.steps * len(single))
        avg_bytes = float(np.mean([attn_bytes[l] for l in single]))
        achieved = avg_bytes / (avg_us * 1e-6) / 1e9
        # the counters are taken on the default configuration (bf16 contiguous KV, token
        # selection, automatic launch shape); other configurations report none
        default_cfg = (args.kv == "bf16" and not args.page_size and not args.block_select and not W
                       and not args.split and not args.waves)
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": load_traffic(w.name) if default_cfg else None,
                "kernel": f"k_attention (d={d}, G={w.group_size}, {'E4M3' if args.kv == 'fp8' else 'bf16'} KV)",
                "avg_launch_us": round(avg_us, 2), "avg_bytes_per_launch": int(avg_bytes),
                "launches_timed": len(single) * args.steps,
                "layers_timed": f"{len(single)} of {L} (calls that are one attention launch)",
                "timing": "HIP events on the launch stream at the edges of those layers inside the timed steps"}
        log(f"[bench] attention launch: avg {avg_us:.2f} us over {len(single)} layers x {args.steps} steps, "
            f"{achieved:.0f} GB/s ({achieved / HBM_PEAK_GBS * 100:.1f}% of peak)")

    value = step_bytes / (ms_step * 1e-3) / 1e9
    wait_ok = True
    try:
        step.workspace.check()
    except ld.LycheeDecodeError as e:
        wait_ok = False
        log(f"[bench] {e}")
    copy_gbs = copy_bandwidth(torch)
    read_gbs = read_bandwidth(torch)
    log(f"[bench] device copy: {copy_gbs:.0f} GB/s (read + write); read-only reduction: {read_gbs:.0f} GB/s")
    nonzero = [l for l in range(1, L) if w.retrieval_masks[l]]
    zero = [l for l in range(1, L) if not w.retrieval_masks[l]]
    result = {
        "metric": "hybrid-head decode attention effective HBM GB/s (us/layer, us/step alongside)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_p10_p50_p90": [round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)],
        "ms_per_step_graph": round(ms_graph, 4) if ms_graph else None,
        "us_per_layer": round(ms_step * 1e3 / L, 2),
        "pct_of_hbm_peak": round(value / HBM_PEAK_GBS * 100, 2),
        "copy_gbs": round(copy_gbs, 1),
        "pct_of_copy": round(value / copy_gbs * 100, 2),
        "read_gbs": round(read_gbs, 1),
        "pct_of_read": round(value / read_gbs * 100, 2),
        "us_layer0": round(float(per_layer[0]), 2),
        "us_layers_with_retrieval": round(float(np.mean(per_layer[nonzero])), 2) if nonzero else None,
        "us_layers_sparse_only": round(float(np.mean(per_layer[zero])), 2) if zero else None,
        "algorithmic_bytes_per_step": int(step_bytes),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.kv == "bf16" else "bf16 q, e4m3 kv",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "layers": L, "q_heads": w.num_q_heads,
                   "kv_heads": w.num_kv_heads, "head_dim": d,
                   "seq_len": w.seq_lens[0] if w.batch == 1 else list(w.seq_lens),
                   "k": w.k_per_seq[0] if w.batch == 1 else list(w.k_per_seq),
                   "retrieval_heads_after_layer0": sum(bin(m).count("1") for m in w.retrieval_masks[1:]),
                   "split_rows": "auto" if args.split == 0 else 256 << (args.split - 1),
                   "kv_layout": f"paged {args.page_size}-row pages" if args.page_size else "contiguous",
                   "kv_format": args.kv,
                   "selection": "64-token blocks" if args.block_select else "tokens",
                   "swa_window": W or None},
        "roofline": roof,
        # sparse layers that read the first layer's cache again may be served from the
        # 256 MB last-level cache, so their GB/s can exceed the HBM figure
        "cache_served": bool(w.shared_kv_from_layer0),
        "device_waits_ok": wait_ok,
        "cpu_baseline": None,
    }

    # ---- CPU oracle baseline on a bounded sample of the same workload
    if W and cpu_leg:
        log("[bench] no CPU baseline with --swa-window (the oracle leg times the plain layers)")
    elif cpu_leg:
        oracle_inputs = logical if args.kv == "bf16" else q8
        result["cpu_baseline"] = cpu_baseline(w, oracle_inputs, total_bytes, args.cpu_seconds, ms_step)
    del inputs, logical, step
    torch.cuda.empty_cache()
    return result


# Token Sparse Attention over a prefill (the page's budget range of 512-1024 kept tokens
# per head, at its 128K context), Llama-3-8B head layout, causal, with the residual form
# of the scatter (unselected rows keep what the caller wrote, so no zero fill).
# The page's form has no mask (every kept token attends to every kept token); the causal
# form (a kept token sees the kept tokens at or before it) is timed beside it.
TSA_WORKLOADS = {
    "tsa_llama3_8b_128k": dict(B=1, Hq=32, Hkv=8, d=128, T=131072, k=1024, causal=False),
}
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, vendor figure


def tsa_bench(args, torch, ld, dev):
    """Time the Token Sparse Attention layer call (selection + dense stage) and the
    dense stage alone (sets given), report the dense kernel against the matrix-core
    roofline, and time the oracle on a few heads."""
    import workloads as wl
    c = TSA_WORKLOADS[args.workload]
    B, Hq, Hkv, d, T, k, causal = c["B"], c["Hq"], c["Hkv"], c["d"], c["T"], c["k"], c["causal"]
    kk = min(k, T)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.stream_seed("tsa", args.workload))
    q = torch.randn((Hq, B * T, d), generator=gen, device=dev).to(torch.bfloat16)
    kc = torch.randn((Hkv, B * T, d), generator=gen, device=dev).to(torch.bfloat16)
    vc = torch.randn((Hkv, B * T, d), generator=gen, device=dev).to(torch.bfloat16)
    scores = torch.randn((B, Hq, T), generator=gen, device=dev)
    out = torch.zeros_like(q)
    idx = torch.empty((B, Hq, kk), dtype=torch.int32, device=dev)
    ws = ld.TsaWorkspace(ld.tsa_shape(q, kc, B), k, dev)
    log(f"[bench] {args.workload}: B={B} Hq={Hq} Hkv={Hkv} d={d} T={T} k={k} causal={causal}")

    def layer(causal=causal):
        ld.tsa_attention(q, kc, vc, scores, k, idx_out=idx, out=out, causal=causal, zero_fill=False, workspace=ws)

    def dense(causal=causal):
        ld.tsa_attention(q, kc, vc, None, k, idx_out=idx, out=out, causal=causal, zero_fill=False, workspace=ws,
                         given_idx=True, batch=B)

    def timed(fn, n):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3   # us

    us_layer = timed(layer, args.steps)
    us_dense = timed(dense, args.steps)

    def dense_flops(c):
        # matrix work of the dense stage: 2 d flops for q.k and 2 d for p.v per allowed pair
        return 4.0 * d * B * Hq * (kk * (kk + 1) // 2 if c else kk * kk)

    flops = dense_flops(causal)
    tflops = flops / (us_dense * 1e-6) / 1e12
    # the other form, timed the same way
    other = not causal
    us_layer_o = timed(lambda: layer(other), args.steps)
    us_dense_o = timed(lambda: dense(other), args.steps)
    tflops_o = dense_flops(other) / (us_dense_o * 1e-6) / 1e12
    # bytes the layer must move: the scores, the kept rows of q, k, v (k, v once per KV
    # group's union of kept rows) and the scattered output rows
    idx_h = idx.cpu().numpy()
    G = Hq // Hkv
    kv_rows = sum(np.unique(idx_h[b, g * G:(g + 1) * G]).size for b in range(B) for g in range(Hkv))
    layer_bytes_ = scores.numel() * 4 + Hq * B * kk * d * 2 * 2 + kv_rows * d * 2 * 2 + idx_h.size * 4
    log(f"[bench] layer {us_layer:.1f} us, dense stage {us_dense:.1f} us = {tflops:.1f} TFLOP/s; "
        f"{'causal' if other else 'unmasked'} form: layer {us_layer_o:.1f} us, dense {us_dense_o:.1f} us = "
        f"{tflops_o:.1f} TFLOP/s")
    result = {
        "metric": "token-sparse prefill attention layer time (select + dense + scatter)",
        "value": round(us_layer, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_layer / 1e3, 4),
        "us_dense_stage": round(us_dense, 2),
        "us_selection": round(us_layer - us_dense, 2),
        "algorithmic_bytes_per_layer": int(layer_bytes_),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "seq_len": T, "k": k, "causal": causal, "scatter": "residual (no zero fill)"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": f"k_tsa (d={d})", "avg_launch_us": round(us_dense, 2),
                     "flops_per_launch": int(flops), "launches_timed": args.steps},
        "cpu_baseline": None,
        ("causal_form" if other else "unmasked_form"): {
            "us_layer": round(us_layer_o, 2), "us_dense_stage": round(us_dense_o, 2),
            "tflops_dense": round(tflops_o, 1), "frac_dense": round(tflops_o / MFMA_BF16_PEAK_TFLOPS, 4),
            "flops_per_launch": int(dense_flops(other))},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = tsa_cpu_baseline(q, kc, vc, scores, k, causal, us_layer, args.cpu_seconds)
    print(json.dumps(result), flush=True)


# The hybrid-head layer over a causal prompt (the prefill extension of the recurrence):
# Llama-3-8B head layout, one 32K prompt, k = 30 % of it; a full layer (every head
# retrieves) followed by a layer with two seeded retrieval heads and a sparse-only one.
PREFILL_WORKLOADS = {
    "prefill_llama3_8b_32k": dict(B=1, Hq=32, Hkv=8, d=128, T=32768, layers=3, per_layer=2),
}


def prefill_flops(masks, S_rows, T, d):
    """Matrix flops of one prefill layer per mask: causal q.k and p.v of retrieval rows
    (4 d per visible pair), the q.k of their column sums (2 d per visible pair), and the
    q.k and p.v of sparse rows over their visible set tokens (a token at position s is
    visible to T - s rows). -> (attention flops, column-sum flops)"""
    pairs = T * (T + 1) // 2
    attn, col = 0, 0
    for h, row in enumerate(S_rows):
        if masks >> h & 1:
            attn += 4 * d * pairs
            col += 2 * d * pairs
        else:
            attn += 4 * d * int(np.sum(T - row.astype(np.int64)))
    return attn, col


def prefill_bench(args, torch, ld, dev):
    """Time each prefill layer of the workload (attention, column sums and selection)
    and the attention launch alone (LD_FLAG_SKIP_TOPK), report the attention kernel
    against the matrix-core roofline, and time the oracle on the first tokens."""
    import workloads as wl
    c = PREFILL_WORKLOADS[args.workload]
    B, Hq, Hkv, d, T, L = c["B"], c["Hq"], c["Hkv"], c["d"], c["T"], c["layers"]
    k = int(0.3 * T)
    masks = wl.seeded_masks(wl.stream_seed("prefill-masks", args.workload) % 1000, L, Hq, c["per_layer"])
    masks[-1] = 0
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.stream_seed("prefill", args.workload))
    layers = []
    for _ in range(L):
        layers.append(tuple(torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
                            for shape in ((Hq, B * T, d), (Hkv, B * T, d), (Hkv, B * T, d))))
    S = torch.empty((B, Hq, k), dtype=torch.int32, device=dev)
    out = torch.empty_like(layers[0][0])
    shape = ld.tsa_shape(layers[0][0], layers[0][1], B)
    ws = ld.PrefillWorkspace(shape, k, dev)
    log(f"[bench] {args.workload}: B={B} Hq={Hq} Hkv={Hkv} d={d} T={T} k={k} masks={[hex(m) for m in masks]}")

    def run_layer(l, flags=0):
        q, kc, vc = layers[l]
        ld.prefill_hybrid_layer(q, kc, vc, masks[l], k, S if l else None, batch=B, s_out=S, out=out,
                                flags=flags, workspace=ws)

    # S before every layer (the accounting pass) -> flops
    flops = []
    for l in range(L):
        S_rows = S.cpu().numpy()[0] if l else np.zeros((Hq, k), dtype=np.int32)
        flops.append(prefill_flops(masks[l], S_rows, T, d))
        run_layer(l)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(L + 1)]

    def timed_steps(n, flags=0):
        spans = []
        for rep in range(n + args.warmup):
            ev[0].record()
            for l in range(L):
                run_layer(l, flags)
                ev[l + 1].record()
            torch.cuda.synchronize()
            if rep >= args.warmup:
                spans.append([ev[l].elapsed_time(ev[l + 1]) * 1e3 for l in range(L)])
        return np.median(np.array(spans), axis=0)        # us per layer

    reps = max(3, args.steps // 4)
    us_layer = timed_steps(reps)
    us_attn = timed_steps(reps, ld.FLAG_SKIP_TOPK)        # the attention launch alone (the S
    # buffer is left as the full steps wrote it, so the sparse layers keep their sets)
    tf_attn = [flops[l][0] / (us_attn[l] * 1e-6) / 1e12 for l in range(L)]
    for l in range(L):
        log(f"[bench] layer {l} mask={masks[l]:#x}: {us_layer[l]:.0f} us (attention alone {us_attn[l]:.0f} us, "
            f"{tf_attn[l]:.0f} TFLOP/s)")
    total_flops = float(sum(a + cc for a, cc in flops))
    us_total = float(np.sum(us_layer))
    result = {
        "metric": "hybrid-head prefill layer time (attention + column sums + selection)",
        "value": round(us_total / L, 1),
        "unit": "us",
        "n_gpus": 1,
        "steps": reps,
        "warmup": args.warmup,
        "ms_per_step": round(us_total / 1e3, 4),
        "us_per_layer": [round(float(x), 1) for x in us_layer],
        "us_attention_per_layer": [round(float(x), 1) for x in us_attn],
        "tflops_attention_per_layer": [round(float(x), 1) for x in tf_attn],
        "tflops_step": round(total_flops / (us_total * 1e-6) / 1e12, 1),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "prompt_len": T, "k": k, "layers": L, "retrieval_masks": [hex(m) for m in masks]},
        "roofline": {"bound": "mfma", "achieved": round(tf_attn[0], 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf_attn[0] / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": f"k_prefill_attn (d={d}, every head retrieving)",
                     "avg_launch_us": round(float(us_attn[0]), 2), "flops_per_launch": int(flops[0][0]),
                     "launches_timed": reps},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = prefill_cpu_baseline(layers[0], B, T, k, masks[0], us_layer[0], args.cpu_seconds)
    print(json.dumps(result), flush=True)


def prefill_cpu_baseline(layer, B, T, k, mask, gpu_us, target_s):
    """The oracle's prefill layer on the first Tp tokens of the prompt (Tp doubled from
    256 while the run stays under about target_s / 4 seconds), scaled to T by (T/Tp)^2
    (the layer's work is quadratic in the prompt length)."""
    from oracle import lychee_oracle as orc
    import workloads as wl
    q, kc, vc = layer
    Hq = q.shape[0]
    ret = [bool(mask >> h & 1) for h in range(Hq)]
    Tp, spent, cpu = 256, 0.0, 0.0
    while True:
        qs = orc.bf16_bits_to_f64(wl.bf16_bits(q[:, :Tp]))
        ks = orc.bf16_bits_to_f64(wl.bf16_bits(kc[:, :Tp]))
        vs = orc.bf16_bits_to_f64(wl.bf16_bits(vc[:, :Tp]))
        t0, c0 = time.perf_counter(), time.process_time()
        orc.prefill_hybrid_layer(qs, ks, vs, 1, ret, max(1, int(0.3 * Tp)))
        spent, cpu = time.perf_counter() - t0, time.process_time() - c0
        log(f"[bench] oracle prefill layer at {Tp} tokens: {spent:.1f}s")
        if spent * 4 * 4 > target_s or Tp * 2 > T:
            break
        Tp *= 2
    est_us = spent * (T / Tp) ** 2 * 1e6
    return {"value": round(est_us, 1), "unit": "us", "cores": round(cpu / spent, 1), "kind": "oracle",
            "cpu_model": _cpu_model(), "gpu_speedup": round(est_us / gpu_us, 1),
            "sample": f"the oracle's layer over the first {Tp} of {T} prompt tokens ({Hq} heads, mask {mask:#x}), "
                      f"{spent:.1f} s wall, scaled by (T/{Tp})^2"}


def tsa_cpu_baseline(q, kc, vc, scores, k, causal, us_layer, target_s):
    """The oracle on the first heads of the layer (one sequence) until about target_s
    seconds of CPU work, scaled to the whole layer."""
    from oracle import lychee_oracle as orc
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    Hq, BT, d = q.shape
    Hkv = kc.shape[0]
    G = Hq // Hkv
    B, _, T = scores.shape
    spent, cpu, heads = 0.0, 0.0, 0
    while spent < target_s:      # passes over the heads until about target_s of CPU work
        for h in range(Hq):
            g = h // G
            qh = orc.bf16_bits_to_f64(wl.bf16_bits(q[h:h + 1, :T]))
            kh = orc.bf16_bits_to_f64(wl.bf16_bits(kc[g:g + 1, :T]))
            vh = orc.bf16_bits_to_f64(wl.bf16_bits(vc[g:g + 1, :T]))
            sh = scores[0:1, h:h + 1].cpu().numpy()
            t0, c0 = time.perf_counter(), time.process_time()
            orc.tsa_attention(qh, kh, vh, sh, k, causal=causal, zero_fill=False)
            spent += time.perf_counter() - t0
            cpu += time.process_time() - c0
            heads += 1
            log(f"[bench] oracle head {h}: cumulative {spent:.1f}s")
            if spent >= target_s:
                break
    per_layer_us = spent / heads * (B * Hq) * 1e6
    return {"value": round(per_layer_us, 1), "unit": "us", "cores": round(cpu / spent, 1),
            "threads_available": int(threads), "kind": "oracle",
            "cpu_model": _cpu_model(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "sample": f"{heads} head evaluations (sequence 0; {heads / (B * Hq):.2f} layers of {B * Hq} heads), "
                      f"fp64 NumPy oracle, {spent:.1f} s, scaled to one layer"}


def cpu_baseline(w, inputs, total_bytes, target_s, gpu_ms_step):
    """Time the fp64 oracle (as it stands) on the first layers of the step until about
    target_s seconds of CPU work; report GB/s of algorithmic bytes processed, the
    oracle's ms per layer and per step (scaled from the sample's layer mix), and the
    cores it kept busy (process CPU time over wall time)."""
    from oracle import lychee_oracle as orc
    import workloads as wl
    import torch
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    offs = w.kv_offsets()
    spent, cpu, done, nbytes = 0.0, 0.0, 0, 0
    per_layer = {}
    # whole steps (layer 0 restarts the recurrence) until about target_s of CPU work
    while spent < target_s:
        S = None
        for l in range(w.layers):
            q, kc, vc = inputs[l]
            ret = [bool(w.retrieval_masks[l] >> h & 1) for h in range(w.num_q_heads)]
            if kc.dtype == torch.uint8:
                k8, v8 = kc.cpu().numpy(), vc.cpu().numpy()
                t0, c0 = time.perf_counter(), time.process_time()
                _, S, _ = orc.hybrid_layer_fp8(wl.bf16_bits(q), k8, v8, 1.0, 1.0, offs, ret, w.k_per_seq, S)
            else:
                qb, kb_, vb = wl.bf16_bits(q), wl.bf16_bits(kc), wl.bf16_bits(vc)
                t0, c0 = time.perf_counter(), time.process_time()
                _, S, _ = orc.hybrid_layer_bf16(qb, kb_, vb, offs, ret, w.k_per_seq, S)
            dt = time.perf_counter() - t0
            cpu += time.process_time() - c0
            spent += dt
            per_layer.setdefault(l, []).append(dt)
            done += 1
            nbytes += total_bytes[l]
            log(f"[bench] oracle layer {l}: cumulative {spent:.1f}s")
            if spent >= target_s:
                break
    # a step's time: measured layers as measured; the others as the mean of the measured
    # layers of their kind (layer 0, layers with retrieval heads, sparse-only layers)
    kind = lambda l: 0 if l == 0 else (1 if w.retrieval_masks[l] else 2)
    mean_of = {}
    for l, ts in per_layer.items():
        mean_of.setdefault(kind(l), []).append(float(np.mean(ts)))
    fallback = float(np.mean([t for v in mean_of.values() for t in v]))
    step_s = sum(float(np.mean(per_layer[l])) if l in per_layer
                 else float(np.mean(mean_of.get(kind(l), [fallback]))) for l in range(w.layers))
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": round(cpu / spent, 1),
            "threads_available": int(threads), "kind": "oracle", "cpu_model": _cpu_model(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "ms_per_layer": round(spent / done * 1e3, 1), "ms_per_step": round(step_s * 1e3, 1),
            "gpu_speedup_per_step": round(step_s * 1e3 / gpu_ms_step, 1),
            "sample": f"{done} layer evaluations ({done / w.layers:.2f} steps of {w.layers} layers) of {w.name} "
                      f"({nbytes / 1e9:.2f} GB algorithmic), fp64 NumPy oracle, {spent:.1f} s wall, "
                      f"{cpu:.1f} s CPU; ms_per_step adds unmeasured layers at the mean of their kind"}


if __name__ == "__main__":
    main()
