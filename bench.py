"""Benchmark of one routed MoE layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|mtp|prefill]

A step is one pass of the whole hot path over one batch: router logits and
top-k, the expert-major union and the quantised SwiGLU experts with the shared
expert and the weighted combine.  Steps of up to 4 tokens (decode, mtp) run as
ONE launch (moe_route_ffn); the prefill chunk as moe_route_union followed by
moe_expert_ffn.  Default workload "decode": 256 experts, top-8 plus one
shared expert, d_model 2048, d_ff 512, Q8_0, one token per step, 38-slot
(15 %) cache.  "mtp": the same layer with Q4_0 weights, four tokens per step
with overlapping routes, 89-slot (35 %) cache.  "prefill": the same layer,
Q8_0, 512 tokens per step with Zipf(1.1)-skewed routes, all experts resident,
bf16 arithmetic on the matrix cores (64-token tiles for buckets of 16+ tokens,
16-token tiles below).

Before each timed step (untimed): the step's experts are found by routing it
once, mapped into the LRU slot cache and filled from the pinned host pack on a
side stream, and then a 512 MiB buffer is read so that neither L2 nor the
256 MB Infinity Cache holds any of the step's weights: the timed step reads
every expert byte from HBM.  The flush reads rather than writes, so the
Infinity Cache is left holding clean lines, as it is after other layers'
weight reads; a written flush would leave 256 MB of dirty lines whose
write-back would be charged to the timed step.  The timed region of a step is
the whole step (route + union + FFN), bracketed by one pair of HIP events on
the stream the kernels run on.  Two more passes over the first min(K, 100) of
the same steps (same staging and flush) time, for comparison, the separate
calls (moe_route_union, then moe_expert_ffn) and the FFN launch alone (for the
prefill chunk the latter is the roofline's kernel; an event recorded between
route and FFN would add idle time of its own, hence separate passes).  Inputs
are resident in HBM when the timed region starts.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, AMD published peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_decode_traffic.json")


CAL_BYTES = 64 << 20  # the plain device-to-device copy each run makes once, for counter calibration


def _code_text(path: str) -> str:
    """A source file without its comments and blank space: what the compiler
    sees, so that editing a comment keeps the counters taken on the code."""
    import re
    s = open(path, encoding="utf-8").read()
    s = re.sub(r"/\*.*?\*/", " ", s, flags=re.S)
    s = re.sub(r"//[^\n]*", "", s)
    return "\n".join(" ".join(line.split()) for line in s.splitlines() if line.strip())


def _kernel_source_digest(workload: str = "decode") -> str:
    h = hashlib.sha256()
    main = "ffn_prefill.hip" if workload == "prefill" else "ffn_decode.hip"
    for f in (main, "device_util.h", "internal.h", "route_device.h"):
        h.update(_code_text(os.path.join(ROOT, "routed_expert_execution_amd", "csrc", f)).encode())
    return h.hexdigest()[:16]


def _traffic(workload: str):
    """HBM bytes per FFN launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    r = t.get(workload)
    if not r or r.get("kernel_source_sha") != _kernel_source_digest(workload):
        return None
    return r["fetch_bytes_per_launch"] + r["write_bytes_per_launch"]


def _counter_rows(d: str):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    out = {}  # dispatch -> (kernel name, value)
    for f in files:
        for r in csv.DictReader(open(f)):
            out[int(r["Dispatch_Id"])] = (r["Kernel_Name"], float(r["Counter_Value"]))
    return [out[k] for k in sorted(out)]


def traffic_from(fetch_dir: str, write_dir: str, workload: str, warmup: int, steps: int) -> int:
    """HBM bytes per launch of the roofline kernel from two rocprofv3 --pmc runs of
    this bench (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what
    the same counter reads for the run's 64 MiB plain copy; written to
    profiles/ffn_decode_traffic.json for the current kernel source."""
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d)
        copies = [v for n, v in rows if "copyBuffer" in n]
        cal = CAL_BYTES / (max(copies) * 1024.0)  # bytes per reported unit
        if workload == "prefill":  # moe_expert_ffn = schedule + tile kernels + combine, per step
            per = {}
            for n, v in rows:
                if any(x in n for x in ("schedule_kernel", "prefill_gate_up", "prefill_down", "prefill_combine")):
                    key = n.replace("(anonymous namespace)::", "").split("(")[0]
                    per.setdefault(key, []).append(v)
            val = sum(float(np.mean(v)) for v in per.values())
        else:  # the one-launch steps of the timed pass
            vals = [v for n, v in rows if "ffn_decode_kernel" in n][warmup:warmup + steps]
            val = float(np.mean(vals))
        res[counter] = (val * 1024.0 * cal, cal)
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        t = {}
    t[workload] = {"kernel_source_sha": _kernel_source_digest(workload),
                   "fetch_bytes_per_launch": res["FETCH_SIZE"][0], "write_bytes_per_launch": res["WRITE_SIZE"][0],
                   "calibration_bytes_per_unit": {"FETCH_SIZE": res["FETCH_SIZE"][1], "WRITE_SIZE": res["WRITE_SIZE"][1]},
                   "calibration": f"{CAL_BYTES} B device-to-device copy in the same run"}
    json.dump(t, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps({workload: t[workload]}))
    return 0


BIG_BUCKET = 167  # tokens from which a Q8_0 bucket of this shape is compute-bound on bf16 MFMA


def big_buckets_mfma(experts, sizes, pack, wl, flush, flush_sink, spin_cycles, no_flush, reps: int = 20,
                     gemm_min: int = 16) -> dict:
    """The grouped GEMM on just the chunk's buckets of at least BIG_BUCKET
    tokens: a context with one routed expert per token, sum(sizes) tokens,
    token i in the bucket of its expert (no shared expert), bf16 mode, cold;
    matrix-core utilisation = 3 d f 2 flops per token over the call's event
    time, against the bf16 dense peak."""
    import torch
    from routed_expert_execution_amd import moe
    import synth
    E, d, f = len(experts), wl["d"], wl["f"]
    T = int(sum(sizes))
    dev = torch.device("cuda", 0)
    cfg = moe.make_config(1, E, 1, d, f, moe.MOE_Q8_0, E, T, device=-1)
    pb = moe.moe_payload_bytes(cfg)
    pool = torch.zeros(E * pb, dtype=torch.uint8, device=dev)
    ctx = moe.Context(1, E, 1, d, f, moe.MOE_Q8_0, E, T, device=0, slot_pool=pool, gemm_min_tokens=gemm_min)
    try:
        for i, e in enumerate(experts):
            pool[i * pb:(i + 1) * pb].copy_(pack[e])
            moe.moe_slot_bind(ctx, 0, i, i)
        ids = torch.from_numpy(np.repeat(np.arange(E, dtype=np.int32), sizes).reshape(T, 1)).to(dev)
        w = torch.ones(T, 1, dtype=torch.float32, device=dev)
        x = torch.from_numpy(synth.activations(wl["seed"], T, d, "bf16", 7).view(np.int16)).view(torch.bfloat16).to(dev)
        y = torch.empty(T, d, dtype=torch.float32, device=dev)
        plan = moe.Plan(ctx, T)
        moe.moe_plan_union(ctx, ids, plan)
        stream = torch.cuda.current_stream(dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps + 2)]
        for e0, e1 in evs:
            if not no_flush:
                flush_sink.copy_(flush.max())
            torch.cuda._sleep(spin_cycles)
            e0.record(stream)
            moe.moe_expert_ffn(ctx, 0, x, plan, w, y, prec=moe.MOE_PREC_BF16)
            e1.record(stream)
        torch.cuda.synchronize()
        if moe.moe_check(ctx) != moe.MOE_OK:
            return None
        us = float(np.mean([a.elapsed_time(b) for a, b in evs[2:]])) * 1e3
    finally:
        ctx.close()
    flops = 3.0 * d * f * 2.0 * T
    return {"sizes": [int(v) for v in sizes], "tokens": T, "us_mean": us, "tflops": flops / (us * 1e-6) / 1e12,
            "mfma_frac": flops / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, "gemm_min_tokens": gemm_min,
            "note": "moe_expert_ffn on only the chunk's buckets of >= %d tokens (one routed expert per token, "
                    "no shared expert), bf16 mode, weights cold" % BIG_BUCKET}


def cpu_baseline(wl: dict, budget_s: float = 10.0, max_steps: int = 100_000, threads: int = 0) -> dict:
    """The oracle, as it stands, timed on a bounded sample of the same steps.

    Only the oracle's own work is timed (router logits, top-k, union, the routed
    and shared experts, the combine); drawing the synthetic inputs is not."""
    import oracle
    import synth

    threads = oracle.set_threads(threads or len(os.sched_getaffinity(0)))
    E, k, d, f, T = wl["E"], wl["k"], wl["d"], wl["f"], wl["T"]
    wr = synth.router_weights(wl["seed"], E, d) if wl["name"] == "decode" else None
    shared = synth.expert_record(wl["seed"], 0, 0, wl["qtype"], d, f, shared=True)
    prec = oracle.PREC_BF16 if wl["prec"] == "bf16" else oracle.PREC_F32
    if wl["name"] == "prefill":  # a bounded sample: groups of 8 tokens of one chunk
        T = 8
        chunk_x = synth.activations(wl["seed"], wl["T"], d, wl["x_dtype"], 0)
        chunk_lg = synth.zipf_gumbel_logits(wl["seed"], wl["T"], E, wl["zipf_s"])
    cache: dict = {}
    steps, compute = 0, 0.0
    while steps < max_steps and compute < budget_s:
        s = 50_000 + steps
        if wl["name"] == "prefill":
            rows = slice((steps * T) % wl["T"], (steps * T) % wl["T"] + T)
            x, lg_in = chunk_x[rows], chunk_lg[rows]
        else:
            x = synth.activations(wl["seed"], T, d, wl["x_dtype"], s)
            if wr is not None:
                lg_in = None
            elif wl["name"] == "stack":  # one layer step of the stack: a one-token Markov chain
                lg_in = synth.markov_logits(wl["seed"], steps % wl["n_layers"], 1, E, k, wl["p_repeat"])
            else:
                lg_in = synth.mtp_logits(wl["seed"], s, T, E, k, wl["p_shared_route"])
        t0 = time.perf_counter()
        x64 = oracle.x_to_f64(x, wl["x_dtype"])
        lg = oracle.router_logits(x64, wr) if wr is not None else lg_in
        ids, w = oracle.topk(lg, k)
        oracle.plan_union(ids, E)
        compute += time.perf_counter() - t0
        recs = [None] * E
        for e in set(ids.reshape(-1).tolist()):
            if e not in cache:
                cache[e] = synth.expert_record(wl["seed"], 0, e, wl["qtype"], d, f)
            recs[e] = cache[e]
        t0 = time.perf_counter()
        oracle.moe_layer(wl["qtype"], prec, recs, shared, d, f, x64, ids, w)
        compute += time.perf_counter() - t0
        steps += 1
    return {"value": steps * T / compute, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"{steps} groups of {T} tokens of one 512-token chunk" if wl["name"] == "prefill"
                       else f"{steps} layer steps of one token" if wl["name"] == "stack"
                       else f"{steps} {wl['name']} steps ({steps * T} tokens)")
                      + f" of the same workload: fp64 C oracle, router/top-k/union + {k} routed experts + "
                      f"shared expert per token, {compute:.1f} s of CPU work"}


def cpu_baseline_pair(wl: dict, budget_s: float = 10.0) -> dict:
    """The oracle on every host core the process may use, and on one core: the
    first is the reported baseline, the second rides along."""
    allc = cpu_baseline(wl, budget_s, threads=len(os.sched_getaffinity(0)))
    one = cpu_baseline(wl, budget_s, threads=1)
    allc["one_core"] = {"value": one["value"], "cores": one["cores"], "sample": one["sample"]}
    return allc


def _median_us(pairs) -> float:
    return float(np.median([a.elapsed_time(b) for a, b in pairs]) * 1e3)


def ceilings(torch, moe) -> int:
    """Peak references on this GPU: a streaming read from cold HBM in one launch
    (512 MiB read before each), pinned host -> device copies, and a bf16
    matrix-core loop.  One JSON line."""
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
    flush_sink = torch.empty((), dtype=torch.int32, device=dev)
    buf = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    reads = []
    for mb in (8, 16, 30, 64, 128, 512):
        n = mb << 20
        best = None
        for wgs in (256, 512, 1024, 2048):
            pairs = []
            for _ in range(10):
                flush_sink.copy_(flush.max())
                torch.cuda._sleep(int(100e-6 * 2.4e9))
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                moe.moe_probe_read(buf[:n], sink, workgroups=wgs)
                e1.record(stream)
                pairs.append((e0, e1))
            torch.cuda.synchronize()
            us = _median_us(pairs[2:])
            if best is None or us < best[0]:
                best = (us, wgs)
        us, wgs = best
        reads.append({"MB": mb, "us": round(us, 2), "GBps": round(n / (us * 1e-6) / 1e9, 1), "workgroups": wgs})
    h2d = []
    host = torch.empty(256 << 20, dtype=torch.uint8).pin_memory()
    dst = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    side = torch.cuda.Stream(device=dev)
    for mb in (1, 3.1875, 16, 64, 256):  # 3.1875 MiB = one Q8_0 expert payload
        n = int(mb * (1 << 20))
        pairs = []
        with torch.cuda.stream(side):
            for _ in range(8):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(side)
                dst[:n].copy_(host[:n], non_blocking=True)
                e1.record(side)
                pairs.append((e0, e1))
        torch.cuda.synchronize()
        us = _median_us(pairs[2:])
        h2d.append({"MB": mb, "us": round(us, 1), "GBps": round(n / (us * 1e-6) / 1e9, 1)})
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    fsink = torch.zeros(1, dtype=torch.float32, device=dev)
    mfma = {}
    for shape, name in ((0, "16x16x32 x4 chains"), (1, "32x32x16 x4 chains"), (2, "16x16x32 x8 chains"),
                        (3, "32x32x16 x8 chains"), (4, "16x16x32 x16 chains"), (5, "32x32x16 x16 chains")):
        best = None
        for per_cu in (2, 4, 8):
            grid, iters = cus * per_cu, 20000 // per_cu
            moe.moe_probe_mfma(100, grid, fsink, shape=shape)
            pairs = []
            for _ in range(4):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                flops = moe.moe_probe_mfma(iters, grid, fsink, shape=shape)
                e1.record(stream)
                pairs.append((e0, e1))
            torch.cuda.synchronize()
            us = _median_us(pairs[1:])
            tf = flops / (us * 1e-6) / 1e12
            if best is None or tf > best["TFLOPs"]:
                best = {"TFLOPs": round(tf, 1), "frac": round(tf / 2500.0, 3), "workgroups": grid,
                        "waves_per_cu": 4 * per_cu, "kernel_us": round(us, 1)}
        mfma[name] = best
    lds = None
    isink = torch.zeros(1, dtype=torch.int32, device=dev)
    for per_cu in (1, 2, 4):
        grid = cus * per_cu
        moe.moe_probe_lds(100, grid, isink)
        pairs = []
        for _ in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            nb = moe.moe_probe_lds(20000 // per_cu, grid, isink)
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        us = _median_us(pairs[1:])
        bpc = nb / (us * 1e-6) / cus / 2.4e9
        if lds is None or bpc > lds["bytes_per_clk_per_cu_at_2.4GHz"]:
            lds = {"TBps": round(nb / (us * 1e-6) / 1e12, 1), "bytes_per_clk_per_cu_at_2.4GHz": round(bpc, 1),
                   "waves_per_cu": 4 * per_cu}
    print(json.dumps({"metric": "peak references", "n_gpus": 1, "data": "synthetic", "lds_read_b128": lds,
                      "hbm_streaming_read_cold": reads, "hbm_peak_spec_GBps": HBM_PEAK_GBS,
                      "pinned_h2d_hipMemcpyAsync": h2d,
                      "mfma_bf16_dense": dict(mfma, peak_spec_TFLOPs=2500.0)}), flush=True)
    return 0


def mfma_sweep(torch, moe, synth) -> int:
    """Single-bucket sweep of the prefill path (bf16 mode, the layer of the
    prefill chunk): all M tokens pick the same 8 experts, so the grouped GEMM
    runs 8 buckets of M tokens plus the shared expert's M.  Cold (512 MiB read
    first); the FFN launch between one event pair."""
    wl = synth.workload("prefill")
    E, k, d, f = wl["E"], wl["k"], wl["d"], wl["f"]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    Ms = (16, 32, 64, 128, 256, 512, 2048, 8192)
    cfg = moe.make_config(1, E, k, d, f, moe.MOE_Q8_0, k, max(Ms), device=-1)
    pb = moe.moe_payload_bytes(cfg)
    pool = torch.zeros(k * pb, dtype=torch.uint8, device=dev)
    ctx = moe.Context(1, E, k, d, f, moe.MOE_Q8_0, k, max(Ms), device=0, slot_pool=pool)
    for e in range(k):
        ctx.slot(e).copy_(torch.from_numpy(moe.moe_pack_expert(ctx.cfg, synth.expert_record(wl["seed"], 0, e, wl["qtype"], d, f))))
        moe.moe_slot_bind(ctx, 0, e, e)
    shared = torch.from_numpy(moe.moe_pack_expert(
        ctx.cfg, synth.expert_record(wl["seed"], 0, 0, wl["qtype"], d, f, shared=True))).to(dev)
    flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
    flush_sink = torch.empty((), dtype=torch.int32, device=dev)
    rows = []
    for M in Ms:
        lg = torch.full((M, E), -4.0, dtype=torch.float32, device=dev)
        lg[:, :k] = torch.arange(k, 0, -1, dtype=torch.float32, device=dev)  # experts 0..7, every token
        x = torch.from_numpy(synth.activations(wl["seed"], M, d, "bf16", M).view(np.int16)).view(torch.bfloat16).to(dev)
        ids = torch.empty(M, k, dtype=torch.int32, device=dev)
        w = torch.empty(M, k, dtype=torch.float32, device=dev)
        y = torch.empty(M, d, dtype=torch.float32, device=dev)
        plan = moe.Plan(ctx, M)
        moe.moe_route_union(ctx, ids, w, plan, logits_in=lg)
        pairs = []
        for _ in range(12):
            flush_sink.copy_(flush.max())
            torch.cuda._sleep(int(200e-6 * 2.4e9))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            moe.moe_expert_ffn(ctx, 0, x, plan, w, y, shared_payload=shared, prec=moe.MOE_PREC_BF16)
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        us = _median_us(pairs[2:])
        flops = (k + 1) * M * 3 * 2 * d * f
        tf = flops / (us * 1e-6) / 1e12
        rows.append({"M": M, "us": round(us, 1), "TFLOPs": round(tf, 1), "mfma_frac_of_spec": round(tf / 2500.0, 3),
                     "GBps": round((k + 1) * pb / (us * 1e-6) / 1e9, 1)})
    assert moe.moe_check(ctx) == moe.MOE_OK
    print(json.dumps({"metric": "prefill bucket sweep (bf16 matrix cores)", "n_gpus": 1, "data": "synthetic",
                      "config": {"workload": f"{k} experts x M tokens + shared expert, d_model {d}, d_ff {f}, Q8_0, "
                                             "bf16 mode, cold"},
                      "peak_spec_TFLOPs": 2500.0, "rows": rows}), flush=True)
    ctx.close()
    return 0


def replay_policies(args, synth, moe) -> int:
    """Host only: the 40-layer stack's route trace (and a cyclic trace) replayed
    against LRU (the library's slot manager), seeded random eviction, a static
    per-layer working set and farthest-next-use.  One JSON line."""
    from routed_expert_execution_amd import replay as R
    wl = synth.workload("stack40")
    L, E, k = wl["n_layers"], wl["E"], wl["k"]
    cfg = moe.make_config(L, E, k, wl["d"], wl["f"], moe.MOE_Q8_0, wl["n_slots"], 1, device=-1)
    pb = moe.moe_payload_bytes(cfg)
    n_tok = args.steps
    trace = synth.markov_trace(wl["seed"], L, n_tok, E, k, wl["p_repeat"])
    rows = []
    for cap in (wl["n_slots"], 2 * wl["n_slots"]):
        for pol, kw in (("lru", {}), ("random", dict(seed=1)), ("static", dict(width=16)),
                        ("static", dict(width=20)), ("belady", {})):
            t0 = time.perf_counter()
            r = R.replay(trace, cap, pol, payload_bytes=pb, n_layers=L, n_experts=E, **kw)
            r["bytes_staged_per_token"] = r.pop("bytes_staged") / n_tok
            r["replay_s"] = round(time.perf_counter() - t0, 2)
            rows.append(r)
    cyc = []
    for cap in (9, 10):
        tr = R.cyclic_trace(10, 50)
        for pol in ("lru", "belady"):
            r = R.replay(tr, cap, pol)
            cyc.append(dict(capacity=cap, policy=pol, hits=r["hits"], misses=r["misses"]))
    print(json.dumps({"metric": "slot policy replay (host only)", "data": "synthetic",
                      "config": {"workload": f"stack route trace: {L} layers x {n_tok} tokens, {E} experts, top-{k}, "
                                             f"Markov p_repeat {wl['p_repeat']}; payload {pb} B",
                                 "cyclic": "one layer cycling through 10 experts, 50 cycles"},
                      "stack": rows, "cyclic": cyc}), flush=True)
    return 0


def run_stack(args, torch, moe, synth) -> int:
    """40 routed layers of the decode shape sharing one 1,536-slot LRU pool:
    per layer the step is routed (synthetic Markov logits), its plan read
    back, its misses staged from pinned host memory on a side stream, and its
    experts run, one token at a time."""
    wl = dict(synth.workload("stack40"), name="stack")
    if args.slots:
        wl["n_slots"] = args.slots
    L, E, k, d, f, n_slots = wl["n_layers"], wl["E"], wl["k"], wl["d"], wl["f"], wl["n_slots"]
    if args.prefetch and args.staging != "native":
        print("--prefetch needs --staging native (moe_prefetch_next follows moe_route_pull)", file=sys.stderr)
        return 2
    if args.split and args.staging != "native":
        print("--split needs --staging native (moe_expert_ffn_split follows moe_route_pull)", file=sys.stderr)
        return 2
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    n_tok = args.warmup + args.steps
    cfg = moe.make_config(L, E, k, d, f, moe.MOE_Q8_0, n_slots, 1, device=-1)
    pb = moe.moe_payload_bytes(cfg)
    pool = torch.zeros(n_slots * pb, dtype=torch.uint8, device=dev)
    ctx = moe.Context(L, E, k, d, f, moe.MOE_Q8_0, n_slots, 1, device=0, slot_pool=pool)
    t_gen = time.perf_counter()
    n_alias = 4  # pinned payload sets; layer l stages from set l % 4
    packs = [torch.empty((E, pb), dtype=torch.uint8).pin_memory() for _ in range(n_alias)]
    for a in range(n_alias):
        for e in range(E):
            moe.moe_pack_expert(ctx.cfg, synth.expert_record(wl["seed"], a, e, wl["qtype"], d, f),
                                out=packs[a].numpy()[e])
    shared = torch.from_numpy(moe.moe_pack_expert(
        ctx.cfg, synth.expert_record(wl["seed"], 0, 0, wl["qtype"], d, f, shared=True))).to(dev)
    if args.follow_routes > 0:
        lg = torch.from_numpy(synth.follow_stack_logits(wl["seed"], L, n_tok, E, k, wl["p_repeat"],
                                                        args.follow_routes)).to(dev)
    else:
        lg = torch.stack([torch.from_numpy(synth.markov_logits(wl["seed"], l, n_tok, E, k, wl["p_repeat"]))
                          for l in range(L)]).to(dev)  # [L, tokens, E]
    # layer 0's input per token (and, with --fresh-inputs, every layer's);
    # otherwise x_{l+1} = bf16(y_l / rms(y_l)), eps 1e-6, no weight
    n_in = L if args.fresh_inputs else 1
    xs = torch.stack([torch.stack([torch.from_numpy(
        (synth.activations(wl["seed"], 1, d, "bf16", t, l) if args.fresh_inputs
         else synth.activations(wl["seed"], 1, d, "bf16", t)).view(np.int16)).view(torch.bfloat16)
        for l in range(n_in)]) for t in range(n_tok)]).to(dev)  # [tokens, n_in, 1, d]
    t_gen = time.perf_counter() - t_gen
    ids = torch.empty(1, k, dtype=torch.int32, device=dev)
    w = torch.empty(1, k, dtype=torch.float32, device=dev)
    y = torch.empty(1, d, dtype=torch.float32, device=dev)
    plan = moe.Plan(ctx, 1)
    tables = [moe.payload_table(ctx, [packs[a][e] for e in range(E)]) for a in range(n_alias)]
    sides = [torch.cuda.Stream(device=dev) for _ in range(max(1, args.fill_streams))]
    side = sides[0]
    split_side = torch.cuda.Stream(device=dev)  # the resident units of a split layer
    stream = torch.cuda.current_stream(dev)
    ffn_ev = []
    pull_ev = []  # (event before the pull, misses): the pull ends where the FFN's first event is
    n_fill = 0
    unique = 0
    pred_n = [0, 0]  # candidates processed, copies queued by moe_prefetch_next

    def token(t, timed):
        nonlocal unique, n_fill
        x = xs[t, 0]
        for l in range(L):
            ev = timed and l % 8 == 0  # kernel times on every 8th layer
            if args.staging == "native":  # route, mirror, host map and pull in one library call
                experts, slots, miss = moe.moe_route_pull(ctx, l, ids, w, plan, tables[l % n_alias],
                                                          logits_in=lg[l, t:t + 1], stream=stream)
                n = len(experts)
            else:
                moe.moe_route_union(ctx, ids, w, plan, logits_in=lg[l, t:t + 1])
                n, experts = plan.experts_host(spin=args.spin_readback)  # the host learns the experts only now
            if args.staging == "native":
                pass
            elif args.staging == "pull":  # map, then the misses copied by a kernel on the compute stream
                if ev:
                    ep = torch.cuda.Event(enable_timing=True)
                    ep.record(stream)
                slots, miss = moe.moe_slot_pull(ctx, l, experts, tables[l % n_alias], stream=stream)
                if ev:
                    pull_ev.append((ep, int(miss.sum())))
            elif args.staging == "stage":  # map + copies over the side streams + one page-table launch
                slots, miss = moe.moe_slot_stage(ctx, l, experts, tables[l % n_alias], sides)
                n_fill += int(miss.sum())
            else:
                slots, miss = moe.moe_slot_map(ctx, l, experts)
                for e, sl, m in zip(experts, slots, miss):
                    if m:  # fills alternate over the side streams (copy engines)
                        moe.moe_slot_fill(ctx, l, int(e), int(sl), packs[l % n_alias][int(e)],
                                          stream=sides[n_fill % len(sides)])
                        n_fill += 1
            if args.prefetch:  # the next layer's predictions, copied on a side stream while this layer runs
                nl = (l + 1) % L  # (layer 0 of the next token after the last)
                ex_p, fl_p = moe.moe_prefetch_next(ctx, l, tables[nl % n_alias], args.prefetch * pb,
                                                   min_weight=args.prefetch_min_weight,
                                                   min_transition=args.prefetch_min_transition, stream=side)
                pred_n[0] += len(ex_p)
                pred_n[1] += int(fl_p.sum())
            if ev:
                # the FFN waits for fills it needs anyway; waiting for the side
                # streams before the first event keeps their copies out of the
                # kernel's time (this layer's own misses; prefetches of the next
                # layer overlap it otherwise)
                if args.staging not in ("pull", "native"):
                    for sd in sides:
                        stream.wait_stream(sd)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            if args.split:  # the resident units on split_side while the pull runs, the pulled ones after it
                moe.moe_expert_ffn_split(ctx, l, xs[t, l] if args.fresh_inputs else x, plan, w, y, experts[miss],
                                         shared_payload=shared, side=split_side, stream=stream)
            else:
                moe.moe_expert_ffn(ctx, l, xs[t, l] if args.fresh_inputs else x, plan, w, y, shared_payload=shared)
            if ev:
                e1.record(stream)
                ffn_ev.append((e0, e1))
                unique += n
            moe.moe_slot_release(ctx, l)
            if not args.fresh_inputs:
                x = torch.nn.functional.rms_norm(y, (d,), eps=1e-6).to(torch.bfloat16)

    for t in range(args.warmup):
        token(t, False)
    torch.cuda.synchronize()
    st0 = moe.moe_stats(ctx)
    pf0 = moe.moe_prefetch_stats(ctx)
    pred0 = list(pred_n)
    wall0 = time.perf_counter()
    for t in range(args.warmup, n_tok):
        token(t, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    st1 = moe.moe_stats(ctx)
    st = moe.moe_check(ctx)
    if st != moe.MOE_OK:
        print(f"device error word set: status {st}", file=sys.stderr)
        return 1
    pf1 = moe.moe_prefetch_stats(ctx)
    pf = {kk: pf1[kk] - pf0[kk] for kk in pf1}  # over the timed tokens
    pf["candidates"] = pred_n[0] - pred0[0]
    pf["copies_queued"] = pred_n[1] - pred0[1]
    hits, misses = st1["hits"] - st0["hits"], st1["misses"] - st0["misses"]
    staged = st1["bytes_staged"] - st0["bytes_staged"]
    ffn = np.array([a.elapsed_time(b) for a, b in ffn_ev]) * 1e3
    ffn_bytes = (unique + len(ffn_ev)) * pb  # unique routed experts + shared, over the timed layer steps
    ffn_gbs = ffn_bytes / (ffn.sum() * 1e-6) / 1e9
    pull = None
    if pull_ev:
        pairs = [(p.elapsed_time(f[0]) * 1e3, m) for (p, m), f in zip(pull_ev, ffn_ev) if m]
        if pairs:
            us = sum(a for a, _ in pairs)
            pull = {"layers_sampled": len(pairs), "us_mean": us / len(pairs),
                    "GBps": sum(m for _, m in pairs) * pb / (us * 1e-6) / 1e9,
                    "note": "moe_slot_pull kernels of every 8th layer with misses, payload bytes over their "
                            "event time; link reference 57 GB/s (pinned host to device, peak_references.md)"}
    line = {
        "metric": "routed MoE tokens/s through a 40-layer decode stack (demand-staged slot cache)",
        "value": args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (q8_0 weights dequantised in registers)",
        "data": "synthetic (seeded; no checkpoint)",
        "config": {
            "workload": (f"stack: {L} MoE layers, {E} experts, top-{k} + 1 shared expert, d_model {d}, d_ff {f}, "
                         f"Q8_0, 1 token/step, one {n_slots}-slot LRU pool shared by the layers, Markov routes "
                         f"(p_repeat {wl['p_repeat']}), misses staged from pinned host memory "
                         f"after each layer's plan readback; payload sets alias mod {n_alias} layers"
                         + (f"; routes also follow the layer below (p_follow {args.follow_routes}; not the "
                            f"pages' workload)" if args.follow_routes > 0 else "")
                         + ("; fresh synthetic input per layer" if args.fresh_inputs
                            else "; layers chained: x_{l+1} = bf16(y_l / rms(y_l)), eps 1e-6")
                         + (f"; moe_prefetch_next after each moe_route_pull: up to {args.prefetch} payloads of the "
                            f"next layer's predicted experts (previous token's weight >= "
                            f"{args.prefetch_min_weight}" + (f", then layer-to-layer transition scores >= "
                                                             f"{args.prefetch_min_transition}"
                                                             if args.prefetch_min_transition > 0 else "")
                            + ") copied on a side stream while the layer computes" if args.prefetch else "")
                         + (f"; copies alternate over {args.fill_streams} side streams"
                            if args.fill_streams > 1 and args.staging != "pull" else "")
                         + ("; hit/miss split: moe_expert_ffn_split runs the resident experts on a second "
                            "stream while the pull runs, the pulled ones after it" if args.split else "")
                         + {"native": "; one moe_route_pull per layer: routing, expert readback through pinned "
                                      "memory, mapping and a pull kernel in one library call",
                            "pull": "; one moe_slot_pull per layer: a kernel on the compute stream copies the misses",
                            "stage": "; one moe_slot_stage call per layer",
                            "fill": "; moe_slot_map + one moe_slot_fill per miss"}[args.staging]),
            "global_batch": 1,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "moe_expert_ffn per layer (one launch, every 8th layer timed); expert payload bytes "
                      "over its event time",
            "achieved": ffn_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": ffn_gbs / HBM_PEAK_GBS,
            "traffic": None,
        },
        "detail": {
            "hit_rate": hits / max(hits + misses, 1),
            "misses_per_token": misses / args.steps,
            "bytes_staged_per_token": staged / args.steps,
            "bytes_staged_equals_misses_x_payload": staged == misses * pb,
            "h2d_GBps_achieved": staged / wall / 1e9,
            "ffn_us_mean": float(ffn.mean()),
            "ffn_us_p50": float(np.median(ffn)),
            "ffn_us_max": float(ffn.max()),
            "ffn_GBps": ffn_gbs,
            "layer_steps_timed": len(ffn_ev),
            "pull": pull,
            "setup_pack_s": t_gen,
            "prefetch": ({"cap_payloads_per_layer": args.prefetch, "min_weight": args.prefetch_min_weight,
                          "min_transition": args.prefetch_min_transition, **pf,
                          "note": "fills/useful/wasted/bytes over the timed tokens (useful: a later demand map "
                                  "found it; wasted: evicted unused)"} if args.prefetch else None),
            "n_slots": n_slots,
            "pages_context": "end-to-end 52.03 tok/s (best layer split) and 14.66 tok/s (exact RAM prefetch) "
                             "on an RTX 3080 PC, a different model and machine",
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(dict(wl, name="stack", T=1), budget_s=10.0)
        line["cpu_baseline"]["value"] /= L  # layer steps/s -> tokens/s through all layers
        line["cpu_baseline"]["unit"] = "tokens/s (40 layers per token)"
    print(json.dumps(line), flush=True)
    ctx.close()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 1000 decode/mtp steps, 200 prefill chunks, 256 stack tokens)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=["decode", "mtp", "prefill", "stack", "replay"])
    ap.add_argument("--prefetch", type=int, default=0, metavar="N",
                    help="stack: after each layer's moe_route_pull, moe_prefetch_next stages up to N payloads "
                         "of the next layer's predicted experts on a side stream while the layer computes")
    ap.add_argument("--prefetch-min-weight", type=float, default=0.20, metavar="W",
                    help="stack: prediction threshold (the previous token's experts of the next layer with "
                         "routing weight >= W; transition scores >= W)")
    ap.add_argument("--prefetch-min-transition", type=float, default=0.0, metavar="S",
                    help="stack: also predict from layer-to-layer transition counts, scores >= S (0: off)")
    ap.add_argument("--slots", type=int, default=0, metavar="S",
                    help="stack: slots in the pool (default: the workload's 1,536)")
    ap.add_argument("--follow-routes", type=float, default=0.0, metavar="P",
                    help="stack: routes that also follow the layer below (new picks the image of an expert of "
                         "the same token one layer down with probability P; not the pages' workload)")
    ap.add_argument("--fresh-inputs", action="store_true",
                    help="stack: a fresh synthetic input per layer instead of the chained x_{l+1} = "
                         "bf16(y_l / rms(y_l))")
    ap.add_argument("--fill-streams", type=int, default=2, metavar="S",
                    help="stack: side streams the misses' copies alternate over")
    ap.add_argument("--no-big-buckets", action="store_true",
                    help="prefill: skip the big-bucket matrix-core run (profiler runs cover the chunk's calls only)")
    ap.add_argument("--big-gemm-min", type=int, default=0, metavar="M",
                    help="prefill: also time the big buckets with this gemm_min_tokens")
    ap.add_argument("--gemm-min", type=int, default=16, metavar="M",
                    help="prefill, bf16 mode: buckets of at least M tokens use 64-token tiles")
    ap.add_argument("--spin-readback", action="store_true",
                    help="stack: poll for the plan readback instead of a blocking synchronise")
    ap.add_argument("--split", action="store_true",
                    help="stack: moe_expert_ffn_split instead of moe_expert_ffn (the resident experts on a second "
                         "stream while the misses are pulled, the pulled ones after)")
    ap.add_argument("--staging", choices=("native", "pull", "stage", "fill"), default="native",
                    help="stack: one moe_route_pull per layer (routing, mapping and pull in one call), "
                         "one moe_slot_pull per layer (kernel copies on the compute stream), one "
                         "moe_slot_stage per layer (copy engines on side streams), or moe_slot_map + one "
                         "moe_slot_fill per miss")
    ap.add_argument("--mfma-sweep", action="store_true",
                    help="prefill buckets of M tokens (M = 16 .. 512) on the matrix cores: time and utilisation")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="parse two rocprofv3 --pmc runs of this bench into the traffic file (no GPU)")
    ap.add_argument("--ceilings", action="store_true",
                    help="print the peak references (streaming read, pinned H2D, matrix-core loop) instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="decode: skip the 512-token chunk that the default run also times")
    ap.add_argument("--no-flush", action="store_true", help="leave L2 / Infinity Cache warm (labelled)")
    ap.add_argument("--separate-calls", action="store_true",
                    help="time steps of up to 4 tokens as moe_route_union + moe_expert_ffn, not one launch")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = {"decode": 1000, "mtp": 1000, "prefill": 200, "stack": 256, "replay": 256}.get(args.workload, 200)
    if args.traffic_from:
        return traffic_from(args.traffic_from[0], args.traffic_from[1], args.workload, args.warmup, args.steps)
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the routed-expert path; --gpus {args.gpus} is not "
              f"available (one process, one GPU).", file=sys.stderr)
        return 2

    import torch

    import synth
    from routed_expert_execution_amd import moe

    # No cyclic garbage collection while measuring (as timeit does): a full
    # collection of this process's heap stops the host for tens of ms, and a
    # stop between a step's launches leaves the GPU idle inside its timing.
    gc.collect()
    gc.disable()

    if args.workload == "replay":
        return replay_policies(args, synth, moe)
    if args.ceilings:
        return ceilings(torch, moe)
    if args.mfma_sweep:
        return mfma_sweep(torch, moe, synth)
    if args.workload == "stack":
        return run_stack(args, torch, moe, synth)

    line = layer_bench(args, torch, moe, synth, args.workload, args.steps, args.warmup, args.no_flush,
                       big=not args.no_big_buckets, warm=args.workload == "decode")
    if line is None:
        return 1
    if args.workload == "decode" and not args.decode_only:
        # the batch-512 half of the metric in the same run: the prefill chunk,
        # cold, with its big buckets on the matrix cores
        pre = layer_bench(args, torch, moe, synth, "prefill", min(args.steps, 20), min(args.warmup, 3),
                          args.no_flush, big=not args.no_big_buckets)
        if pre is None:
            return 1
        bb = pre["detail"]["big_buckets"] or {}
        line["detail"]["prefill_chunk_512"] = {
            "tokens_per_s": pre["value"], "ms_per_chunk": pre["ms_per_step"], "chunks_timed": pre["steps"],
            "ffn_us_mean": pre["detail"]["ffn_us_mean"], "ffn_GBps": pre["detail"]["ffn_GBps"],
            "hbm_frac_spec": pre["roofline"]["frac"],
            "hbm_frac_measured": pre["roofline"].get("frac_of_measured"),
            "expert_bytes_per_chunk": pre["detail"]["expert_bytes_per_step"],
            "unique_experts": pre["detail"]["unique_experts_per_step"],
            "big_buckets_mfma_frac_spec": bb.get("mfma_frac"), "big_buckets": bb or None,
            "workload": pre["config"]["workload"],
        }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_pair(dict(synth.workload(args.workload), name=args.workload))
    print(json.dumps(line), flush=True)
    return 0


def measured_read_ceiling(torch, moe, n_bytes: int, reps: int = 8) -> dict:
    """The streaming-read reference for n_bytes: one launch reading that many
    bytes from cold HBM (512 MiB read before each), best over workgroup counts."""
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    n = (int(n_bytes) + 15) // 16 * 16
    buf = torch.ones(n, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)
    flush_sink = torch.empty((), dtype=torch.int32, device=dev)
    best = None
    for wgs in (256, 512, 1024, 2048):
        pairs = []
        for _ in range(reps):
            flush_sink.copy_(flush.max())
            torch.cuda._sleep(int(100e-6 * 2.4e9))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            moe.moe_probe_read(buf, sink, workgroups=wgs)
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        us = _median_us(pairs[2:])
        if best is None or us < best[0]:
            best = (us, wgs)
    del buf
    return {"bytes": n, "us": best[0], "GBps": n / (best[0] * 1e-6) / 1e9, "workgroups": best[1],
            "note": "moe_probe_read: one launch streaming the same byte count from cold HBM (512 MiB read first)"}


def layer_bench(args, torch, moe, synth, name, steps, warmup, no_flush, big=True, warm=False):
    wl = dict(synth.workload(name), name=name)
    E, k, d, f, T = wl["E"], wl["k"], wl["d"], wl["f"], wl["T"]
    qt = moe.MOE_Q8_0 if wl["qtype"] == synth.Q8_0 else moe.MOE_Q4_0
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    # ---- resident inputs -------------------------------------------------
    cfg = moe.make_config(1, E, k, d, f, qt, wl["n_slots"], T, device=-1)
    pb = moe.moe_payload_bytes(cfg)
    pool = torch.zeros(wl["n_slots"] * pb, dtype=torch.uint8, device=dev)
    ctx = moe.Context(1, E, k, d, f, qt, wl["n_slots"], T, device=0, slot_pool=pool, gemm_min_tokens=args.gemm_min)
    t_gen = time.perf_counter()
    pack = torch.empty((E, pb), dtype=torch.uint8).pin_memory()  # pinned host pack
    pack_np = pack.numpy()
    for e in range(E):
        moe.moe_pack_expert(ctx.cfg, synth.expert_record(wl["seed"], 0, e, wl["qtype"], d, f), out=pack_np[e])
    shared = torch.from_numpy(moe.moe_pack_expert(
        ctx.cfg, synth.expert_record(wl["seed"], 0, 0, wl["qtype"], d, f, shared=True))).to(dev)
    t_gen = time.perf_counter() - t_gen
    wr = torch.from_numpy(synth.router_weights(wl["seed"], E, d)).to(dev) if name == "decode" else None
    prec = moe.MOE_PREC_BF16 if wl["prec"] == "bf16" else moe.MOE_PREC_F32

    n_steps = warmup + steps
    x_all = torch.stack([
        torch.from_numpy(synth.activations(wl["seed"], T, d, "bf16", s).view(np.int16)).view(torch.bfloat16)
        for s in range(n_steps)]).to(dev)  # [steps, T, d]
    lg_all = None
    if name == "mtp":
        lg_all = torch.stack([torch.from_numpy(synth.mtp_logits(wl["seed"], s, T, E, k, wl["p_shared_route"]))
                              for s in range(n_steps)]).to(dev)
    elif name == "prefill":
        lg_all = torch.stack([torch.from_numpy(synth.zipf_gumbel_logits(wl["seed"] + s, T, E, wl["zipf_s"]))
                              for s in range(n_steps)]).to(dev)
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    y = torch.empty(T, d, dtype=torch.float32, device=dev)
    plan = moe.Plan(ctx, T)
    flush = torch.ones(128 << 20, dtype=torch.int32, device=dev)  # 512 MiB, read before every step
    cal = torch.empty(CAL_BYTES // 4, dtype=torch.int32, device=dev)
    cal.copy_(flush[: CAL_BYTES // 4])  # a plain copy of known size (counter calibration)
    flush_sink = torch.empty((), dtype=torch.int32, device=dev)
    spin_cycles = int(300e-6 * 2.4e9)  # ~300 us of GPU-side spin before each timed step
    side = torch.cuda.Stream(device=dev)
    stream = torch.cuda.current_stream(dev)

    def route_plan(s):
        if lg_all is not None:
            moe.moe_route_union(ctx, ids, w, plan, logits_in=lg_all[s])
        else:
            moe.moe_route_union(ctx, ids, w, plan, x=x_all[s], w_router=wr)

    one_launch = T <= 4 and not args.separate_calls  # the step as one moe_route_ffn launch

    def whole_step(s):
        if one_launch:
            kw = dict(logits_in=lg_all[s]) if lg_all is not None else dict(w_router=wr)
            moe.moe_route_ffn(ctx, 0, x_all[s], ids, w, plan, y, shared_payload=shared, prec=prec, **kw)
        else:
            route_plan(s)
            moe.moe_expert_ffn(ctx, 0, x_all[s], plan, w, y, shared_payload=shared, prec=prec)

    misses = 0

    def prepare(s, cold=True):
        """Untimed: learn step s's experts, stage misses, flush caches (unless
        cold is False or the run is warm), then spin."""
        nonlocal misses
        route_plan(s)
        n, experts, _, _ = plan.host()
        slots, miss = moe.moe_slot_map(ctx, 0, experts)
        for e, sl, m in zip(experts, slots, miss):
            if m:
                moe.moe_slot_fill(ctx, 0, int(e), int(sl), pack[int(e)], stream=side)
                misses += 1
        side.synchronize()
        if cold and not no_flush:
            flush_sink.copy_(flush.max())
        # keep the GPU busy while the host enqueues the timed kernels, so the
        # timed region measures GPU work, not Python launch latency
        torch.cuda._sleep(spin_cycles)
        return n

    def new_events(m):
        return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(m)]

    # Pass 1 (the K timed steps): the whole step between one event pair.
    ev = new_events(n_steps)
    n_unique = []
    torch.cuda.synchronize()
    for s in range(n_steps):
        if s == warmup:
            torch.cuda.synchronize()
            wall_t0 = time.perf_counter()
        n = prepare(s)
        e0, e2 = ev[s]
        e0.record(stream)
        whole_step(s)
        e2.record(stream)
        moe.moe_slot_release(ctx, 0)
        n_unique.append(n)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall_t0
    # Pass 2: the same steps as separate calls (route + union, then FFN).
    # Pass 3: the FFN launch alone between the events (route and union before
    # them, untimed).
    n_ffn = min(steps, 100)
    ev_sep, ev_ffn = new_events(n_ffn), new_events(n_ffn)
    for i in range(n_ffn):
        s = warmup + i
        prepare(s)
        e1, e2 = ev_sep[i]
        e1.record(stream)
        route_plan(s)
        moe.moe_expert_ffn(ctx, 0, x_all[s], plan, w, y, shared_payload=shared, prec=prec)
        e2.record(stream)
        moe.moe_slot_release(ctx, 0)
        prepare(s)
        route_plan(s)
        e1, e2 = ev_ffn[i]
        e1.record(stream)
        moe.moe_expert_ffn(ctx, 0, x_all[s], plan, w, y, shared_payload=shared, prec=prec)
        e2.record(stream)
        moe.moe_slot_release(ctx, 0)
    # Pass 4 (decode only, labelled warm): the whole step again on the first
    # n_ffn steps with no cache flush before it, each step run twice in a row
    # so the second finds its weights in the Infinity Cache and L2.
    ev_warm = new_events(n_ffn) if warm else []
    for i in range(len(ev_warm)):
        s = warmup + i
        prepare(s, cold=False)
        whole_step(s)
        torch.cuda._sleep(spin_cycles)
        e1, e2 = ev_warm[i]
        e1.record(stream)
        whole_step(s)
        e2.record(stream)
        moe.moe_slot_release(ctx, 0)
    torch.cuda.synchronize()
    st = moe.moe_check(ctx)
    if st != moe.MOE_OK:
        print(f"device error word set: status {st}", file=sys.stderr)
        return None
    big_res = None
    if name == "prefill":
        route_plan(warmup)
        n, experts, offsets, _ = plan.host()
        sizes = np.diff(offsets)
        sel = [i for i in range(n) if sizes[i] >= BIG_BUCKET]
        if sel and big:
            big_res = big_buckets_mfma([int(experts[i]) for i in sel], [int(sizes[i]) for i in sel], pack, wl,
                                   flush, flush_sink, spin_cycles, no_flush)
            if args.big_gemm_min:
                big_res["alt"] = big_buckets_mfma([int(experts[i]) for i in sel], [int(sizes[i]) for i in sel], pack, wl,
                                              flush, flush_sink, spin_cycles, no_flush,
                                              gemm_min=args.big_gemm_min)

    span = np.array([ev[s][0].elapsed_time(ev[s][1]) for s in range(warmup, n_steps)]) * 1e3  # us
    sep = np.array([a.elapsed_time(b) for a, b in ev_sep]) * 1e3
    ffn = np.array([a.elapsed_time(b) for a, b in ev_ffn]) * 1e3
    uniq = np.array(n_unique[warmup:])
    uniq_ffn = uniq[:n_ffn]
    algo_bytes = (uniq + 1) * pb  # unique routed experts + the shared expert, per step
    ffn_gbs = ((uniq_ffn + 1) * pb).mean() / (ffn.mean() * 1e-6) / 1e9
    span_gbs = algo_bytes.mean() / (span.mean() * 1e-6) / 1e9
    # roofline kernel: the one launch of the whole step (T <= 4), else the FFN launch
    roof_gbs = span_gbs if one_launch else ffn_gbs
    traffic = _traffic(name)
    # the achievable streaming rate for the same byte count, measured now
    ceil = measured_read_ceiling(torch, moe, algo_bytes.mean()) if not no_flush else None
    warm_res = None
    if ev_warm:
        wspan = np.array([a.elapsed_time(b) for a, b in ev_warm]) * 1e3
        warm_res = {"label": "WARM: no cache flush; the same step run just before, so its weights sit in the "
                             "Infinity Cache / L2 (not the headline)",
                    "steps": len(ev_warm), "span_us_mean": float(wspan.mean()),
                    "span_us_p50": float(np.percentile(wspan, 50)), "tokens_per_s": T / (wspan.mean() * 1e-6),
                    "expert_GBps": float(((uniq[:len(ev_warm)] + 1) * pb).mean() / (wspan.mean() * 1e-6) / 1e9)}

    line = {
        "metric": "routed MoE-layer tokens/s (batch %d %s step: route + union + expert FFN)"
                  % (T, "prefill" if name == "prefill" else "decode"),
        "value": T / (span.mean() * 1e-6),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": span.mean() * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 x bf16 -> f32 (matrix cores), %s weights" if prec == moe.MOE_PREC_BF16
                  else "f32 (%s weights dequantised in registers)") % ("q8_0" if qt == moe.MOE_Q8_0 else "q4_0"),
        "data": "synthetic (seeded; no checkpoint)",
        "config": {
            "workload": (f"{name}: 1 MoE layer, {E} experts, top-{k} + 1 shared expert, d_model {d}, "
                         f"d_ff {f}, {'Q8_0' if qt == moe.MOE_Q8_0 else 'Q4_0'}, {T} token(s)/step, "
                         f"{wl['n_slots']}-slot LRU cache, "
                         + ("512 MiB read before every step (weights cold in L2 and Infinity Cache)" if not no_flush
                            else "caches warm")),
            "global_batch": T,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("moe_route_ffn: one launch of router, top-k, union, routed + shared experts and "
                       "the weighted merge; bytes = expert payloads only" if one_launch else
                       "moe_expert_ffn (one call: its expert kernels and the combine)"),
            "achieved": roof_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": roof_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "measured_peak": ceil["GBps"] if ceil else None,
            "frac_of_measured": roof_gbs / ceil["GBps"] if ceil else None,
        },
        "detail": {
            "layer_span_us_p50": float(np.percentile(span, 50)),
            "layer_span_us_p90": float(np.percentile(span, 90)),
            "one_launch": one_launch,
            "separate_calls_span_us_mean": float(sep.mean()),
            "separate_calls_span_us_p50": float(np.percentile(sep, 50)),
            "ffn_us_mean": float(ffn.mean()),
            "ffn_us_p50": float(np.percentile(ffn, 50)),
            "ffn_us_p90": float(np.percentile(ffn, 90)),
            "ffn_GBps": ffn_gbs,
            "route_union_us_mean_est": float(sep.mean() - ffn.mean()),
            "ffn_timed_steps": int(n_ffn),
            "expert_bytes_per_step": float(algo_bytes.mean()),
            "layer_span_GBps": span_gbs,
            "unique_experts_per_step": float(uniq.mean()),
            "assignments_per_step": T * k,
            "dedupe_fraction": float(1.0 - uniq.mean() / (T * k)),
            "slot_misses_staged": misses,
            "big_buckets": big_res,
            "measured_read_ceiling": ceil,
            "warm_cache": warm_res,
            "wall_s_timed_loop_incl_staging_and_flush": wall,
            "setup_pack_s": t_gen,
        },
    }
    ctx.close()
    return line


if __name__ == "__main__":
    sys.exit(main())
