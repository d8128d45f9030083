"""Benchmark of the chunked KDA forward on one MI355X.

One step = one forward call over one batch of seeded synthetic input already
resident in HBM: the scheduler kernel, then chunk prep and chunk recurrence
(two kernels on the split path, one on the fused path).  The headline is the
library's own path choice, kda_fwd_ex(path = KDA_PATH_AUTO), on T = 8192,
H = 96, K = V = 128, one fixed-length sequence, bf16 initial and final state,
lower_bound = -5 (it runs the split path there).  Every one of the five
workloads (gated_delta_rule_prep_amd.inputs.configs) gets its own entry with
the library's choice and the explicit paths (split and fused with 16-token
chunks, split with 32- and 64-token chunks) timed beside it.

Protocol (the pages' benchmark runs 30 warmup calls, then 5 repeats of 200
timed calls, and reports the median; these are the defaults): W warmup steps,
then R repeats of K timed steps each, bracketed by device synchronisation; the step time is the
median over the repeats (min and max beside it).  Per-kernel times come from
HIP events that kda_fwd_ex records around every kernel on the stream it runs
on (median over K profiled calls).  The roofline is computed for the kernel
that takes the most time, with algorithmic bytes only (the method's inputs and
outputs that kernel is responsible for), and for the whole path; us per chunk
step is the chain kernel's (recurrence or fused) time over the chunk steps a
workgroup slot runs in sequence (sequential_steps).  The
fp64 oracle is timed on a bounded sample of the headline workload on the host
cores (cpu_baseline).

Also timed (not the headline): one decode step (kda_decode) of 256
one-token sequences x 96 heads with a bf16 state updated in place, and one
long sequence with 4 heads on the segmented form.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--repeats R] [--no-cpu]
                       [--only 0|1|2|3|4|fixed|varlen|decode|segmented] [--chunk 16|32|64]
                       [--path auto|fused|split]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16/fp16 matrix, TFLOP/s
METRIC = "KDA fwd ms + token·heads/s at T=8192,D=128,H=96 (fixed, varlen 8x1024)"

# Algorithmic bytes per token-head (q, k, v, g: 4 x 256 B; beta 2 B; out 256 B),
# split by the kernel that moves them.
PREP_BYTES_PER_TH = 3 * 256 + 2      # q, k, g, beta
RECUR_BYTES_PER_TH = 256 + 256       # v in, out
PATH_BYTES_PER_TH = PREP_BYTES_PER_TH + RECUR_BYTES_PER_TH   # = 1282
FLOPS_PER_TH = 6 * 128 * 128 + (6 * 128 + 4 * 128) * 16     # chunked form at C = 16


def state_bytes(inp):
    if inp.state_dtype is None:
        return 0
    per = 2 if inp.state_dtype == "bf16" else 4
    n = inp.N * inp.H * inp.V * inp.K * per
    return n * ((inp.initial_state is not None) + int(inp.output_final_state))


def param_bytes(inp):
    return inp.H * 4 + inp.H * inp.K * 4


def timed_repeats(torch, step, steps, warmup, repeats):
    """W warmup calls, then `repeats` runs of `steps` calls each, every run
    bracketed by device synchronisation; returns the per-call ms of each run."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    out = []
    for _ in range(repeats):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(steps):
            step()
        t1.record()
        torch.cuda.synchronize()
        out.append(t0.elapsed_time(t1) / steps)
    return out


def chunk_counts(inp, chunk):
    lens = [inp.T] * inp.B if inp.cu_seqlens is None else list(np.diff(inp.cu_seqlens))
    return [(int(n) + chunk - 1) // chunk for n in lens]


def run_workload(cfg, steps, warmup, torch, kda, device_inputs, chunk=None, path=None, precision=None,
                 repeats=1, inp=None, d=None):
    inp = cfg.make() if inp is None else inp
    d = device_inputs(inp, "cuda") if d is None else d
    out = torch.empty((inp.B, inp.T, inp.H, inp.V), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((inp.N, inp.H, inp.V, inp.K),
                      dtype=torch.bfloat16 if inp.state_dtype == "bf16" else torch.float32, device="cuda")
    path = path or "auto"
    if precision is not None:   # the precision study entry point: split path, 16-token chunks
        chunk, path = 16, "split"
    used = kda.path_used(chunk, None, path)
    ws = kda.alloc_workspace(inp.B, inp.T, inp.H, inp.N, inp.cu_seqlens is not None, "cuda", chunk, None, path)

    def step(events=None):
        if precision is not None:
            kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
                    inp.lower_bound, initial_state=d["initial_state"], final_state=fin,
                    cu_seqlens=d["cu_seqlens"], workspace=ws, precision=precision)
            return
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
                inp.lower_bound, initial_state=d["initial_state"], final_state=fin,
                cu_seqlens=d["cu_seqlens"], workspace=ws, events=events, chunk=chunk, path=path)

    reps = timed_repeats(torch, step, steps, warmup, repeats)
    ms = float(np.median(reps))
    th = inp.B * inp.T * inp.H
    if precision is not None:   # kda_fwd_precision records no events
        return dict(inp=inp, ms=ms, reps=reps, kernels={}, path=used, taken="split", token_heads=th,
                    status=kda.check_status(ws), chunk=16)

    # per-kernel durations: kda_fwd_ex records HIP events before and after
    # every kernel on the stream it launches that kernel on
    n_prof = max(steps, 5)
    n_ev = kda.num_events(inp.B, inp.T, chunk, None, path)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(n_prof)]
    for row in ev:
        for e in row:
            e.record()          # creates the underlying HIP event
    torch.cuda.synchronize()
    for row in ev:
        step(events=row)
    torch.cuda.synchronize()
    span = lambda row, i: row[i].elapsed_time(row[i + 1])
    if used == "fused":         # [0, 1] scheduler, [2, 3] the fused kernel
        k_ms = np.median(np.array([[span(row, 0), span(row, 2)] for row in ev]), axis=0)
        kernels = {"sched": float(k_ms[0]), "fused": float(k_ms[1])}
    else:                       # [0, 1] scheduler, then prep and recurrence of each part (+ [6, 7] fused)
        P = (n_ev - 2) // 4
        k_ms = np.median(np.array([[span(row, 0), sum(span(row, 2 + 2 * p) for p in range(P)),
                                    sum(span(row, 2 + 2 * P + 2 * p) for p in range(P))]
                                   + ([span(row, 6)] if used == "auto" else []) for row in ev]), axis=0)
        kernels = {"sched": float(k_ms[0]), "prep": float(k_ms[1]), "recur": float(k_ms[2])}
        if used == "auto":      # the kernels of the path not taken exit at once
            kernels["fused"] = float(k_ms[3])
    status = kda.check_status(ws)
    taken = kda.path_taken(ws)
    return dict(inp=inp, ms=ms, reps=reps, kernels=kernels, path=used, taken=taken, token_heads=th,
                status=status, chunk=chunk or 16)


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "hbm_traffic.md")


def load_traffic():
    """Per-kernel HBM bytes per dispatch from the committed counter summary,
    keyed by workload, or {} when the kernels changed since it was taken (the
    summary records a hash of the kernel sources)."""
    from gated_delta_rule_prep_amd import prof_summary
    try:
        with open(TRAFFIC_FILE) as f:
            entries = [json.loads(l.split("traffic-json:", 1)[1]) for l in f if l.startswith("traffic-json:")]
    except OSError:
        return {}
    cur = prof_summary.source_hash()
    return {e["workload"]: e["kernels"] for e in entries if e.get("source_hash") == cur}


CUS = 256   # compute units of a whole MI355X; main() reads the device's own count


def sequential_steps(inp, res):
    """Chunk steps one workgroup slot runs in sequence in the chain kernel:
    the longest sequence's chunk count (plus the fused kernel's five pipeline
    steps), or, when the launch has more workgroups than can run at once, the
    workgroup steps per slot.  Mirrors the library's tiling (kda_internal.h:
    recur_tiles, fused_two_tiles; two recurrence workgroups share a CU when
    64-column tiles outnumber the CUs)."""
    counts = chunk_counts(inp, res["chunk"])
    pairs = inp.N * inp.H
    if res["taken"] == "fused":
        tiles = 2 if 2 * pairs <= CUS else 1
        wg_steps, chain, slots = tiles * inp.H * sum(c + 5 for c in counts), max(counts) + 5, CUS
    else:
        if res["chunk"] == 32:
            tiles, per_cu = 2, 1
        else:
            equal = inp.cu_seqlens is None
            tiles = 4 if 4 * pairs <= CUS else (2 if 2 * pairs <= CUS or not equal else 1)
            per_cu = 2 if tiles == 2 and tiles * pairs > CUS else 1
        wg_steps, chain, slots = tiles * inp.H * sum(counts), max(counts), CUS * per_cu
    return max(chain, wg_steps / min(tiles * pairs, slots))


def roofline(res, traffic=None):
    inp, th, km = res["inp"], res["token_heads"], res["kernels"]
    prep_bytes = th * PREP_BYTES_PER_TH + param_bytes(inp)
    recur_bytes = th * RECUR_BYTES_PER_TH + state_bytes(inp)
    path_bytes = prep_bytes + recur_bytes
    if res["taken"] == "fused":   # one kernel moves every algorithmic byte of the path
        name, kbytes, kms = "kda::fused_kernel", path_bytes, km["fused"]
    elif km["recur"] >= km["prep"]:
        name, kbytes, kms = "kda::recur_kernel", recur_bytes, km["recur"]
    else:
        name, kbytes, kms = "kda::prep_kernel", prep_bytes, km["prep"]
    ach = kbytes / (kms * 1e-3) / 1e9
    t = (traffic or {}).get(name.split("::")[1])
    tbytes = None if t is None else int(t["fetch_bytes"] + t["write_bytes"])
    path_ms = res["ms"]
    path_ach = path_bytes / (path_ms * 1e-3) / 1e9
    steps = sequential_steps(inp, res)
    chain_ms = km["fused"] if res["taken"] == "fused" else km["recur"]
    res["us_per_chunk_step"] = round(1e3 * chain_ms / steps, 4) if steps > 0 else None
    return dict(kernel=name, bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(ach / HBM_PEAK_GBS, 4), traffic=tbytes, kernel_ms=round(kms, 4),
                algorithmic_bytes_per_launch=int(kbytes)), \
        dict(bound="hbm", achieved=round(path_ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
             frac=round(path_ach / HBM_PEAK_GBS, 4), algorithmic_bytes=int(path_bytes),
             mfma_frac=round(th * FLOPS_PER_TH / (path_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4))


DECODE_N, DECODE_H = 256, 96   # one decode step of a serving batch: 256 sequences, 96 heads


def run_decode(steps, warmup, torch, kda, device_inputs, repeats=1):
    """kda_decode on a batch of DECODE_N one-token sequences, bf16 state updated
    in place (the state is 805 MB, past the 256 MB Infinity Cache, so every
    step streams it from and to HBM).  Roofline: the state bytes (in + out) and
    the token bytes per launch over the median step time."""
    from gated_delta_rule_prep_amd.inputs import make_inputs
    inp = make_inputs(DECODE_N, 1, DECODE_H, seed=9, state_dtype="bf16", name="decode_N256_H96_bf16state")
    d = device_inputs(inp, "cuda")
    st = d["initial_state"]
    out = torch.empty((DECODE_N, 1, DECODE_H, 128), dtype=torch.bfloat16, device="cuda")

    def step():
        kda.decode(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
                   inp.lower_bound, initial_state=st, final_state=st)

    ms = float(np.median(timed_repeats(torch, step, steps, warmup, repeats)))
    pairs = DECODE_N * DECODE_H
    nbytes = pairs * (2 * 128 * 128 * 2 + PATH_BYTES_PER_TH) + param_bytes(inp)
    ach = nbytes / (ms * 1e-3) / 1e9
    return {"workload": inp.name, "ms_per_step": round(ms, 4), "token_heads_per_s": round(pairs / (ms * 1e-3), 1),
            "roofline": {"kernel": "kda::decode_kernel", "bound": "hbm", "achieved": round(ach, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": int(nbytes)}}


def run_segmented(steps, warmup, torch, kda, device_inputs, T=8192, H=4, repeats=1):
    """One long sequence with few heads, the case the segmented forward is for:
    kda_fwd (which cuts the sequence into the library's count of segments here)
    next to kda_fwd_ex with the library's path (one chain per head and value
    tile), on the same synthetic inputs (fp32 state)."""
    from gated_delta_rule_prep_amd.inputs import make_inputs
    inp = make_inputs(1, T, H, seed=7, state_dtype="fp32")
    d = device_inputs(inp, "cuda")
    out = torch.empty((1, T, H, 128), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((1, H, 128, 128), dtype=torch.float32, device="cuda")
    S = kda.segments_for(1, T, H)
    ws = kda.alloc_workspace(1, T, H, 1, False, "cuda")   # every form kda_fwd may take

    def timed(path):
        f = lambda: kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], inp.scale, out, d["A_log"], d["dt_bias"],
                            inp.lower_bound, initial_state=d["initial_state"], final_state=fin,
                            workspace=ws, path=path)
        return float(np.median(timed_repeats(torch, f, steps, warmup, repeats)))

    chain = timed("auto")   # kda_fwd_ex: never cuts
    seg = timed(None)       # kda_fwd
    return {"workload": "T%d_H%d_fixed_fp32state" % (T, H), "segments": S, "ms_per_step": round(seg, 4),
            "one_chain_ms": round(chain, 4), "value": round(T * H / (seg * 1e-3), 1),
            "speedup_vs_one_chain": round(chain / seg, 3), "status_ok": kda.check_status(ws) == 0}


def cpu_baseline(cfg, heads: int):
    """The fp64 oracle on the first `heads` heads of the workload (all tokens)."""
    import oracle
    inp = cfg.make()
    hs = list(range(heads))
    sl = lambda x: np.ascontiguousarray(x[:, :, hs])
    s0 = inp.initial_state_f64()
    threads = len(os.sched_getaffinity(0))
    t = time.perf_counter()
    oracle.kda_fwd(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.g), sl(inp.beta), inp.scale, inp.A_log[hs].copy(),
                   inp.dt_bias[hs].copy(), inp.lower_bound,
                   initial_state=None if s0 is None else np.ascontiguousarray(s0[:, hs]),
                   cu_seqlens=inp.cu_seqlens, threads=threads)
    dt = time.perf_counter() - t
    th = inp.B * inp.T * heads
    return dict(value=round(th / dt, 1), unit="token·heads/s", cores=threads, kind="oracle",
                sample="%s, heads 0..%d of %d, all %d tokens (%d token-heads), fp64 token-by-token, %.2f s wall"
                % (cfg.name, heads - 1, inp.H, inp.T, th, dt), cpu_model=cpu_model())


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_for_counters(torch, mib):
    """Three device-to-device copies of `mib` MiB: a plain copy kernel of known
    size whose byte counters scale the workload's (prof_summary traffic)."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 3}))


def copy_bandwidth(torch, mib=1024, reps=20):
    """The box's device-to-device copy rate (read + written bytes per second,
    torch's copy of `mib` MiB, median of `reps` event-timed copies): the
    practical streaming ceiling the kernels are read against."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ms = sorted(ts)[len(ts) // 2]
    del src, dst
    return {"GB_per_s": round(2 * n / ms / 1e6, 1), "bytes_copied": n, "ms": round(ms, 4)}


def workload_entry(cfg, runs, paths, traffic):
    """One workload's entry of the JSON line: the library's choice (runs[0])
    with its roofline, per-kernel times and us per chunk step, and every
    timed path's median step time."""
    res = runs[paths[0]]
    rl, prl = roofline(res, traffic.get(cfg.name))
    inp = res["inp"]
    return {"workload": cfg.name, "B": inp.B, "T": inp.T, "H": inp.H, "N": inp.N,
            "state": inp.state_dtype, "lower_bound": inp.lower_bound,
            "path": res["path"], "path_taken": res["taken"], "chunk": res["chunk"],
            "ms_per_step": round(res["ms"], 4),
            "ms_repeats": {"min": round(min(res["reps"]), 4), "max": round(max(res["reps"]), 4)},
            "value": round(res["token_heads"] / (res["ms"] * 1e-3), 1),
            "kernels_ms": {k: round(v, 4) for k, v in res["kernels"].items()},
            "us_per_chunk_step": res["us_per_chunk_step"],
            "paths_ms": {p: round(runs[p]["ms"], 4) for p in paths},
            "roofline": rl, "path_roofline": prl, "status": res["status"]}


# (label, chunk, path) of the forms timed per workload; the first is the library's choice
FORMS = [("auto", None, "auto"), ("split16", 16, "split"), ("fused16", 16, "fused"), ("split32", 32, "split"),
         ("split64", 64, "split")]
ONLY = {"fixed": 2, "varlen": 3}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--repeats", type=int, default=5, help="timed runs of --steps calls; the median is reported")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--cpu-heads", type=int, default=96, help="heads of the headline workload the oracle runs")
    ap.add_argument("--only", default="all",
                    choices=["all", "0", "1", "2", "3", "4", "fixed", "varlen", "decode", "segmented"],
                    help="time only one workload (for profiler runs: 0-4, fixed = 2, varlen = 3); the JSON "
                         "line needs all")
    ap.add_argument("--chunk", type=int, default=0, choices=[0, 16, 32, 64],
                    help="with --only: tokens per chunk (0: the library's choice)")
    ap.add_argument("--path", choices=["auto", "fused", "split"], default="auto",
                    help="with --only: execution path of kda_fwd_ex (auto: the library's choice)")
    ap.add_argument("--precision", type=int, default=None, choices=list(range(16)),
                    help="with --only 0-4: time kda_fwd_precision with this KDA_PREC_* variant")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="with --only: afterwards run 3 device-to-device copies of this many MiB, a plain copy "
                         "kernel of known size that scales the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the forward runs on one GPU's share of the heads and sequences, "
              "which shard across GPUs with no communication; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_prep_amd import kda
    from gated_delta_rule_prep_amd.inputs import configs
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from tests.kda_gpu import device_inputs

    global CUS
    CUS = torch.cuda.get_device_properties(0).multi_processor_count or CUS
    cfgs = configs()
    R = max(1, args.repeats)
    if args.only == "decode":
        print(json.dumps(run_decode(args.steps, args.warmup, torch, kda, device_inputs, R)))
        if args.copy_mib > 0:
            copy_for_counters(torch, args.copy_mib)
        return
    if args.only == "segmented":
        print(json.dumps(run_segmented(args.steps, args.warmup, torch, kda, device_inputs, repeats=R)))
        return
    if args.only != "all":
        cfg = cfgs[ONLY.get(args.only, None) if args.only in ONLY else int(args.only)]
        res = run_workload(cfg, args.steps, args.warmup, torch, kda, device_inputs, args.chunk or None, args.path,
                           args.precision, repeats=R)
        print(json.dumps({"workload": res["inp"].name, "path": res["path"], "path_taken": res["taken"],
                          "chunk": res["chunk"], "precision": args.precision,
                          "ms_per_step": round(res["ms"], 4), "ms_repeats": [round(x, 4) for x in res["reps"]],
                          "kernels_ms": {k: round(v, 4) for k, v in res["kernels"].items()}}))
        if args.copy_mib > 0:
            copy_for_counters(torch, args.copy_mib)
        return

    traffic = load_traffic()
    entries = []
    for cfg in cfgs:
        inp = cfg.make()
        d = device_inputs(inp, "cuda")
        runs = {label: run_workload(cfg, args.steps, args.warmup, torch, kda, device_inputs, chunk, pth,
                                    repeats=R, inp=inp, d=d) for label, chunk, pth in FORMS}
        entries.append(workload_entry(cfg, runs, [f[0] for f in FORMS], traffic))
        del d, runs
        torch.cuda.empty_cache()
    head = entries[2]
    decode = run_decode(args.steps, args.warmup, torch, kda, device_inputs, R)
    t = traffic.get(decode["workload"], {}).get("decode_kernel")
    decode["roofline"]["traffic"] = None if t is None else int(t["fetch_bytes"] + t["write_bytes"])
    segmented = run_segmented(args.steps, args.warmup, torch, kda, device_inputs, repeats=R)
    cpu = None if args.no_cpu else cpu_baseline(cfgs[2], args.cpu_heads)
    line = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "token·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "repeats": R,
        "ms_per_step": head["ms_per_step"],
        "ms_repeats": head["ms_repeats"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in/out, fp16 and fp32 MFMA with fp32 accumulation, fp32 state on chip",
        "data": "synthetic (seeded normal q/k/v/g/beta, A_log=log U[1,16], dt_bias~N(0,0.1), state~N(0,0.05))",
        "config": {"workload": cfgs[2].name, "B": 1, "T": 8192, "H": 96, "K": 128, "V": 128,
                   "state": "bf16", "lower_bound": -5.0, "chunk": head["chunk"], "path": head["path"],
                   "path_taken": head["path_taken"]},
        "roofline": head["roofline"],
        "path_roofline": head["path_roofline"],
        "kernels_ms": head["kernels_ms"],
        "us_per_chunk_step": head["us_per_chunk_step"],
        "paths_ms": head["paths_ms"],
        "workloads": entries,
        "decode_256x96": decode,
        "segmented_8192x4": segmented,
        "status_ok": all(e["status"] == 0 for e in entries) and segmented["status_ok"],
        "cpu_baseline": cpu,
        "hbm_copy": copy_bandwidth(torch),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
