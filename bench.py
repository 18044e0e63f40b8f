#!/usr/bin/env python3
"""Benchmark of the capacity-limited MoE layer forward on one MI355X.

One step = one moe_layer_forward over a batch of synthetic input already resident in HBM:
router, dispatch (capacity cut, slot assignment), expert GEMM 1 (+bias, SiLU), expert GEMM 2
(+bias), combine.  Prints ONE JSON line:
  value          tokens/s of the whole layer (T / wall-clock time per step)
  roofline       the dominant kernel (the larger expert GEMM) against the bf16 MFMA peak; its
                 duration comes from HIP events that the GEMM kernel launches of the timed
                 steps record themselves (moe_set_gemm_timing, hipExtLaunchKernel), so the
                 steps `value` is timed on carry no extra marker between launches
  cpu_baseline   the CPU oracle timed on this host on the same workload (a baseline only)
  route_kernel_GBps, combine_kernel_GBps
                 the router's and the combine's bytes over their own kernel time (events that
                 their launches record, moe_set_stage_timing), from a run of plain steps after
                 the timed ones; route_GBps / combine_GBps use the stage events (gaps included)
Before the timed steps: at least --warmup untimed steps, continued until --warmup-ms (100 ms)
of wall time have passed, since the GPU reaches its steady clocks only after about 30 ms of
sustained load.  roofline.traffic: HBM bytes per launch of the dominant GEMM from two
rocprofv3 --pmc child runs of this command (skipped with --traffic none).
Workload: the mid-size layer (T 4096, d_model 2048, d_ff 8192, 8 experts, top-2, capacity
factor 1.25) unless --config names another.  --layout dropless times the dropless pair-order
flow instead (no capacity: pair dispatch, pair-order GEMMs with the top-k weight applied in
GEMM 2, moe_sum in place of the combine).  --config decode_pool times a pool of decode batches
run one after another, in the original grouping and regrouped by the Token Scheduler; `value`
is the consolidated run's tokens/s.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import re
import shutil
import signal
import subprocess
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MoE-layer tokens/s; expert GEMM TFLOP/s as % of MI355X bf16 peak"
STAGES = ["route", "dispatch", "expert_up", "expert_down", "combine"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_digest(path: str) -> str:
    """SHA-256 of a source file with its comments and blank space removed, so that a counter
    summary stays tied to the code and survives comment-only edits."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(re.sub(r"\s+", " ", text).strip().encode()).hexdigest()


GEMM_SOURCE = os.path.join(ROOT, "capacity_routing_expert_amd", "csrc", "gemm_bf16.hip")


def warm_up(step, min_steps: int, min_ms: float, sync) -> dict:
    """Untimed warm-up: at least `min_steps` steps, continued until `min_ms` of wall time have
    passed (checked every 8 steps, after a sync).  Under sustained load this GPU takes about
    30 ms to settle: the mid layer's step time falls from about 516 to 400 us over its first
    60 to 80 steps, and ramps again after two idle seconds."""
    t0 = time.perf_counter()
    n = 0
    while True:
        step()
        n += 1
        if n >= min_steps and n % 8 == 0:
            sync()
            if (time.perf_counter() - t0) * 1e3 >= min_ms:
                break
    sync()
    return {"steps": n, "ms": (time.perf_counter() - t0) * 1e3}


def traffic_from_profiles(kernel_tag: str, config_key: str):
    """HBM bytes per launch of the dominant kernel from a committed counter summary, scaled by
    the copy-kernel calibration, or None if no summary matches the current kernel code."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_{config_key}_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = {k: re.search(rf"^{k}\s*=\s*(\S+)", text, re.M) for k in
         ("code_sha256", "fetch_kib_per_dispatch", "write_kib_per_dispatch", "fetch_scale",
          "write_scale")}
    if not all(m.values()):
        return None
    if code_digest(GEMM_SOURCE) != m["code_sha256"].group(1):
        return None  # the kernel code changed since the counters were taken
    kib = (float(m["fetch_kib_per_dispatch"].group(1)) * float(m["fetch_scale"].group(1)) +
           float(m["write_kib_per_dispatch"].group(1)) * float(m["write_scale"].group(1)))
    return kib * 1024.0


def traffic_live(args):
    """HBM bytes per launch of the two expert GEMMs, measured on this machine: two child runs
    of this same command under rocprofv3 --pmc (FETCH_SIZE, then WRITE_SIZE; 8 warm-up and 3
    timed steps, plus a 1 GiB device copy as the calibration), started before this process
    touches the GPU.  FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by what it reads
    for the copy.  Returns {"expert_up": bytes, "expert_down": bytes, ...} or None when
    rocprofv3 is missing, a run fails or times out (its process group is then killed)."""
    prof = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
    if not os.path.exists(prof):
        return None
    base = tempfile.mkdtemp(prefix="moe_bench_pmc_", dir=os.environ.get("TMPDIR", "/tmp"))
    vals = {}
    try:
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            out = os.path.join(base, ctr)
            cmd = [prof, "--pmc", ctr, "-f", "csv", "-d", out, "-o", "run", "--", sys.executable,
                   os.path.abspath(__file__), "--config", args.config, "--layout", args.layout,
                   "--weights", args.weights, "--steps", "3", "--warmup", "1",
                   "--warmup-ms", "0", "--no-cpu-baseline", "--copy-probe", "--traffic", "none"]
            log(f"[bench] HBM counters: {ctr} child run")
            # the child's progress lines go to stderr; its JSON line is dropped
            child = subprocess.Popen(cmd, stdout=subprocess.DEVNULL, start_new_session=True,
                                     cwd=ROOT)
            try:
                rc = child.wait(timeout=240)
            except subprocess.TimeoutExpired:
                os.killpg(child.pid, signal.SIGKILL)  # the group this call started
                child.wait()
                return None
            files = glob.glob(os.path.join(out, "**", "*counter_collection.csv"), recursive=True)
            if rc != 0 or not files:
                return None
            with open(files[0]) as f:
                vals[ctr] = sorted((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]),
                                    float(r["Counter_Value"])) for r in csv.DictReader(f)
                                   if r["Counter_Name"] == ctr)
    finally:
        shutil.rmtree(base, ignore_errors=True)

    return pmc_gemm_traffic(vals)


def pmc_gemm_traffic(vals):
    """Per-launch HBM bytes of the two expert GEMMs from rocprofv3 counter rows.  vals maps
    "FETCH_SIZE" and "WRITE_SIZE" to (dispatch id, kernel name, grid size, KiB) in dispatch
    order.  In each layer call GEMM 1 is the first grouped-GEMM launch after the router and
    GEMM 2 the next one; each counter is scaled by what it reads for the largest device copy
    (the 1 GiB calibration copy, 1 GiB read and 1 GiB written)."""
    def scale(ctr):
        copies = [v for v in vals[ctr] if v[1].startswith("__amd_rocclr_copyBuffer")]
        big = max(copies, key=lambda v: v[2]) if copies else None
        return (1 << 30) / (big[3] * 1024.0) if big and big[3] > 0 else None

    def per_gemm(ctr):
        g = ([], [])
        state = 0
        for _, name, _, v in vals[ctr]:
            if "k_route" in name:
                state = 1
            elif "k_grouped_gemm" in name and state in (1, 2):
                g[state - 1].append(v)
                state += 1
        return [float(np.mean(x)) if x else None for x in g]

    fs, ws = scale("FETCH_SIZE"), scale("WRITE_SIZE")
    f1, f2 = per_gemm("FETCH_SIZE")
    w1, w2 = per_gemm("WRITE_SIZE")
    if None in (fs, ws, f1, f2, w1, w2):
        return None
    return {"expert_up": (f1 * fs + w1 * ws) * 1024.0, "expert_down": (f2 * fs + w2 * ws) * 1024.0,
            "fetch_scale": fs, "write_scale": ws}


def cpu_baseline(inp, wl, cap, dropless=False):
    """The oracle on this host: the whole layer on the same workload, repeated for about 10 s."""
    import oracle.moe_oracle as O
    from capacity_routing_expert_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    dt = inp["dtype"]
    x = W.to_float64(inp["x"], dt)
    wr = W.to_float64(inp["w_router"], dt)

    class F64:
        def __init__(self, a):
            self.a = a

        def __getitem__(self, e):
            return W.to_float64(self.a[e], dt)

    # the whole layer on the full batch, repeated until about 10 s of host time has been spent
    # (at least once); the mean time per run gives tokens/s
    times = []
    while not times or (sum(times) < 10.0 and len(times) < 20):
        t0 = time.perf_counter()
        r = O.route(x, wr, inp["b_router"], wl.top_k)
        if dropless:
            if wl.expert == "gated":
                w13, w2 = F64(inp["w1"]), F64(inp["w2"])
                fn = lambda e, rows: O.expert_ffn_gated(rows, w13[e], w2[e])
            else:
                w1, b1, w2, b2 = (F64(inp[n]) for n in ("w1", "b1", "w2", "b2"))
                fn = lambda e, rows: O.expert_ffn(rows, w1[e], b1[e], w2[e], b2[e])
            O.forward_dropless_with_routing(x, r["ids"], r["gates"], wl.n_experts, fn)
            res = {"n_kept": wl.T * wl.top_k}
        elif wl.expert == "gated":
            disp = O.dispatch(r["ids"], r["gates"], wl.n_experts, cap)
            Y = O.expert_ffn_slots_gated(x, disp["row_token"], disp["offsets"], F64(inp["w1"]),
                                         F64(inp["w2"]))
            O.combine(x, r["gates"], disp["slot_of"], Y)
            res = disp
        else:
            res = O.forward_with_routing(x, r["ids"], r["gates"], cap, wl.n_experts,
                                         F64(inp["w1"]), F64(inp["b1"]), F64(inp["w2"]),
                                         F64(inp["b2"]))
        times.append(time.perf_counter() - t0)
    t = float(np.mean(times))
    # the per-expert float64 weight conversion is inside the timed region: it is part of
    # what the oracle does to evaluate the layer
    # expert-GEMM FLOP of the layer (a gated expert's GEMM 1 has 2 d_ff outputs) over the whole
    # oracle layer's time
    flop = 2 * int(res["n_kept"]) * wl.d_model * wl.d_ff * (3 if wl.expert == "gated" else 2)
    return {"value": wl.T / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"whole layer on the full {wl.name} batch ({wl.T} tokens), "
                      f"{len(times)} runs, {t:.2f} s each, float64 NumPy/BLAS",
            "seconds": round(t, 3),
            "n_kept": int(res["n_kept"]),
            "expert_gemm_gflops": round(flop / t / 1e9, 1)}


def bench_pool(args, wl, inp):
    """A pool of batches, one after another: the original grouping against the Token
    Scheduler's.  Roofline: the pool is bound by streaming the active experts' weights once per
    batch; achieved = those weight bytes / the batch loop's event-bracketed time (dispatch and
    combine included)."""
    import torch
    from capacity_routing_expert_amd import binding as B
    from capacity_routing_expert_amd import layer as L

    dev = torch.device("cuda:0")
    d = L.upload(inp, dev)
    if args.weights == "packed":
        d = L.pack_weights(d)
    Bsz = wl.batch_size
    M = wl.T // Bsz
    cap = B.capacity(Bsz, wl.top_k, wl.n_experts, wl.capacity_factor)
    dtype = B.MOE_BF16 if wl.dtype == "bf16" else B.MOE_F32
    shape = B.make_shape(Bsz, wl.d_model, wl.d_ff, wl.n_experts, wl.top_k, cap, dtype,
                         d.get("weight_layout", B.MOE_WEIGHTS_ROW_MAJOR))
    ws = torch.empty(max(B.workspace_bytes_batches(shape, M), 256), dtype=torch.uint8, device=dev)
    out = torch.empty_like(d["x"])
    bexp = torch.empty((M,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    esz = inp["x"].itemsize
    w_bytes = (2 * wl.d_model * wl.d_ff + wl.d_ff + wl.d_model) * esz  # one expert's W1 b1 W2 b2

    def run(cons, events=None):
        B.moe_layer_forward_batches(shape, M, cons, d["x"], d["w_router"], d["b_router"], d["w1"],
                                    d["b1"], d["w2"], d["b2"], out, batch_experts=bexp, ws=ws,
                                    events=events)

    result = {}
    warm = {}
    for cons in (False, True):
        warm[cons] = warm_up(lambda: run(cons), args.warmup, args.warmup_ms, torch.cuda.synchronize)
        evsets = []
        for _ in range(args.steps):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            for ev in evs:
                ev.record(stream)  # creates the underlying hipEvent_t
            evsets.append(evs)
        # timed region: the stage events are recorded by the timed steps themselves
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for evs in evsets:
            run(cons, evs)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / args.steps
        st = {name: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evsets]))
              for j, name in enumerate(["route", "schedule", "batches", "scatter"])}
        active = [int(v) for v in bexp.cpu().numpy()]
        loop_s = st["batches"] / 1e3
        result[cons] = {"tokens_per_s": wl.T / wall, "ms_per_step": wall * 1e3, "stages_ms": st,
                        "active_experts": active,
                        "mean_active_experts": float(np.mean(active)),
                        "tokens_per_active_expert": float(Bsz * wl.top_k / np.mean(active)),
                        "weight_GBps": sum(active) * w_bytes / loop_s / 1e9}
    c, o = result[True], result[False]
    res = {
        "metric": METRIC,
        "value": c["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": c["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded numpy PCG64 draws of the workload's shapes and distributions)",
        "config": {"workload": wl.name, "T": wl.T, "batch_size": Bsz, "n_batches": M,
                   "d_model": wl.d_model, "d_ff": wl.d_ff, "n_experts": wl.n_experts,
                   "top_k": wl.top_k, "capacity_factor": wl.capacity_factor, "capacity": cap,
                   "layout": "batches, Token Scheduler regrouping", "weights": args.weights},
        "roofline": {"kernel": "k_grouped_gemm skinny tiles (active experts' weight stream), "
                               "batch loop", "bound": "hbm", "achieved": c["weight_GBps"],
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": c["weight_GBps"] / PEAK_HBM_GBS,
                     "traffic": None,
                     "units_per_launch": f"{sum(c['active_experts'])} active (batch, expert) "
                                         f"pairs x {w_bytes} B of weights"},
        "warmup_run": {"consolidated": warm[True], "original": warm[False]},
        "consolidated": c,
        "original": o,
        "speedup_vs_original": c["tokens_per_s"] / o["tokens_per_s"],
        "stage_timing": "HIP events recorded by the timed steps themselves: route, schedule + "
                        "regroup, batch loop, scatter back",
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline_pool(inp, wl)
    print(json.dumps(res), flush=True)


def bench_shard(args, wl, inp):
    """One GPU's share under expert parallelism: the expert FFN (moe_expert_ffn, both GEMMs) of
    the one expert this GPU owns, over the rows it received (x rows in receive order, all kept).
    The all-to-all exchanges around it are not built; the roofline is the dominant GEMM's kernel
    time, recorded by its launch in each timed step."""
    import torch
    from capacity_routing_expert_amd import binding as B
    from capacity_routing_expert_amd import layer as L

    dev = torch.device("cuda:0")
    d = L.upload(inp, dev)
    if args.weights == "packed":
        d = L.pack_weights(d)
    rows = wl.T
    shape = L.shape_of(d, wl.top_k, rows)
    ws = L.workspace(shape, dev)
    row_token = torch.arange(rows, dtype=torch.int32, device=dev)
    offsets = torch.tensor([0, rows], dtype=torch.int32, device=dev)
    y = torch.empty((rows, wl.d_model), dtype=d["x"].dtype, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        B.moe_expert_ffn(shape, d["x"], row_token, offsets, d["w1"], d["b1"], d["w2"], d["b2"],
                         y, ws)

    def new_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for ev in evs:
            ev.record(stream)
        return evs

    log(f"[bench] warmup {args.warmup} steps, {args.warmup_ms:.0f} ms at least")
    warm = warm_up(step, args.warmup, args.warmup_ms, torch.cuda.synchronize)
    evsets = [new_events(4) for _ in range(args.steps)]
    arms = [(ctypes.c_void_p * 4)(*[ctypes.c_void_p(ev.cuda_event) for ev in evs])
            for evs in evsets]
    set_timing = B.lib().moe_set_gemm_timing
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if set_timing(arms[i]) != 0:
            raise RuntimeError(B.last_error())
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    up_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evsets]))
    down_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evsets]))
    flop = 2.0 * rows * wl.d_model * wl.d_ff  # per GEMM
    dom = "expert_up" if up_ms >= down_ms else "expert_down"
    dom_ms = max(up_ms, down_ms)
    achieved = flop / (dom_ms / 1e3) / 1e12
    res = {
        "metric": "expert FFN rows/s of one GPU's share (expert parallel over 8 GPUs, the hot "
                  "expert's owner); expert GEMM TFLOP/s as % of MI355X bf16 peak",
        "value": rows / wall,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy PCG64 draws of the workload's shapes and distributions)",
        "config": {"workload": wl.name, "rows": rows, "d_model": wl.d_model, "d_ff": wl.d_ff,
                   "n_experts_on_this_gpu": 1, "weights": args.weights,
                   "step": "moe_expert_ffn: GEMM 1 (gather by row_token + W1 + b1 + SiLU), "
                           "GEMM 2 (W2 + b2); no routing, dispatch, exchange or combine"},
        "roofline": {"kernel": "k_grouped_gemm, 8 waves (GEMM 1)" if dom == "expert_up"
                               else "k_grouped_gemm_loaders (GEMM 2)",
                     "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "units_per_launch": f"{rows} rows x 2*{wl.d_model}*{wl.d_ff} FLOP"},
        "gemm_kernel_ms": {"expert_up": up_ms, "expert_down": down_ms},
        "expert_gemm_tflops": 2 * flop / ((up_ms + down_ms) / 1e3) / 1e12,
        "expert_gemm_frac_of_bf16_peak": 2 * flop / ((up_ms + down_ms) / 1e3) / 1e12
                                         / PEAK_BF16_TFLOPS,
        "cpu_baseline": None,
        "warmup_run": warm,
        "gemm_timing": "start and end of each GEMM's kernel, recorded by its launch in each timed "
                       "step (moe_set_gemm_timing), averaged over the K steps",
    }
    print(json.dumps(res), flush=True)


def cpu_baseline_pool(inp, wl):
    """The oracle's pooled layer (route, Token Scheduler, per-batch layer) on this host."""
    import oracle.moe_oracle as O
    from capacity_routing_expert_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    dt = inp["dtype"]
    f = {n: W.to_float64(inp[n], dt) for n in ("x", "w_router", "w1", "b1", "w2", "b2")}
    times = []
    while not times or (sum(times) < 10.0 and len(times) < 20):
        t0 = time.perf_counter()
        O.forward_batches(f["x"], f["w_router"], inp["b_router"], f["w1"], f["b1"], f["w2"],
                          f["b2"], wl.top_k, wl.capacity_factor, wl.batch_size, True)
        times.append(time.perf_counter() - t0)
    t = float(np.mean(times))
    return {"value": wl.T / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"the whole consolidated pool ({wl.T} tokens in batches of "
                      f"{wl.batch_size}), {len(times)} runs, {t:.2f} s each, float64 NumPy/BLAS",
            "seconds": round(t, 3)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5,
                    help="warm-up steps before the timed ones (at least this many; see --warmup-ms)")
    ap.add_argument("--warmup-ms", type=float, default=100.0,
                    help="keep warming up until this much wall time has passed: the GPU needs "
                         "about 30 ms of sustained load to reach its steady clocks")
    ap.add_argument("--config", default="mid",
                    help="worked_example | mid | fine | decode | collapse | gated | decode_pool | "
                         "ep8_hot_shard")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layout", default="compact", choices=["compact", "padded", "dropless"],
                    help="compact: the expert FFN runs over the kept rows only; padded: over "
                         "every slot of the fixed per-expert buffers (n_experts x capacity rows); "
                         "dropless: no capacity, every (token, choice) pair in pair order")
    ap.add_argument("--weights", default="packed", choices=["packed", "rowmajor"],
                    help="expert weight storage: packed by moe_pack_weights once before timing "
                         "(K-block-major, the expert GEMMs' read order), or row-major [E, rows, "
                         "cols]; the results are bit-identical")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--traffic", default="live", choices=["live", "profiles", "none"],
                    help="roofline.traffic: live = two rocprofv3 --pmc child runs of this "
                         "command (FETCH_SIZE, WRITE_SIZE) before the measurement; profiles = "
                         "the committed counter summary of the current kernel code; none")
    ap.add_argument("--flush", action="store_true",
                    help="also time K steps each preceded by a 512 MiB write on the stream (the "
                         "Infinity Cache and the L2s hold none of the step's data), reporting the "
                         "median and mean per-step time beside the steady-state value")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the layer's "
              "multi-GPU sharding (expert parallel, all-to-all exchange of kept rows) is a "
              "design, not built", file=sys.stderr)
        sys.exit(2)
    # live HBM counters of the compact layout's expert GEMMs, taken before this process touches
    # the GPU (the counter runs are child processes of their own)
    import torch  # device_count() does not initialise the GPU: the counter runs start first

    from capacity_routing_expert_amd import workloads as W

    live = None
    wl0 = W.WORKLOADS.get(args.config)
    if (args.traffic == "live" and args.layout == "compact" and wl0 is not None
            and wl0.dtype == "bf16" and not wl0.batch_size and wl0.key != "ep8_hot_shard"
            and torch.cuda.device_count() > 0):
        live = traffic_live(args)

    from capacity_routing_expert_amd import binding as B
    from capacity_routing_expert_amd import layer as L

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.lib()
    dev = torch.device("cuda:0")
    wl = W.WORKLOADS[args.config]
    cap = B.capacity(wl.T, wl.top_k, wl.n_experts, wl.capacity_factor)
    log(f"[bench] generating {wl.name}")
    inp = W.make_inputs(wl)
    if wl.batch_size:
        bench_pool(args, wl, inp)
        return
    if wl.key == "ep8_hot_shard":
        bench_shard(args, wl, inp)
        return
    d = L.upload(inp, dev)
    if args.weights == "packed" and inp["dtype"] != "bf16":
        args.weights = "rowmajor"  # the packed layout is bf16 only
    if args.weights == "packed":  # a one-time preparation of the weights, outside the timing
        d = L.pack_weights(d)
    shape = L.shape_of(d, wl.top_k, cap)
    padded = args.layout == "padded"
    dropless = args.layout == "dropless"
    if padded:
        ws = torch.empty(max(B.workspace_bytes_padded(shape), 256), dtype=torch.uint8, device=dev)
    elif dropless:
        ws = L.workspace_dropless(shape, dev)
    else:
        ws = L.workspace(shape, dev)
    out = torch.empty_like(d["x"])
    counts = torch.empty((wl.n_experts,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    gated = wl.expert == "gated"
    if gated and padded:
        print("the padded layout is built for the FFN expert only", file=sys.stderr)
        sys.exit(2)

    def step_dropless(events=None):
        if gated:
            B.moe_layer_forward_dropless_gated(shape, d["x"], d["w_router"], d["b_router"],
                                               d["w1"], d["w2"], out, expert_counts=counts,
                                               ws=ws, events=events)
        else:
            B.moe_layer_forward_dropless(shape, d["x"], d["w_router"], d["b_router"], d["w1"],
                                         d["b1"], d["w2"], d["b2"], out, expert_counts=counts,
                                         ws=ws, events=events)

    def step():
        if dropless:
            step_dropless()
        elif gated:
            B.moe_layer_forward_gated(shape, d["x"], d["w_router"], d["b_router"], d["w1"],
                                      d["w2"], out, expert_counts=counts, ws=ws)
        elif padded:
            B.moe_layer_forward_padded(shape, d["x"], d["w_router"], d["b_router"], d["w1"],
                                       d["b1"], d["w2"], d["b2"], out, expert_counts=counts, ws=ws)
        else:
            B.moe_layer_forward(shape, d["x"], d["w_router"], d["b_router"], d["w1"], d["b1"],
                                d["w2"], d["b2"], out, expert_counts=counts, ws=ws)

    def step_profiled(events):
        if dropless:
            step_dropless(events)
        elif gated:
            B.moe_layer_forward_gated(shape, d["x"], d["w_router"], d["b_router"], d["w1"],
                                      d["w2"], out, expert_counts=counts, ws=ws, events=events)
        elif padded:
            B.moe_layer_forward_padded(shape, d["x"], d["w_router"], d["b_router"], d["w1"],
                                       d["b1"], d["w2"], d["b2"], out, expert_counts=counts,
                                       ws=ws, events=events)
        else:
            B.moe_layer_forward_profiled(shape, d["x"], d["w_router"], d["b_router"], d["w1"],
                                         d["b1"], d["w2"], d["b2"], out, events,
                                         expert_counts=counts, ws=ws)

    def new_events(n=6):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for ev in evs:
            ev.record(stream)  # creates the underlying hipEvent_t
        return evs

    log(f"[bench] warmup {args.warmup} steps, {args.warmup_ms:.0f} ms at least")
    warm = warm_up(step, max(args.warmup - 1, 0), args.warmup_ms, torch.cuda.synchronize)
    warm["steps"] += 1  # and the probe step below
    # the last warm-up step times both expert GEMMs' kernels, to find the dominant one
    probe = new_events(4)
    torch.cuda.synchronize()
    B.moe_set_gemm_timing(probe)
    step()
    torch.cuda.synchronize()
    dom = ("expert_up" if probe[0].elapsed_time(probe[1]) >= probe[2].elapsed_time(probe[3])
           else "expert_down")

    # timed region: K plain layer calls bracketed by a sync.  Each is armed with
    # moe_set_gemm_timing, so the dominant expert GEMM's kernel launch records its own start
    # and end in HIP events on the launch stream (hipExtLaunchKernel); the roofline's kernel
    # time comes from these very steps.
    gemm_evsets = [new_events(2) for _ in range(args.steps)]

    def arm_handles(evs):
        h = [ctypes.c_void_p(ev.cuda_event) for ev in evs]
        n = [ctypes.c_void_p(None)] * 2
        return (ctypes.c_void_p * 4)(*(h + n if dom == "expert_up" else n + h))

    arms = [arm_handles(evs) for evs in gemm_evsets]  # built ahead: the loop only passes them
    set_timing = B.lib().moe_set_gemm_timing
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if set_timing(arms[i]) != 0:
            raise RuntimeError(B.last_error())
        step()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    dom_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in gemm_evsets]))

    # stage breakdown (route, dispatch, combine): the same number of steps again, with HIP
    # events recorded between the stages (each such event adds a short launch gap, which is why
    # these are not the timed steps)
    evsets = [new_events() for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step_profiled(evsets[i])
    torch.cuda.synchronize()
    # the router's and the combine's own kernels, timed by their launches (moe_set_stage_timing,
    # hipExtLaunchKernel) over a third run of plain steps: the stage events above include
    # launch gaps
    route_kernel_ms = combine_kernel_ms = None
    if not dropless:
        kev = [new_events(4) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            B.moe_set_stage_timing(kev[i])
            step()
        torch.cuda.synchronize()
        route_kernel_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in kev]))
        combine_kernel_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in kev]))

    stage_ms = {s: float(np.mean([evs[j].elapsed_time(evs[j + 1]) for evs in evsets]))
                for j, s in enumerate(STAGES)}
    step_ms = float(np.mean([evs[0].elapsed_time(evs[5]) for evs in evsets]))
    c = counts.cpu().numpy()
    n_kept = int(c.sum()) if dropless else int(np.minimum(c, cap).sum())
    dm, ff = wl.d_model, wl.d_ff
    # kept rows only; a gated expert's first GEMM has 2 d_ff outputs (gate and up)
    gemm2_flop = 2.0 * n_kept * dm * ff
    gemm1_flop = 2.0 * gemm2_flop if gated else gemm2_flop
    expert_s = (stage_ms["expert_up"] + stage_ms["expert_down"]) / 1e3
    up_kernel = "k_grouped_gemm, 8 waves"  # the large-batch up-projection
    dom_kernel = {"expert_up": f"{up_kernel} (GEMM 1: gather + W1 + b1 + SiLU)",
                  "expert_down": "k_grouped_gemm_loaders (GEMM 2: W2 + b2)"}[dom]
    if dropless:
        dom_kernel = {"expert_up": f"{up_kernel} (GEMM 1 in pair order: row p // top_k in, "
                                   "row p out)",
                      "expert_down": "k_grouped_gemm_loaders (GEMM 2 in pair order: x topk_weights[p])"}[dom]
    gemm_flop = gemm1_flop if dom == "expert_up" else gemm2_flop
    achieved = gemm_flop / (dom_ms / 1e3) / 1e12  # the timed steps' kernel time
    roof = {"kernel": dom_kernel, "bound": "mfma", "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
            "units_per_launch": f"{n_kept} kept rows x 2*{dm}*{ff}"
                                f"{'*2' if gated and dom == 'expert_up' else ''} FLOP"}
    # decode-sized batches (the library's small-tile rule: at most 64 rows per expert on
    # average) stream the active experts' weights: the GEMM is bound by HBM
    rows_ub = (wl.n_experts * cap if padded else wl.T * wl.top_k if dropless
               else min(wl.T * wl.top_k, wl.n_experts * cap))
    if rows_ub <= 64 * wl.n_experts:
        esz = inp["x"].itemsize
        active = int(np.count_nonzero(c if dropless else np.minimum(c, cap)))
        rows = n_kept if not padded else wl.n_experts * cap
        if dom == "expert_up":  # W1 (W13) + b1 of each active expert, x rows in, H rows out
            w = ((2 if gated else 1) * ff * dm + (0 if gated else ff)) * esz
            act = rows * (dm + ff) * esz
        else:  # W2 + b2, H rows in, Y rows out
            w = (dm * ff + (0 if gated else dm)) * esz
            act = rows * (ff + dm) * esz
        gbs = (active * w + act) / (dom_ms / 1e3) / 1e9
        small_kernel = ("k_grouped_gemm, decode-sized tiles ("
                        + ("GEMM 1: 128 x 32 tiles" if dom == "expert_up" and not gated else
                           "GEMM 1: 128 x 64 gate/up tiles" if dom == "expert_up" else
                           "GEMM 2: 64 x 64 tiles") + ")")
        roof = {"kernel": small_kernel, "bound": "hbm", "achieved": gbs,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                "units_per_launch": f"{active} active experts x {w} B of weights + {act} B of "
                                    f"activations ({rows} rows)",
                "tflops": achieved}
    # HBM bytes of the dominant GEMM per launch: the live counter runs, else the committed
    # counter summary when it is of the current kernel code (both are of the compact layout)
    traffic, traffic_src = None, None
    if live is not None:
        traffic, traffic_src = live[dom], ("live: rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE child "
                                           f"runs, copy scale {live['fetch_scale']:.3f} / "
                                           f"{live['write_scale']:.3f}")
    elif not padded and not dropless and args.traffic != "none":
        traffic = traffic_from_profiles("gemm1" if dom == "expert_up" else "gemm2", args.config)
        traffic_src = "committed counter summary" if traffic is not None else None

    route_bytes = wl.T * dm * inp["x"].itemsize + wl.n_experts * dm * inp["x"].itemsize + 8 * wl.T * wl.top_k
    # combine: x, the kept Y rows, out, gates + slots; moe_sum: x, the T * k pair rows, out, ids
    combine_bytes = ((2 * wl.T + n_kept) * dm * inp["x"].itemsize
                     + (4 if dropless else 8) * wl.T * wl.top_k)

    # the optional x_routed output of moe_dispatch (the token rows copied into slot order), an
    # HBM-bound gather of N_kept rows: K staged dispatch calls without it and K with it, each
    # bracketed by events; the difference is the gather
    x_routed_res = None
    if not padded and not dropless:
        rt = L.route(d, wl.top_k, cap, ws=ws)
        plain_ev = [new_events(2) for _ in range(args.steps)]
        gather_ev = [new_events(2) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for evs, with_x in ((plain_ev, False), (gather_ev, True)):
            for i in range(args.steps):
                evs[i][0].record(stream)
                L.dispatch(shape, rt["ids"], rt["gates"], ws, x=d["x"] if with_x else None)
                evs[i][1].record(stream)
        torch.cuda.synchronize()
        t_plain = float(np.median([e[0].elapsed_time(e[1]) for e in plain_ev]))
        t_gather = float(np.median([e[0].elapsed_time(e[1]) for e in gather_ev]))
        gather_bytes = 2 * n_kept * dm * inp["x"].itemsize
        x_routed_res = {"dispatch_ms": t_plain, "dispatch_with_x_routed_ms": t_gather,
                        "gather_bytes": gather_bytes,
                        "gather_GBps": gather_bytes / max(t_gather - t_plain, 1e-6) * 1e3 / 1e9}
        del rt

    flush_res = None
    if args.flush:
        # cold-cache steps: a 512 MiB write (twice the 256 MiB Infinity Cache) before each one;
        # events bracket the step alone, so the flush is not counted
        fbuf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        fev = [new_events(2) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            fbuf.fill_(i & 0xFF)
            fev[i][0].record(stream)
            step()
            fev[i][1].record(stream)
        torch.cuda.synchronize()
        per = np.array([e[0].elapsed_time(e[1]) for e in fev])
        flush_res = {"median_ms": float(np.median(per)), "mean_ms": float(np.mean(per)),
                     "min_ms": float(per.min()), "max_ms": float(per.max()),
                     "tokens_per_s_median": wl.T / (float(np.median(per)) / 1e3),
                     "steady_state_median_ms": None,
                     "flush_bytes": 512 << 20}
        del fbuf
        # the same per-step event timing without the flush, for a like-for-like median
        sev = [new_events(2) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            sev[i][0].record(stream)
            step()
            sev[i][1].record(stream)
        torch.cuda.synchronize()
        flush_res["steady_state_median_ms"] = float(np.median([e[0].elapsed_time(e[1]) for e in sev]))

    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    res = {
        "metric": METRIC,
        "value": wl.T / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": warm,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded numpy PCG64 draws of the workload's shapes and distributions)",
        "config": {"workload": wl.name, "T": wl.T, "d_model": dm, "d_ff": ff,
                   "n_experts": wl.n_experts, "top_k": wl.top_k,
                   "capacity_factor": wl.capacity_factor, "capacity": None if dropless else cap,
                   "layout": args.layout, "weights": args.weights},
        "expert_gemm_tflops": (gemm1_flop + gemm2_flop) / expert_s / 1e12,
        "expert_gemm_frac_of_bf16_peak": (gemm1_flop + gemm2_flop) / expert_s / 1e12
                                         / PEAK_BF16_TFLOPS,
        "roofline": dict(roof, traffic=traffic, traffic_source=traffic_src),
        "flush": flush_res,
        "x_routed": x_routed_res,
        "dominant_kernel_ms": dom_ms,
        "dominant_kernel_timing": "start and end of the dominant GEMM's kernel, recorded by its "
                                  "launch in each timed step (moe_set_gemm_timing, "
                                  "hipExtLaunchKernel), averaged over the K steps; the roofline "
                                  "uses it, expert_gemm_* use the stage times below",
        "stages_ms": stage_ms,
        "stage_timing": "HIP events at the stage boundaries over a second run of the same number "
                        "of steps right after the timed region (events between launches add "
                        "short gaps, so these steps are not the timed ones)",
        "event_step_ms": step_ms,
        "route_GBps": route_bytes / (stage_ms["route"] / 1e3) / 1e9,
        "combine_GBps": combine_bytes / (stage_ms["combine"] / 1e3) / 1e9,
        # the same bytes over the kernels' own durations (recorded by their launches in a third
        # run of plain steps)
        "route_kernel_ms": route_kernel_ms,
        "route_kernel_GBps": (route_bytes / (route_kernel_ms / 1e3) / 1e9
                              if route_kernel_ms else None),
        "combine_kernel_ms": combine_kernel_ms,
        "combine_kernel_GBps": (combine_bytes / (combine_kernel_ms / 1e3) / 1e9
                                if combine_kernel_ms else None),
        "n_kept": n_kept,
        "expert_rows_computed": wl.n_experts * cap if padded else n_kept,
        "combine_stage": "moe_sum over pair rows" if dropless else "combine (slot gather)",
        # FLOP rate of what the matrix cores executed (buffer rows included), padded layout
        "expert_gemm_tflops_executed": (3 if gated else 2) * 2.0
                                       * (wl.n_experts * cap if padded else n_kept) * dm * ff
                                       / expert_s / 1e12,
        "drop_rate": 1.0 - n_kept / (wl.T * wl.top_k),
        "expert_rows": [int(v) for v in (c if dropless else np.minimum(c, cap))],
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(inp, wl, cap, dropless)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
