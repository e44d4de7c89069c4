"""Benchmark: routed tokens/s of one rank's MoE expert-layer forward on one MI355X.

A step is the whole path on one batch already resident in HBM: route top-k ->
dispatch -> grouped GEMM (gate/up + SwiGLU, then down) -> combine, through the
C ABI, with every buffer allocated before timing. Prints ONE JSON line.

Timing: W warm-up steps, then K timed steps, each bracketed by events on the
stream the kernels run on. Before each step, outside its events, 512 MiB are
written to one scratch buffer and then 512 MiB of another are read, so the 4 MB
L2s and the 256 MB Infinity Cache hold none of the step's inputs when it starts
(the read pass also writes back the dirty lines the write left, which would
otherwise be written back during the step). The K steps are
bracketed by a device synchronisation on both sides; `value` and `ms_per_step`
use the median of the per-step event times. The same K steps back to back, with
no flush, give `back_to_back_ms_per_step` (wall clock) for comparison.

The roofline object covers the grouped GEMM call (its two MFMA launches, and
the blocked copy of the gathered rows that precedes them where the call makes
one), timed with events around it inside every timed step (median). The CPU baseline is
the fp64 oracle on a bounded sample of the same workload, timed on the host
cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import moe_inputs as mi  # noqa: E402

METRIC = "routed tokens/sec per MoE layer fwd on 1 MI355X; grouped-GEMM % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0
# Sources that decide the grouped GEMM's machine code; a stored traffic figure is
# reported only while they are unchanged since its counters were taken.
GEMM_SOURCES = ["gemm_common.h", "lds_pipe.h", "moe_internal.h", "grouped_gemm.hip", "grouped_gemm_lds.hip"]


def host_cores() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit():
        n = min(n, int(omp))
    return n


def gemm_sources_sha256() -> str:
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "token_dispatch_grouped_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(workload: str):
    """HBM bytes per step of the grouped GEMM from the FETCH_SIZE / WRITE_SIZE
    summary under profiles/, or None if there is none for this workload or the
    kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if " = " in line:
                key, val = line.strip().split(" = ", 1)
                kv[key] = val
    if kv.get("workload") != workload or kv.get("gemm_sources_sha256") != gemm_sources_sha256():
        return None
    return int(kv["traffic_bytes_per_step"])


def sample_sclk(step, seconds: float, torch):
    """Median shader clock (MHz) reported by rocm-smi while `step` runs back to back."""
    import re
    import subprocess
    import threading

    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                out = subprocess.run(["rocm-smi", "--showclocks", "--csv"], capture_output=True,
                                     text=True, timeout=10).stdout
            except (OSError, subprocess.SubprocessError):
                return
            lines = [l for l in out.splitlines() if l.startswith("card0")]
            if lines:
                mhz = re.findall(r"\((\d+)Mhz\)", lines[0])
                if len(mhz) >= 2:
                    samples.append(int(mhz[1]))  # fields: mclk, then sclk
            stop.wait(0.3)

    th = threading.Thread(target=sampler)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    samples = samples[2:] or samples  # the first samples may precede the clock settling
    return float(np.median(samples)) if samples else None


def sha256_of(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).view(np.uint8)).hexdigest()


def versions(torch) -> dict:
    v = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
    try:
        with open("/opt/rocm/.info/version") as fh:
            v["rocm"] = fh.read().strip()
    except OSError:
        v["rocm"] = None
    try:
        v["device"] = torch.cuda.get_device_properties(0).gcnArchName
    except (AttributeError, RuntimeError):
        v["device"] = None
    return v


def cpu_baseline(w: mi.Workload, logits, x, wgu, wdn, budget_s: float = 12.0) -> dict:
    """The oracle, as it stands, on the first T_s tokens of the same workload."""
    import oracle

    x64 = mi.to_f64(x, w.dtype)
    gu64 = [mi.to_f64(wgu[e], w.dtype) for e in range(w.E_loc)]
    dn64 = [mi.to_f64(wdn[e], w.dtype) for e in range(w.E_loc)]
    ts = min(w.T, 64)
    while True:
        t0 = time.perf_counter()
        oracle.moe_layer(x64[:ts], logits[:ts], w.k, w.e_begin, w.e_end, gu64, dn64)
        dt = time.perf_counter() - t0
        if dt * 2 > budget_s or ts >= w.T:
            break
        ts = min(w.T, ts * 2)
    return {"value": ts / dt, "unit": "tokens/s", "cores": host_cores(), "kind": "oracle",
            "sample": f"oracle.moe_layer (fp64, numpy BLAS) on the first {ts} of {w.T} tokens of "
                      f"workload {w.name}, {dt:.2f} s; fp64 weight conversion untimed"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense8", choices=sorted(mi.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=["fused", "staged"], default="fused",
                    help="fused: dispatch indices only, the gate/up GEMM gathers rows from x; "
                         "staged: dispatch gathers rows into x_perm first")
    ap.add_argument("--train", action="store_true",
                    help="a step is the forward and then the backward of the layer (seeded d_out); the "
                         "roofline object then covers moe_grouped_gemm_backward")
    ap.add_argument("--graph", action="store_true",
                    help="record one step in a HIP graph and time graph replays (the GEMM roofline "
                         "then comes from an eager pass after the timed replays)")
    ap.add_argument("--clock-seconds", type=float, default=0.0,
                    help="after timing, repeat the step for this many seconds while sampling the "
                         "shader clock with rocm-smi; reports the median as sclk_mhz")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="MiB written to one scratch buffer, then read from another, before each timed "
                         "step and outside its events (0: no flush)")
    ap.add_argument("--flush-mode", choices=["write-read", "write", "read"], default="write-read",
                    help="which flush passes run before each timed step")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (3 times), the "
                         "reference for scaling FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {args.gpus} is not supported "
              "(the multi-GPU exchange is not part of this library)", file=sys.stderr)
        return 2

    import torch

    import token_dispatch_grouped_amd as moe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}), flush=True)
        return 0
    w = mi.WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    logits = mi.router_logits(w)
    x = mi.hidden_states(w)
    wgu, wdn = mi.expert_weights(w)
    print(f"[bench] inputs for {w.name} drawn in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    def to_dev(a, dtype):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    dx, dl = to_dev(x, w.dtype), to_dev(logits, "f32")
    dgu, ddn = to_dev(wgu, w.dtype), to_dev(wdn, w.dtype)
    # every buffer the step writes, allocated once
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    # the row gather inside the GEMM exists for bf16 only; the fp32 workload runs staged
    fused = args.path == "fused" and w.dtype == "bf16"
    disp = moe.dispatch_alloc(dx, w.k, w.E, w.e_begin, w.e_end, gather=not fused)
    h = torch.empty((w.n_max, w.d_ff), dtype=dx.dtype, device=dev)
    y = torch.empty((w.n_max, w.d), dtype=dx.dtype, device=dev)
    out = torch.empty((w.T, w.d), dtype=dx.dtype, device=dev)
    # the stream every call goes to: torch's current stream at call time (the
    # capture stream while a graph is being recorded)
    cur = torch.cuda.current_stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    ev_step = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    flush_buf = (torch.empty(args.flush_mib << 18, dtype=torch.float32, device=dev)
                 if args.flush_mib > 0 else None)
    flush_src = (torch.ones(args.flush_mib << 18, dtype=torch.float32, device=dev)
                 if args.flush_mib > 0 else None)
    flush_sink = torch.zeros((), dtype=torch.float32, device=dev)

    def flush(i):
        if flush_buf is None:
            return
        if args.flush_mode != "read":
            flush_buf.fill_(float(i + 1))
        if args.flush_mode != "write":
            torch.sum(flush_src, dim=0, out=flush_sink)

    gu = None  # training: the gate/up pre-activations the forward keeps for the backward

    def gemm():
        if fused:
            moe.grouped_gemm_gather(dx, disp.perm, disp.offsets, dgu, ddn, w.k, w.E, w.e_begin, w.e_end,
                                    h=h, y=y, stream=cur(), gu=gu)
        else:
            moe.grouped_gemm(disp.x_perm, disp.offsets, dgu, ddn, w.T, w.k, w.E, w.e_begin, w.e_end,
                             h=h, y=y, stream=cur())

    train = args.train
    if train:
        if w.dtype != "bf16" or not fused:
            print("--train runs the fused bf16 path", file=sys.stderr)
            return 2
        rng = np.random.default_rng(w.seed + 500)
        d_out = to_dev(mi.f32_to_bf16_bits(rng.standard_normal((w.T, w.d)).astype(np.float32)), "bf16")
        d_y = torch.empty((w.n_max, w.d), dtype=dx.dtype, device=dev)
        d_w = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
        d_xp = torch.empty((w.n_max, w.d), dtype=dx.dtype, device=dev)
        d_wgu, d_wdn = torch.empty_like(dgu), torch.empty_like(ddn)
        d_x = torch.empty((w.T, w.d), dtype=dx.dtype, device=dev)
        d_logits = torch.empty((w.T, w.E), dtype=torch.float32, device=dev)
        ws_bytes = moe.grouped_gemm_backward_workspace_bytes(w.T, w.d, w.d_ff, w.E, w.k, w.e_begin, w.e_end)
        bws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        gu = torch.empty((w.n_max, 2 * w.d_ff), dtype=dx.dtype, device=dev)

    def bwd_gemm():
        moe.grouped_gemm_backward(dx, disp.perm, disp.offsets, dgu, ddn, h, d_y, w.k, w.E, w.e_begin, w.e_end,
                                  d_x_perm=d_xp, d_w_gate_up=d_wgu, d_w_down=d_wdn, workspace=bws, stream=cur(),
                                  gu=gu)

    # the calls of one step, in order: (name, call)
    calls = [
        ("route_topk", lambda: moe.route_topk(dl, w.k, idx, wts, stream=cur())),
        ("dispatch", lambda: moe.dispatch(dx, idx, w.E, w.e_begin, w.e_end, out=disp, stream=cur(),
                                          gather=not fused)),
        ("grouped_gemm", gemm),
        ("combine", lambda: moe.combine(y, disp.pair_pos, wts, w.T, w.k, w.E, w.e_begin, w.e_end, out=out,
                                        stream=cur())),
    ]
    if train:
        calls += [
            ("combine_backward", lambda: moe.combine_backward(d_out, y, disp.pair_pos, wts, w.T, w.k, w.E, w.e_begin,
                                                              w.e_end, d_y=d_y, d_topk_w=d_w, stream=cur())),
            ("grouped_gemm_backward", bwd_gemm),
            ("dispatch_backward", lambda: moe.dispatch_backward(d_xp, disp.pair_pos, w.T, w.k, w.E, w.e_begin,
                                                                w.e_end, d_x=d_x, stream=cur())),
            ("route_topk_backward", lambda: moe.route_topk_backward(idx, wts, d_w, w.E, d_logits=d_logits,
                                                                    stream=cur())),
        ]
    timed = "grouped_gemm_backward" if train else "grouped_gemm"  # the roofline's kernel

    def step(i=None):
        for name, call in calls:
            if i is not None and name == timed:
                ev[i][0].record(cur())
            call()
            if i is not None and name == timed:
                ev[i][1].record(cur())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    offs = disp.offsets.cpu().numpy()
    n_loc = int(offs[w.e_end] - offs[w.e_begin])
    active = int(np.count_nonzero(disp.counts.cpu().numpy()[w.e_begin:w.e_end]))

    graph = None
    if args.graph:
        # one step recorded into a HIP graph (warmed up on a side stream first)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()

    # K timed steps, each after a flush and between its own events (median)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush(i)
        ev_step[i][0].record(cur())
        if graph is not None:
            graph.replay()
        else:
            step(i)
        ev_step[i][1].record(cur())
    torch.cuda.synchronize()
    wall_flushed_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    step_ms = [a.elapsed_time(b) for a, b in ev_step]
    ms_step = float(np.median(step_ms))
    if graph is not None:  # the GEMM's events come from an eager pass after the timed replays
        for i in range(args.steps):
            flush(i)
            step(i)
        torch.cuda.synchronize()
    gemm_all = [a.elapsed_time(b) for a, b in ev]
    gemm_ms = float(np.median(gemm_all))
    # the same K steps back to back, no flush: wall clock per step
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    host_ms = (time.perf_counter() - t0) * 1e3 / args.steps  # enqueueing only
    torch.cuda.synchronize()
    b2b_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # forward: gate/up (4 N d d_ff) + down (2 N d d_ff); backward (the forward kept the gate/up
    # pre-activations): dH (2), dX (4), dW_dn (2), dW_gu (4)
    flops = (12.0 if train else 6.0) * n_loc * w.d * w.d_ff
    b = 2 if w.dtype == "bf16" else 4
    # forward: weights of every active local expert once, one activation row per local pair and
    # H read once, H and Y written once. backward: W_gu and W_dn read once, both weight gradients
    # written once (6 d d_ff per active expert); per local row, the d-wide blocks moved 6 times
    # (x read, x_perm written and read, dY read twice, dX written) and the d_ff-wide ones 9 times
    # (the kept gate/up read, their gradient written and read twice, H read)
    if train:
        gemm_bytes = 6.0 * active * w.d * w.d_ff * b + n_loc * (6.0 * w.d + 9.0 * w.d_ff) * b
    else:
        gemm_bytes = 3.0 * active * w.d * w.d_ff * b + 2.0 * n_loc * (w.d + w.d_ff) * b
    peak_flops = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    t_gemm = gemm_ms * 1e-3
    # the bound is whichever of MFMA time and HBM time is longer at peak
    if w.dtype == "bf16" and gemm_bytes / (PEAK_HBM_GBS * 1e9) > flops / (peak_flops * 1e12):
        bound, achieved, peak, unit = "hbm", gemm_bytes / t_gemm / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        bound = "mfma" if w.dtype == "bf16" else "alu"
        achieved, peak, unit = flops / t_gemm / 1e12, peak_flops, "TFLOP/s"
    roofline = {
        "kernel": ("moe_grouped_gemm_backward_saved (row gather, blocked copy of dY, dH+SwiGLU "
                   "backward, dX, dW_down, dW_gate_up launches; gate/up pre-activations kept by "
                   "the forward)" if train else
                   ("moe_grouped_gemm_gather" if fused else "moe_grouped_gemm")
                   + " (blocked copy of the gathered rows where the call makes one, gate/up+SwiGLU "
                   "launch, then down launch)"),
        "bound": bound,
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": unit,
        "frac": round(achieved / peak, 4),
        "traffic": None if train else stored_traffic(w.name),
        "flops_per_launch": flops,
        "algorithmic_bytes_per_launch": gemm_bytes,
        "median_ms": round(gemm_ms, 4),
        "mean_ms": round(float(np.mean(gemm_all)), 4),
        "timings": len(gemm_all),
    }
    result = {
        "metric": METRIC,
        "value": round(w.T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal draws; see moe_inputs)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "d_ff": w.d_ff, "E": w.E, "k": w.k,
                   "local_experts": [w.e_begin, w.e_end], "N_loc": n_loc, "active_local_experts": active,
                   "parallelism": "one rank's share on 1 GPU", "path": "fused" if fused else "staged",
                   "launch": "hip graph" if args.graph else "eager",
                   "step": "forward + backward" if args.train else "forward"},
        "local_pairs_per_s": round(n_loc / (ms_step * 1e-3), 1),
        "timing": {"per_step": f"median of {args.steps} per-step event times, each step after a "
                               f"{args.flush_mib} MiB flush ({args.flush_mode}) outside its events",
                   "step_ms_min": round(float(np.min(step_ms)), 4),
                   "step_ms_max": round(float(np.max(step_ms)), 4),
                   "wall_ms_per_step_incl_flush": round(wall_flushed_ms, 4),
                   "back_to_back_ms_per_step": round(b2b_ms, 4),
                   "back_to_back_host_enqueue_ms_per_step": round(host_ms, 4)},
        "roofline": roofline,
        "cpu_baseline": None,
        "seed": w.seed,
        "inputs_sha256": {"logits": sha256_of(logits), "x": sha256_of(x), "w_gate_up": sha256_of(wgu),
                          "w_down": sha256_of(wdn)},
        "versions": versions(torch),
    }
    # per entry point, in a separate untimed pass: events between the calls
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        e = evs[i]
        e[0].record(cur())
        for j, (_, call) in enumerate(calls):
            call()
            e[j + 1].record(cur())
    torch.cuda.synchronize()
    result["entry_point_ms"] = {name: round(float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])), 4)
                                for j, (name, _) in enumerate(calls)}
    if args.clock_seconds > 0:
        result["sclk_mhz"] = sample_sclk(step, args.clock_seconds, torch)
    del dgu, ddn
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, logits, x, wgu, wdn)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
