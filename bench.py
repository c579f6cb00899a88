#!/usr/bin/env python3
"""Throughput of the KDA chunkwise backward (kda_chunk_bwd) on one MI355X.

One step = one kda_chunk_bwd call over the whole workload (backward preparation, reverse
state-gradient scan, chunk gradients). Its inputs -- q, k, v, g, beta, dO, dS_final and the
per-chunk states and WY/UT inverses written beforehand by kda_fwd_states -- are resident in
HBM before timing starts. Before every timed step a 1 GiB buffer is written so that neither
L2 nor the 256 MB Infinity Cache holds the inputs (cold-cache timing); the flush itself is
outside the timed interval, which HIP events bracket on the call's stream. Warm-cache
(back-to-back) timing is reported alongside.

Prints one JSON line. `value` is token-heads per second (tokens x value heads / time).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_BYTES = 8.0e12      # MI355X HBM3E, bytes/s
PEAK_BF16_FLOPS = 2.5e15     # MI355X dense bf16 MFMA, flop/s
PEAK_F32_FLOPS = 157.3e12    # MI355X dense fp32 MFMA


def recorded_traffic(workload_name):
    """HBM bytes per bwd_grad launch measured with rocprofv3 counters (FETCH_SIZE, WRITE_SIZE,
    scaled by a plain copy's readings) as recorded in profiles/bwd_grad_w1_counters.md, or None
    when that record is for another workload or the kernel's sources have changed since."""
    import hashlib
    rec = os.path.join(HERE, "profiles", "bwd_grad_w1_counters.md")
    if not os.path.exists(rec):
        return None
    h = hashlib.sha256()
    for f in ("kda_bwd.hip", "kda_device.h"):
        with open(os.path.join(HERE, "chunked_gated_delta_09_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    with open(rec) as fh:
        for line in fh:
            if line.startswith("bench-traffic:"):
                kv = dict(t.split("=", 1) for t in line.split()[1:])
                if kv.get("workload") == workload_name and kv.get("sources-sha256") == h.hexdigest():
                    return int(kv["bytes"])
    return None


def algorithmic_bytes(w, inp):
    """Bytes the backward must move at least once: reads of q, k, v, dO, g, beta, the chunk
    states and inverses, dS_final; writes of dq, dk, dv, dg, dbeta, dh0."""
    es = 4 if w.dtype == "f32" else 2
    T, N = inp["B"] * inp["T"], inp["N"]
    nt = sum(math.ceil((b - a) / w.C) for a, b in zip(flat_cu(inp)[:-1], flat_cu(inp)[1:]))
    reads = (2 * T * w.H * w.K * es + 2 * T * w.HV * w.V * es + T * w.HV * w.K * 4 + T * w.HV * 4
             + nt * w.HV * (w.K * w.V + w.C * w.C) * es)
    writes = 2 * T * w.H * w.K * es + T * w.HV * w.V * es + T * w.HV * w.K * 4 + T * w.HV * 4
    if inp["dS_final"] is not None:
        reads += N * w.HV * w.K * w.V * es
    writes += N * w.HV * w.K * w.V * 4
    return reads + writes


def algorithmic_flops(w, inp):
    """14 K V + 10 C K flop per token-head: seven C x K x V products and ten triangular
    C x C x D products per chunk (C^2 D / 2 multiply-adds each), at 2 flop per multiply-add."""
    return (14 * w.K * w.V + 10 * w.C * w.K) * inp["B"] * inp["T"] * w.HV


def flat_cu(inp):
    from chunked_gated_delta_09_amd import inputs as kin
    return kin.flat_cu(inp)


def cpu_baseline(inp):
    """The fp64 oracle (forward + hand-derived backward) on the host cores, timed on the
    whole workload: every (sequence, value head) task."""
    import oracle
    from tests.kda_cases import run_oracle
    oracle.build(force=False)
    # repeated until about a second of wall time (10-20 s of CPU work on the machine's cores)
    runs, t0 = 0, time.perf_counter()
    while True:
        r = run_oracle(oracle, inp)
        runs += 1
        dt = time.perf_counter() - t0
        if dt > 1.0 and runs >= 2:
            break
    th = inp["B"] * inp["T"] * inp["workload"].HV
    return {"value": runs * th / dt, "unit": "token-heads/s", "cores": int(r["threads"]), "kind": "oracle",
            "sample": f"whole workload ({th} token-heads, {inp['N']} sequences x {inp['workload'].HV} heads), "
                      f"fp64 forward+backward, {runs} runs in {dt:.2f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=1, help="workload id (1 = B=2,T=2048,H=8,K=V=128,C=64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB a few times (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters of a profiler run) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the KDA chunk backward here runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        src = torch.empty(args.copy_calibration << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": args.copy_calibration << 20, "copies": 3}), flush=True)
        return
    import chunked_gated_delta_09_amd as kda
    from chunked_gated_delta_09_amd import inputs as kin

    w = kin.WORKLOADS[args.workload]
    inp = kin.make_inputs(w, wid=args.workload)
    dev = torch.device("cuda:0")
    d = {k: (inp[k].contiguous().to(dev) if inp[k] is not None else None)
         for k in ("q", "k", "v", "g", "beta", "h0", "dS_final", "dO")}
    fw = kda.fwd_states(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], cu_seqlens=inp["cu_seqlens"],
                        C=w.C, scale=inp["scale"])
    cu_dev = (torch.tensor(inp["cu_seqlens"], dtype=torch.int32, device=dev)
              if inp["cu_seqlens"] is not None else None)
    B, T = inp["B"], inp["T"]
    dims, keep = kda.make_dims(B, T, w.H, w.HV, w.K, w.V, w.C, inp["scale"], w.dtype, inp["cu_seqlens"], cu_dev)
    tdt = w.torch_dtype
    dq = torch.empty(B, T, w.H, w.K, dtype=tdt, device=dev)
    dk = torch.empty_like(dq)
    dv = torch.empty(B, T, w.HV, w.V, dtype=tdt, device=dev)
    dg = torch.empty(B, T, w.HV, w.K, dtype=torch.float32, device=dev)
    dbeta = torch.empty(B, T, w.HV, dtype=torch.float32, device=dev)
    dh0 = torch.empty(inp["N"], w.HV, w.K, w.V, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.bwd_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    lib = kda.load()
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch has loaded
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    nk = 4 if inp["cu_seqlens"] is not None else 3  # kernels per call
    kernel_names = (["chunk_table"] if nk == 4 else []) + ["bwd_prep", "bwd_scan", "bwd_grad"]

    def new_events(n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = ev.value
        return arr

    def elapsed(e0, e1):
        ms = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def step():
        kda.chunk_bwd_into(dims, d["q"], d["k"], d["v"], d["g"], d["beta"], fw["states"], fw["inv"], d["dO"],
                           d["dS_final"], dq, dk, dv, dg, dbeta, dh0, ws, stream=stream)

    def timed(nsteps, flush, per_kernel):
        """nsteps calls; HIP events around each call on its stream, and (per_kernel) the
        library's events around each of its kernels. The timed region is bracketed by
        device synchronisation."""
        call_ev = new_events(2 * nsteps)
        kern_ev = new_events(2 * nk * nsteps) if per_kernel else None
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(nsteps):
            if flush:
                flush_buf.fill_(i & 0xFF)
            if per_kernel:
                lib.kda_set_kernel_events(
                    ctypes.cast(ctypes.byref(kern_ev, 2 * nk * i * ctypes.sizeof(ctypes.c_void_p)),
                                ctypes.POINTER(ctypes.c_void_p)), 2 * nk)
            hip.hipEventRecord(call_ev[2 * i], stream)
            step()
            hip.hipEventRecord(call_ev[2 * i + 1], stream)
        lib.kda_set_kernel_events(None, 0)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        calls = [elapsed(call_ev[2 * i], call_ev[2 * i + 1]) for i in range(nsteps)]
        kern = {}
        if per_kernel:
            kern = {name: [elapsed(kern_ev[2 * nk * i + 2 * j], kern_ev[2 * nk * i + 2 * j + 1])
                           for i in range(nsteps)] for j, name in enumerate(kernel_names)}
        for arr in (call_ev, kern_ev or []):
            for e in arr:
                hip.hipEventDestroy(e)
        return calls, kern, wall

    for _ in range(args.warmup):
        step()
    cold_calls, _, cold_wall = timed(args.steps, flush=True, per_kernel=False)
    warm_calls, _, _ = timed(args.steps, flush=False, per_kernel=False)
    _, cold_kern, _ = timed(args.steps, flush=True, per_kernel=True)
    _, warm_kern, _ = timed(args.steps, flush=False, per_kernel=True)

    # The training forward (kda_fwd_states with the output o), timed the same way (cold):
    # reported beside the backward, not part of the step.
    def fwd_step():
        return kda.fwd_states(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], cu_seqlens=inp["cu_seqlens"],
                              C=w.C, scale=inp["scale"], output_o=True)

    for _ in range(2):
        fwd_step()
    fwd_ev = new_events(2 * args.steps)
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush_buf.fill_(i & 0xFF)
        hip.hipEventRecord(fwd_ev[2 * i], stream)
        fwd_step()
        hip.hipEventRecord(fwd_ev[2 * i + 1], stream)
    torch.cuda.synchronize()
    fwd_ms = statistics.mean(elapsed(fwd_ev[2 * i], fwd_ev[2 * i + 1]) for i in range(args.steps))
    for e in fwd_ev:
        hip.hipEventDestroy(e)

    th = B * T * w.HV
    ms = statistics.mean(cold_calls)
    value = th / (ms * 1e-3)
    abytes = algorithmic_bytes(w, inp)
    aflops = algorithmic_flops(w, inp)
    grad_ms = statistics.mean(cold_kern["bwd_grad"])
    achieved = abytes / (grad_ms * 1e-3) / 1e9
    peak_flops = PEAK_F32_FLOPS if w.dtype == "f32" else PEAK_BF16_FLOPS
    t_roof = max(abytes / PEAK_HBM_BYTES, aflops / peak_flops)
    out = {
        "metric": "KDA chunk-bwd token-heads/s at K=V=128, C=64 (HBM roofline fraction)",
        "value": value,
        "unit": "token-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v,dO N(0,1), g=logsigmoid(N(3,1)), "
                "beta=sigmoid(N(0,1)), h0,dS_final N(0,0.1))",
        "config": {"workload": w.name, "B": B, "T": T, "H": w.H, "HV": w.HV, "K": w.K, "V": w.V, "C": w.C,
                   "token_heads": th, "cache": "cold (1 GiB flush before each step, outside the timed interval)"},
        "roofline": {"bound": "hbm", "kernel": "bwd_grad", "achieved": achieved, "peak": PEAK_HBM_BYTES / 1e9,
                     "unit": "GB/s", "frac": achieved / (PEAK_HBM_BYTES / 1e9), "traffic": recorded_traffic(w.name),
                     "algorithmic_bytes_per_launch": abytes,
                     "launch_ms": grad_ms},
        "call_roofline": {"t_roofline_ms": t_roof * 1e3, "frac": t_roof / (ms * 1e-3),
                          "algorithmic_bytes": abytes, "algorithmic_flops": aflops},
        "kernels_ms_cold": {k: statistics.mean(v) for k, v in cold_kern.items()},
        "kernels_ms_warm": {k: statistics.mean(v) for k, v in warm_kern.items()},
        "ms_per_step_p10_p50_p90_cold": [sorted(cold_calls)[int(0.1 * (len(cold_calls) - 1))],
                                         statistics.median(cold_calls),
                                         sorted(cold_calls)[int(0.9 * (len(cold_calls) - 1))]],
        "ms_per_step_warm": statistics.mean(warm_calls),
        "forward": {"entry": "kda_fwd_states with o (chunk prep, forward state scan, output)",
                    "ms_cold": fwd_ms, "token_heads_per_s": th / (fwd_ms * 1e-3)},
        "wall_s_timed_cold_incl_flush": cold_wall,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)
    del keep


if __name__ == "__main__":
    main()
