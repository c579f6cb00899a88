#!/usr/bin/env python3
"""Throughput of the KDA chunkwise backward (kda_chunk_bwd) on one MI355X.

One step = one kda_chunk_bwd call over the whole workload (backward preparation, reverse
state-gradient scan, chunk gradients). Its inputs -- q, k, v, g, beta, dO, dS_final and the
per-chunk states and WY/UT inverses written beforehand by kda_fwd_states -- are resident in
HBM before timing starts. Before every timed step a 1 GiB buffer is written so that neither
L2 nor the 256 MB Infinity Cache holds the inputs (cold-cache timing); the flush itself is
outside the timed interval, which HIP events bracket on the call's stream. That flush leaves
the caches full of dirty lines, which the call's reads then have to write back; `cold_clean`
repeats the timing with a second 1 GiB buffer read after the write, so that the caches hold
clean lines of neither input (the headline keeps the dirty-cache figure). Warm-cache
(back-to-back) timing is reported alongside.

Prints one JSON line. `value` is token-heads per second (tokens x value heads / median cold
call time) on the B=2, T=2048, H=8, K=V=128, C=64 workload; the other three K=V=128
workloads are measured the same way (fewer steps) under `per_workload`.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
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
CPU_SHARE = 16               # host threads of one GPU's share of the box

# Kernels of one kda_chunk_bwd call, in launch order (the chunk table only for packed sequences).
BWD_KERNELS = ["bwd_prep", "bwd_scan", "bwd_grad"]
FWD_KERNELS = ["fwd_prep", "fwd_scan", "fwd_out"]  # kda_fwd_states with o, after the chunk table
# Sources whose text fixes the backward kernels and their workspace layout.
BWD_SOURCES = ["kda_api.cpp", "kda_bwd.hip", "kda_scan.hip", "kda_device.h", "kda_launch.h"]
TRAFFIC_RECORD = os.path.join(HERE, "profiles", "kda_chunk_bwd_w1_hbm_counters.md")


def sources_sha256():
    h = hashlib.sha256()
    for f in BWD_SOURCES:
        with open(os.path.join(HERE, "chunked_gated_delta_09_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload_name, kernel="call", record=TRAFFIC_RECORD):
    """HBM bytes per launch of `kernel` (or per call, the sum over the call's kernels)
    measured with rocprofv3 counters (FETCH_SIZE, WRITE_SIZE, scaled by a plain copy's
    readings) as recorded in the counters profile, or None when the record is for another
    workload or the backward's sources have changed since it was taken."""
    if not os.path.exists(record):
        return None
    sha = sources_sha256()
    per = {}
    with open(record) as fh:
        for line in fh:
            if line.startswith("bench-traffic:"):
                kv = dict(t.split("=", 1) for t in line.split()[1:])
                if kv.get("workload") == workload_name and kv.get("sources-sha256") == sha:
                    per[kv["kernel"]] = int(kv["bytes"])
    if kernel == "call":
        return sum(per[k] for k in BWD_KERNELS) if all(k in per for k in BWD_KERNELS) else None
    return per.get(kernel)


def algorithmic_bytes(w, inp):
    """Bytes the backward must move at least once: reads of q, k, v, dO, g, beta, the chunk
    states and inverses, dS_final; writes of dq, dk, dv, dg, dbeta, dh0."""
    es = 4 if w.dtype == "f32" else 2
    T, N = inp["B"] * inp["T"], inp["N"]
    nt = num_chunks(w, inp)
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


def fwd_algorithmic_bytes(w, inp):
    """Bytes kda_fwd_states with the output o must move at least once: reads of q, k, v, g,
    beta, h0; writes of the chunk states and inverses, o and the final state."""
    es = 4 if w.dtype == "f32" else 2
    T, N = inp["B"] * inp["T"], inp["N"]
    nt = num_chunks(w, inp)
    reads = 2 * T * w.H * w.K * es + T * w.HV * w.V * es + T * w.HV * w.K * 4 + T * w.HV * 4
    if inp["h0"] is not None:
        reads += N * w.HV * w.K * w.V * es
    writes = nt * w.HV * (w.K * w.V + w.C * w.C) * es + T * w.HV * w.V * es + N * w.HV * w.K * w.V * 4
    return reads + writes


def num_chunks(w, inp):
    cu = flat_cu(inp)
    return sum(math.ceil((b - a) / w.C) for a, b in zip(cu[:-1], cu[1:]))


def flat_cu(inp):
    from chunked_gated_delta_09_amd import inputs as kin
    return kin.flat_cu(inp)


def cpu_baseline(inp):
    """The fp64 oracle (forward + hand-derived backward) on the host cores, timed on the
    whole workload: every (sequence, value head) task, on at most one GPU's share of the
    host's threads."""
    import oracle
    from tests.kda_cases import run_oracle
    oracle.build(force=False)
    nthreads = max(1, min(CPU_SHARE, os.cpu_count() or 1))
    # repeated until about a second of wall time (10-20 s of CPU work on the threads used)
    runs, t0 = 0, time.perf_counter()
    while True:
        r = run_oracle(oracle, inp, nthreads=nthreads)
        runs += 1
        dt = time.perf_counter() - t0
        if dt > 1.0 and runs >= 2:
            break
    th = inp["B"] * inp["T"] * inp["workload"].HV
    return {"value": runs * th / dt, "unit": "token-heads/s", "cores": int(r["threads"]), "kind": "oracle",
            "threads": int(r["threads"]), "host_nproc": os.cpu_count(),
            "sample": f"whole workload ({th} token-heads, {inp['N']} sequences x {inp['workload'].HV} heads), "
                      f"fp64 forward+backward, {runs} runs in {dt:.2f} s"}


def _pct(xs, p):
    s = sorted(xs)
    return s[int(round(p * (len(s) - 1)))]


class Hip:
    """The HIP runtime torch has loaded, for events on the call's stream."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = ev.value
        return arr

    def record(self, ev, stream):
        self.lib.hipEventRecord(ev, stream)

    def elapsed(self, e0, e1):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), e0, e1) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, arr):
        for e in arr:
            self.lib.hipEventDestroy(e)


def scan_forms_w(w, inp):
    """Whether the reverse scan forms W itself (4 or more value slices per workgroup, the
    library's scan_wq rule), so that the saved-operand backward launches no W kernel."""
    slices = inp["N"] * w.HV * (w.V // 16)
    nc = 1
    while nc < w.V // 16 and slices // nc > 256:
        nc *= 2
    return w.dtype != "f32" and nc >= 4


def saved_read_bytes(w, inp):
    """Bytes of the forward's save that the saved-operand backward reads: kr, -w^T, Q'^T
    (C x K each) and e^gam (K, fp32) per chunk-head."""
    es = 4 if w.dtype == "f32" else 2
    return num_chunks(w, inp) * w.HV * (3 * w.C * w.K * es + w.K * 4)


def measure(wid, steps, warmup, hip, flush_buf, warm=True, forward=True, saved=True, recompute=True,
            clean_buf=None):
    """Times kda_chunk_bwd on workload `wid`: cold and (optionally) warm call times, and the
    per-kernel times from the library's event hook; with `clean_buf`, cold times again after a
    flush that leaves clean lines (the write, then a read of clean_buf); optionally the forward
    with o, and the saved-operand pair (kda_fwd_states_save + kda_chunk_bwd_saved)."""
    import torch
    import chunked_gated_delta_09_amd as kda
    from chunked_gated_delta_09_amd import inputs as kin
    from chunked_gated_delta_09_amd import measure as kmeas

    w = kin.WORKLOADS[wid]
    inp = kin.make_inputs(w, wid=wid)
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
    stream = torch.cuda.current_stream().cuda_stream
    table = ["chunk_table"] if inp["cu_seqlens"] is not None else []
    names = table + BWD_KERNELS

    def step():
        kda.chunk_bwd_into(dims, d["q"], d["k"], d["v"], d["g"], d["beta"], fw["states"], fw["inv"], d["dO"],
                           d["dS_final"], dq, dk, dv, dg, dbeta, dh0, ws, stream=stream)

    def timed(nsteps, flush, per_kernel, step=step, names=names):
        """nsteps calls; HIP events around each call on its stream, and (per_kernel) the
        library's events around each of its kernels. The timed region is bracketed by
        device synchronisation."""
        nk = len(names)
        call_ev = hip.events(2 * nsteps)
        kern_ev = hip.events(2 * nk * nsteps) if per_kernel else None
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(nsteps):
            if flush:
                flush_buf.fill_(i & 0xFF)
            if flush == "clean":
                clean_buf.max()
            if per_kernel:
                kmeas.set_kernel_events(
                    ctypes.cast(ctypes.byref(kern_ev, 2 * nk * i * ctypes.sizeof(ctypes.c_void_p)),
                                ctypes.POINTER(ctypes.c_void_p)), 2 * nk)
            hip.record(call_ev[2 * i], stream)
            step()
            hip.record(call_ev[2 * i + 1], stream)
        kmeas.set_kernel_events(None, 0)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        calls = [hip.elapsed(call_ev[2 * i], call_ev[2 * i + 1]) for i in range(nsteps)]
        kern = {}
        if per_kernel:
            kern = {name: [hip.elapsed(kern_ev[2 * nk * i + 2 * j], kern_ev[2 * nk * i + 2 * j + 1])
                           for i in range(nsteps)] for j, name in enumerate(names)}
        hip.destroy(call_ev)
        if kern_ev is not None:
            hip.destroy(kern_ev)
        return calls, kern, wall

    res = {"workload": w, "inp": inp}
    if not recompute:  # only the saved-operand pair (profiler runs of its kernels)
        warm = forward = False
    else:
        for _ in range(warmup):
            step()
        res["cold_calls"], _, res["cold_wall"] = timed(steps, flush=True, per_kernel=False)
        _, res["cold_kern"], _ = timed(steps, flush=True, per_kernel=True)
        if clean_buf is not None:
            res["clean_calls"], _, _ = timed(steps, flush="clean", per_kernel=False)
            _, res["clean_kern"], _ = timed(steps, flush="clean", per_kernel=True)
    if warm:
        res["warm_calls"], _, _ = timed(steps, flush=False, per_kernel=False)
        _, res["warm_kern"], _ = timed(steps, flush=False, per_kernel=True)
    if forward:
        # The training forward (kda_fwd_states with the output o), timed the same way
        # (cold): reported beside the backward, not part of the step.
        def fwd_step():
            return kda.fwd_states(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"],
                                  cu_seqlens=inp["cu_seqlens"], C=w.C, scale=inp["scale"], output_o=True)

        for _ in range(2):
            fwd_step()
        fwd_ev = hip.events(2 * steps)
        torch.cuda.synchronize()
        for i in range(steps):
            flush_buf.fill_(i & 0xFF)
            hip.record(fwd_ev[2 * i], stream)
            fwd_step()
            hip.record(fwd_ev[2 * i + 1], stream)
        torch.cuda.synchronize()
        res["fwd_calls"] = [hip.elapsed(fwd_ev[2 * i], fwd_ev[2 * i + 1]) for i in range(steps)]
        hip.destroy(fwd_ev)
        # per-kernel times of the same calls, from the library's events (separate passes)
        fnames = table + FWD_KERNELS
        nf = len(fnames)
        fk_ev = hip.events(2 * nf * steps)
        torch.cuda.synchronize()
        for i in range(steps):
            flush_buf.fill_(i & 0xFF)
            kmeas.set_kernel_events(
                ctypes.cast(ctypes.byref(fk_ev, 2 * nf * i * ctypes.sizeof(ctypes.c_void_p)),
                            ctypes.POINTER(ctypes.c_void_p)), 2 * nf)
            fwd_step()
        kmeas.set_kernel_events(None, 0)
        torch.cuda.synchronize()
        res["fwd_kern"] = {name: [hip.elapsed(fk_ev[2 * nf * i + 2 * j], fk_ev[2 * nf * i + 2 * j + 1])
                                  for i in range(steps)] for j, name in enumerate(fnames)}
        hip.destroy(fk_ev)
    if saved:
        # Saved-operand mode: the forward also keeps kr, -w^T, Q'^T and e^gam; the backward
        # then runs without its prep kernel (a small W kernel where the scan takes W as seeds).
        fs = kda.fwd_states(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], cu_seqlens=inp["cu_seqlens"],
                            C=w.C, scale=inp["scale"], save=True)
        snames = table + ([] if scan_forms_w(w, inp) else ["bwd_w"]) + ["bwd_scan", "bwd_grad"]

        def sstep():
            kda.chunk_bwd_into(dims, d["q"], d["k"], d["v"], d["g"], d["beta"], fs["states"], fs["inv"], d["dO"],
                               d["dS_final"], dq, dk, dv, dg, dbeta, dh0, ws, stream=stream, saved=fs["saved"])

        def sfwd():
            return kda.fwd_states(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"],
                                  cu_seqlens=inp["cu_seqlens"], C=w.C, scale=inp["scale"], save=True)

        for _ in range(warmup):
            sstep()
        res["saved_calls"], _, _ = timed(steps, flush=True, per_kernel=False, step=sstep, names=snames)
        _, res["saved_kern"], _ = timed(steps, flush=True, per_kernel=True, step=sstep, names=snames)
        for _ in range(2):
            sfwd()
        res["saved_fwd_calls"], _, _ = timed(steps, flush=True, per_kernel=False, step=sfwd,
                                             names=table + FWD_KERNELS)
        _, res["saved_fwd_kern"], _ = timed(steps, flush=True, per_kernel=True, step=sfwd,
                                            names=table + FWD_KERNELS)
        res["saved_bytes"] = fs["saved"].numel()
        del fs
    del keep, fw, d, ws
    torch.cuda.empty_cache()
    return res


def summarize(res):
    """Median-based figures of one workload: call time, token-heads/s, the call's HBM
    roofline fraction and per-kernel times."""
    w, inp = res["workload"], res["inp"]
    th = inp["B"] * inp["T"] * w.HV
    ms = statistics.median(res["cold_calls"])
    abytes = algorithmic_bytes(w, inp)
    aflops = algorithmic_flops(w, inp)
    peak_flops = PEAK_F32_FLOPS if w.dtype == "f32" else PEAK_BF16_FLOPS
    t_roof = max(abytes / PEAK_HBM_BYTES, aflops / peak_flops)
    out = {"workload": w.name, "token_heads": th, "ms_cold_median": ms,
           "ms_cold_p10_p90": [_pct(res["cold_calls"], 0.1), _pct(res["cold_calls"], 0.9)],
           "token_heads_per_s": th / (ms * 1e-3), "algorithmic_bytes": abytes, "algorithmic_flops": aflops,
           "t_roofline_ms": t_roof * 1e3, "call_frac": t_roof / (ms * 1e-3),
           "kernels_ms_cold": {k: statistics.median(v) for k, v in res["cold_kern"].items()}}
    traffic = recorded_traffic(w.name)
    out["traffic"] = traffic  # rocprofv3 HBM bytes per call, or None (see recorded_traffic)
    out["traffic_over_algorithmic"] = None if traffic is None else traffic / abytes
    if "clean_calls" in res:
        cms = statistics.median(res["clean_calls"])
        out["cold_clean"] = {"ms_median": cms, "token_heads_per_s": th / (cms * 1e-3),
                             "call_frac": t_roof / (cms * 1e-3),
                             "kernels_ms": {k: statistics.median(v) for k, v in res["clean_kern"].items()}}
    if "warm_calls" in res:
        out["ms_warm_median"] = statistics.median(res["warm_calls"])
        out["kernels_ms_warm"] = {k: statistics.median(v) for k, v in res["warm_kern"].items()}
    if "fwd_calls" in res:
        fms = statistics.median(res["fwd_calls"])
        fb = fwd_algorithmic_bytes(w, inp)
        out["forward"] = {"entry": "kda_fwd_states with o (chunk prep, forward state scan, output)",
                          "ms_cold_median": fms, "token_heads_per_s": th / (fms * 1e-3),
                          "algorithmic_bytes": fb, "achieved_GBps": fb / (fms * 1e-3) / 1e9,
                          "hbm_frac": fb / (fms * 1e-3) / PEAK_HBM_BYTES,
                          "kernels_ms_cold": {k: statistics.median(v) for k, v in res.get("fwd_kern", {}).items()}}
    if "saved_calls" in res:
        bms = statistics.median(res["saved_calls"])
        fsms = statistics.median(res["saved_fwd_calls"])
        sb = abytes + saved_read_bytes(w, inp)
        blk = {"entries": "kda_fwd_states_save (forward with o, keeping kr, -w^T, Q'^T, e^gam) + "
                          "kda_chunk_bwd_saved",
               "bwd_ms_cold_median": bms, "bwd_token_heads_per_s": th / (bms * 1e-3),
               "bwd_kernels_ms_cold": {k: statistics.median(v) for k, v in res["saved_kern"].items()},
               "bwd_algorithmic_bytes": sb,
               "bwd_algorithmic_bytes_note": "the call's own algorithmic bytes plus the save it reads",
               "bwd_hbm_frac": sb / (bms * 1e-3) / PEAK_HBM_BYTES,
               "fwd_ms_cold_median": fsms,
               "fwd_kernels_ms_cold": {k: statistics.median(v) for k, v in res["saved_fwd_kern"].items()},
               "saved_bytes": res["saved_bytes"]}
        if "fwd_calls" in res:
            fms = statistics.median(res["fwd_calls"])
            blk["training_step_ms"] = {"recompute (kda_fwd_states with o + kda_chunk_bwd)": fms + ms,
                                       "saved operands": fsms + bms}
        out["saved_mode"] = blk
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=1, help="workload id (1 = B=2,T=2048,H=8,K=V=128,C=64)")
    ap.add_argument("--others", default="2,3,4",
                    help="further workload ids measured under per_workload ('' for none)")
    ap.add_argument("--other-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-saved", action="store_true",
                    help="skip the saved-operand pair (kda_fwd_states_save + kda_chunk_bwd_saved)")
    ap.add_argument("--saved-only", action="store_true",
                    help="time only the saved-operand pair on --workload and print its figures (for profiler "
                         "runs of its kernels)")
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

    hip = Hip()
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device=torch.device("cuda:0"))
    clean_buf = torch.zeros(1 << 30, dtype=torch.uint8, device=torch.device("cuda:0"))
    if args.saved_only:
        r = measure(args.workload, args.steps, args.warmup, hip, flush_buf, recompute=False)
        print(json.dumps({"workload": r["workload"].name, "saved_bwd_ms_cold_median": statistics.median(r["saved_calls"]),
                          "saved_bwd_kernels_ms_cold": {k: statistics.median(v) for k, v in r["saved_kern"].items()},
                          "saved_fwd_ms_cold_median": statistics.median(r["saved_fwd_calls"])}), flush=True)
        return
    main_res = measure(args.workload, args.steps, args.warmup, hip, flush_buf, saved=not args.no_saved,
                       clean_buf=clean_buf)
    s = summarize(main_res)
    w, inp = main_res["workload"], main_res["inp"]
    others = [int(x) for x in args.others.split(",") if x.strip()]
    per_workload = {}
    for wid in others:
        if wid == args.workload:
            continue
        r = measure(wid, args.other_steps, 2, hip, flush_buf, warm=False, forward=True, saved=not args.no_saved,
                    clean_buf=clean_buf)
        per_workload[str(wid)] = summarize(r)
        del r

    ms = s["ms_cold_median"]
    abytes = s["algorithmic_bytes"]
    achieved = abytes / (ms * 1e-3) / 1e9
    grad_ms = s["kernels_ms_cold"]["bwd_grad"]
    grad_achieved = abytes / (grad_ms * 1e-3) / 1e9
    traffic = recorded_traffic(w.name, "call")
    out = {
        "metric": "KDA chunk-bwd token-heads/s at K=V=128, C=64 (HBM roofline fraction)",
        "value": s["token_heads_per_s"],
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
        "config": {"workload": w.name, "B": inp["B"], "T": inp["T"], "H": w.H, "HV": w.HV, "K": w.K, "V": w.V,
                   "C": w.C, "token_heads": s["token_heads"],
                   "cache": "cold (1 GiB flush before each step, outside the timed interval)",
                   "timing": "median of the timed steps"},
        # The whole kda_chunk_bwd call is the unit: its algorithmic bytes over its median cold
        # time, against the HBM peak; traffic is the counters' HBM bytes of one call (the
        # three kernels' FETCH_SIZE and WRITE_SIZE, calibrated), null if the sources changed.
        "roofline": {"bound": "hbm", "unit": "GB/s", "achieved": achieved, "peak": PEAK_HBM_BYTES / 1e9,
                     "frac": achieved / (PEAK_HBM_BYTES / 1e9), "traffic": traffic,
                     "scope": "kda_chunk_bwd call (prep + reverse scan + gradients)",
                     "algorithmic_bytes_per_call": abytes, "call_ms": ms,
                     "traffic_over_algorithmic": (traffic / abytes) if traffic else None,
                     "dominant_kernel": {"kernel": "bwd_grad", "launch_ms": grad_ms,
                                         "achieved": grad_achieved,
                                         "frac": grad_achieved / (PEAK_HBM_BYTES / 1e9),
                                         "traffic": recorded_traffic(w.name, "bwd_grad"),
                                         "note": "every algorithmic byte of the call credited to this one "
                                                 "kernel's time"},
                     "flops_frac_bf16": s["algorithmic_flops"] / (ms * 1e-3) / PEAK_BF16_FLOPS},
        "ms_per_step_p10_p50_p90_cold": [s["ms_cold_p10_p90"][0], ms, s["ms_cold_p10_p90"][1]],
        "ms_per_step_warm_median": s["ms_warm_median"],
        # The same call after a flush that leaves the caches holding clean lines (1 GiB written,
        # then another 1 GiB read): the headline's flush leaves them dirty, so its reads also
        # wait for the flush's write-backs.
        "cold_clean": dict(s["cold_clean"], flush="1 GiB written, then a second 1 GiB buffer read"),
        "kernels_ms_cold": s["kernels_ms_cold"],
        "kernels_ms_warm": s["kernels_ms_warm"],
        "forward": s["forward"],
        "saved_mode": s.get("saved_mode"),
        "per_workload": per_workload,
        "wall_s_timed_cold_incl_flush": main_res["cold_wall"],
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
