"""kda_chunk_bwd_noalloc (the entry point for callers that cannot allocate) against
kda_chunk_bwd with a caller workspace, through the C ABI: two calls in a row, the second on
a smaller (packed, grouped-head) input, each bitwise equal to the workspace entry point's
result on the same inputs -- the same kernels run, only the workspace differs, and the
library's static one still holds the first call's contents during the second."""
import numpy as np
import pytest
import torch

import chunked_gated_delta_09_amd as kda
from chunked_gated_delta_09_amd import inputs as kin
from tests.kda_cases import small_workload, to_dev

OUTS = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _setup(inp):
    w = inp["workload"]
    d = {n: to_dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "h0", "dS_final", "dO")}
    f = kda.fwd_states(d["q"], d["k"], d["v"], d["g"], d["beta"], h0=d["h0"], cu_seqlens=inp["cu_seqlens"], C=w.C,
                       scale=inp["scale"])
    cu = inp["cu_seqlens"]
    cu_dev = torch.tensor(cu, dtype=torch.int32, device="cuda") if cu is not None else None
    dims, keep = kda.make_dims(inp["B"], inp["T"], w.H, w.HV, w.K, w.V, w.C, inp["scale"], w.dtype, cu, cu_dev)
    return d, f, dims, keep


def _outputs(inp, d):
    w = inp["workload"]
    return dict(dq=torch.full_like(d["q"], float("nan")), dk=torch.full_like(d["k"], float("nan")),
                dv=torch.full_like(d["v"], float("nan")), dg=torch.full_like(d["g"], float("nan")),
                dbeta=torch.full_like(d["beta"], float("nan")),
                dh0=torch.full((inp["N"], w.HV, w.K, w.V), float("nan"), dtype=torch.float32, device="cuda"))


def _run(inp, noalloc):
    d, f, dims, keep = _setup(inp)
    o = _outputs(inp, d)
    args = (dims, d["q"], d["k"], d["v"], d["g"], d["beta"], f["states"], f["inv"], d["dO"], d["dS_final"],
            o["dq"], o["dk"], o["dv"], o["dg"], o["dbeta"], o["dh0"])
    if noalloc:
        kda.chunk_bwd_noalloc_into(*args)
    else:
        ws = torch.empty(kda.bwd_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
        kda.chunk_bwd_into(*args, ws)
    torch.cuda.synchronize()
    del keep
    return {k: v.float().cpu().numpy() for k, v in o.items()}


def test_noalloc_rejects_oversized_calls():
    """No GPU work: a call whose workspace exceeds the static array fails validation."""
    import ctypes
    lib = kda.load()
    dims, _ = kda.make_dims(1, 16384, 16, 16, 128, 128, 64)  # 4096 chunk-heads: far beyond 64 MiB
    assert kda.bwd_workspace_bytes(dims) > 64 << 20
    p = ctypes.c_void_p(1)
    st = lib.kda_chunk_bwd_noalloc(ctypes.byref(dims), p, p, p, p, p, p, p, p, None, p, p, p, p, p, None, None)
    assert st == -1
    assert "static scratch" in lib.kda_last_error().decode()
    dims.H = 3  # invalid dims are reported as by kda_chunk_bwd
    assert lib.kda_chunk_bwd_noalloc(ctypes.byref(dims), p, p, p, p, p, p, p, p, None, p, p, p, p, p, None,
                                     None) == -1
    assert "multiple of H" in lib.kda_last_error().decode()


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice():
    big = kin.make_inputs(kin.WORKLOADS[1], wid=1)  # B=2, T=2048, H=8, K=V=128, C=64
    small = kin.make_inputs(small_workload("noalloc_small", H=2, HV=6, varlen=3, total=300, len_lo=20, len_hi=200,
                                           has_h0=True, has_dsf=True), seed=21)
    d, _, dims, keep = _setup(big)
    assert kda.bwd_workspace_bytes(dims) <= 64 << 20
    del d, keep
    for tag, inp in (("bench workload", big), ("smaller packed grouped-head input", small)):
        print(f"[noalloc] {tag}", flush=True)
        ref = _run(inp, noalloc=False)
        got = _run(inp, noalloc=True)
        for key in OUTS:
            assert np.isfinite(got[key]).all(), (tag, key)
            np.testing.assert_array_equal(got[key], ref[key], err_msg=f"{tag}: {key}")
