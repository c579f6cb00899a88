"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (relative L2): 1e-4 for fp32 workloads, 2e-2 for bf16 ones, held by every
tensor as a whole and by each of its (chunk, head) pieces (tests/kda_cases.compare). Small
cases span several chunks and ragged tails; the five full workloads run at full size on the
GPU with the oracle evaluated on sampled heads (every sequence of those heads).
"""
import numpy as np
import pytest
import torch

from chunked_gated_delta_09_amd import inputs as kin
from oracle.chunked import chunked_fwd_bwd
from tests.kda_cases import GRADS, TOL, compare, rel_l2, run_gpu, run_oracle, small_workload

pytestmark = pytest.mark.gpu


def _report(tag, errs):
    print(f"[{tag}] " + " ".join(f"{k}={v:.2e}" for k, v in sorted(errs.items())), flush=True)


def test_workload0_tiny_fp32_all_outputs(oracle_mod):
    inp = kin.make_inputs(kin.WORKLOADS[0], wid=0)
    out = run_gpu(inp)
    ref = run_oracle(oracle_mod, inp)
    errs, bad = compare(inp, out, ref)
    _report("w0", errs)
    assert set(errs) >= set(GRADS) | {"o", "final_state"}
    assert not bad, bad


SMALL = {
    "dense_ragged": small_workload("dense_ragged", B=2, T=200, H=2, HV=2, has_h0=True, has_dsf=True),
    "gva_ragged": small_workload("gva_ragged", B=1, T=130, H=1, HV=4, has_h0=True, has_dsf=True),
    "varlen_edges": small_workload("varlen_edges", H=2, HV=2, varlen=5, total=264, len_lo=0, len_hi=200,
                                   has_h0=True, has_dsf=True),
    "c16": small_workload("c16", B=1, T=90, H=2, HV=2, C=16, has_h0=True, has_dsf=True),
    "single_partial_chunk": small_workload("single_partial_chunk", B=3, T=37, H=1, HV=2, has_dsf=True),
    "gva3_varlen": small_workload("gva3_varlen", H=2, HV=6, varlen=3, total=300, len_lo=20, len_hi=200,
                                  has_h0=True, has_dsf=True),
    "gva8": small_workload("gva8", B=1, T=96, H=1, HV=8, has_h0=False, has_dsf=True),
    # enough (sequence, head) pairs that the reverse scan holds 4 (many_heads) or 8 (many_seqs)
    # value slices per workgroup and forms W = Q'^T dO itself
    "many_heads": small_workload("many_heads", B=1, T=200, H=72, HV=72, has_h0=True, has_dsf=True),
    "many_seqs": small_workload("many_seqs", H=4, HV=8, varlen=40, total=3000, len_lo=0, len_hi=150,
                                has_h0=True, has_dsf=True),
    "many_heads_c16": small_workload("many_heads_c16", B=1, T=90, H=72, HV=72, C=16, has_h0=True, has_dsf=True),
}


def _small_inputs(name):
    w = SMALL[name]
    inp = kin.make_inputs(w, seed=77)
    if name == "varlen_edges":
        # fixed lengths with an empty sequence, a single token, exact and ragged chunks
        lens = [70, 0, 1, 129, 64]
        cu = [0]
        for ln in lens:
            cu.append(cu[-1] + ln)
        inp["cu_seqlens"] = cu
    if name == "many_seqs":
        # an empty sequence, a single token and exact one- and two-chunk sequences among them
        cu = inp["cu_seqlens"]
        lens = [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]
        lens[3], lens[7], lens[11], lens[12] = 0, 1, 64, 128
        lens[-1] = cu[-1] - sum(lens[:-1])
        assert lens[-1] >= 1
        inp["cu_seqlens"] = [0] + [int(x) for x in np.cumsum(lens)]
    return inp


@pytest.mark.parametrize("name", list(SMALL))
def test_small_cases(oracle_mod, name):
    inp = _small_inputs(name)
    out = run_gpu(inp)
    ref = run_oracle(oracle_mod, inp)
    errs, bad = compare(inp, out, ref)
    _report(name, errs)
    assert not bad, bad


def test_stage_parity_states_and_inverse(oracle_mod):
    """Per-chunk S_in and INV of the forward against the fp64 chunked reference."""
    inp = _small_inputs("gva_ragged")
    out = run_gpu(inp)
    B, T = inp["B"], inp["T"]
    f = lambda t: t.float().numpy().astype(np.float64).reshape(B * T, *t.shape[2:])
    ref = chunked_fwd_bwd(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["g"]), f(inp["beta"]).reshape(B * T, -1),
                          kin.flat_cu(inp), inp["scale"], 64, h0=inp["h0"].double().numpy(),
                          dO=f(inp["dO"]), dS_final=inp["dS_final"].double().numpy())
    e_states = rel_l2(out["states"], ref["states"])
    e_inv = rel_l2(out["inv"], ref["inv"])
    print(f"[stage] states={e_states:.2e} inv={e_inv:.2e}", flush=True)
    assert e_states < 1e-2 and e_inv < 1e-2


@pytest.mark.parametrize("name", ["varlen_edges", "gva3_varlen", "c16", "many_heads", "many_seqs", "many_heads_c16"])
def test_stage_parity_state_gradients(name):
    """Per-chunk state gradients of the reverse scan (the dS_out each chunk's products consume;
    FlashKDA backward page, step 2) against the fp64 chunked reference's, on packed ragged
    sequences (an empty and a one-token sequence among them), grouped heads and C = 16."""
    import chunked_gated_delta_09_amd as kda
    from chunked_gated_delta_09_amd.measure import bwd_state_grads
    from tests.kda_cases import chunk_errors, to_dev
    inp = _small_inputs(name)
    w = inp["workload"]
    q, k, v, g, beta, h0, dsf, dO = (to_dev(inp[n]) for n in ("q", "k", "v", "g", "beta", "h0", "dS_final", "dO"))
    f = kda.fwd_states(q, k, v, g, beta, h0=h0, cu_seqlens=inp["cu_seqlens"], C=w.C, scale=inp["scale"])
    cu = inp["cu_seqlens"]
    cu_dev = torch.tensor(cu, dtype=torch.int32, device="cuda") if cu is not None else None
    dims, keep = kda.make_dims(inp["B"], inp["T"], w.H, w.HV, w.K, w.V, w.C, inp["scale"], w.dtype, cu, cu_dev)
    outs = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                dg=torch.empty_like(g), dbeta=torch.empty_like(beta),
                dh0=torch.empty(inp["N"], w.HV, w.K, w.V, dtype=torch.float32, device="cuda"))
    ws = torch.empty(kda.bwd_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    kda.chunk_bwd_into(dims, q, k, v, g, beta, f["states"], f["inv"], dO, dsf, outs["dq"], outs["dk"], outs["dv"],
                       outs["dg"], outs["dbeta"], outs["dh0"], ws)
    got = bwd_state_grads(dims, ws).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    B, T = inp["B"], inp["T"]
    fl = lambda t: t.float().numpy().astype(np.float64).reshape(B * T, *t.shape[2:])
    ref = chunked_fwd_bwd(fl(inp["q"]), fl(inp["k"]), fl(inp["v"]), fl(inp["g"]),
                          fl(inp["beta"]).reshape(B * T, -1), kin.flat_cu(inp), inp["scale"], w.C,
                          h0=None if inp["h0"] is None else inp["h0"].double().numpy(), dO=fl(inp["dO"]),
                          dS_final=None if inp["dS_final"] is None else inp["dS_final"].double().numpy())
    e = rel_l2(got, ref["dstates"])
    # each chunk-head's K x V gradient judged on its own (a chunk is one row of this tensor)
    per = chunk_errors(got.reshape(got.shape[0], w.HV, -1), ref["dstates"].reshape(got.shape[0], w.HV, -1),
                       [0, got.shape[0]], 1)
    print(f"[stage dS {name}] all={e:.2e} worst chunk-head={per.max():.2e}", flush=True)
    assert got.shape == ref["dstates"].shape
    assert e < 1e-2 and per.max() < 1e-2
    del keep


def test_chunk_size_invariance_bf16(oracle_mod):
    """C = 16 and C = 64 are two tilings of the same map."""
    w = small_workload("cinv", B=1, T=160, H=1, HV=2, has_h0=True, has_dsf=True)
    inp = kin.make_inputs(w, seed=5)
    a = run_gpu(inp, C=64)
    b = run_gpu(inp, C=16)
    ref = run_oracle(oracle_mod, inp)
    for out in (a, b):
        errs, bad = compare(inp, out, ref)
        assert not bad, bad
    for key in GRADS:
        assert rel_l2(a[key], b[key]) < 2e-2, key


def test_bitwise_determinism():
    inp = _small_inputs("gva_ragged")
    a = run_gpu(inp)
    b = run_gpu(inp)
    for key in GRADS + ["states", "inv", "o", "final_state"]:
        assert np.array_equal(a[key], b[key]), key


def test_empty_input():
    """T = 0: no chunk; final state = h0 and dh0 = dS_final."""
    import chunked_gated_delta_09_amd as kda
    w = small_workload("empty", B=2, T=0, H=1, HV=1, has_h0=True, has_dsf=True)
    inp = kin.make_inputs(w, seed=3)
    out = run_gpu(inp, output_o=False)
    assert out["states"].shape[0] == 0
    np.testing.assert_allclose(out["final_state"], inp["h0"].float().numpy(), rtol=0, atol=0)
    np.testing.assert_allclose(out["dh0"], inp["dS_final"].float().numpy(), rtol=0, atol=0)
    del kda


# Full-size workloads: GPU on everything, oracle on sampled q/k heads (the last head of
# every workload among them), every sequence of those heads, judged per tensor and per
# (chunk, head).
FULL_SAMPLES = {1: [0, 5, 7], 2: [3, 15], 3: [7, 15], 4: [2, 7]}


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_full_workload_sampled_heads(oracle_mod, wid):
    inp = kin.make_inputs(kin.WORKLOADS[wid], wid=wid)
    print(f"[full w{wid}] running GPU", flush=True)
    out = run_gpu(inp, output_o=False)
    for key in GRADS:
        assert np.isfinite(out[key]).all(), key
    heads = FULL_SAMPLES[wid]
    print(f"[full w{wid}] running oracle on q/k heads {heads}", flush=True)
    ref = run_oracle(oracle_mod, inp, qk_heads=heads)
    errs, bad = compare(inp, out, ref, qk_heads=heads)
    _report(f"full w{wid}", errs)
    assert not bad, bad


@pytest.mark.parametrize("name", ["dense_ragged", "varlen_edges", "w0_fp32"])
def test_beta_logits(oracle_mod, name):
    """beta given as logits (sigmoid in the kernels, dbeta w.r.t. the logits) against the
    oracle in the same mode."""
    inp = kin.make_inputs(kin.WORKLOADS[0], wid=0) if name == "w0_fp32" else _small_inputs(name)
    gen = torch.Generator().manual_seed(33)
    inp["beta"] = 1.5 * torch.randn(inp["beta"].shape, generator=gen)
    out = run_gpu(inp, beta_logits=True)
    ref = run_oracle(oracle_mod, inp, beta_logits=True)
    errs, bad = compare(inp, out, ref)
    _report(f"logits {name}", errs)
    assert "dbeta" in errs and not bad, bad


def test_strong_decay_c16(oracle_mod):
    """Per-token gates in [-5, -0.5] (a chunk of 64 tokens would sum to about -175, beyond the
    fp32 range of the factorised e^{+-G}); with C = 16 every chunk-local cumsum stays above -80,
    so the kernels' e^{-G} stays below ~6e34, and the result matches the oracle."""
    w = small_workload("strong_decay", B=2, T=100, H=2, HV=4, C=16, has_h0=True, has_dsf=True)
    inp = kin.make_inputs(w, seed=21)
    gen = torch.Generator().manual_seed(22)
    inp["g"] = -(0.5 + 4.5 * torch.rand(inp["g"].shape, generator=gen))
    assert float(inp["g"].min()) >= -5.0
    out = run_gpu(inp)
    for key in GRADS:
        assert np.isfinite(out[key]).all(), key
    ref = run_oracle(oracle_mod, inp)
    errs, bad = compare(inp, out, ref)
    _report("strong decay C=16", errs)
    # Per tensor: the usual 2e-2. Per (chunk, head): within twice (plus 1e-3) what the bf16
    # error model of the chunk form predicts for the same chunk -- under this decay a bf16
    # implementation of the factorised form loses up to ~8e-2 of dg in single chunks.
    assert not {k: v for k, v in bad.items() if "@chunk" not in k}, bad
    B, T = inp["B"], inp["T"]
    f = lambda t: t.float().numpy().astype(np.float64).reshape(B * T, *t.shape[2:])
    model = chunked_fwd_bwd(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["g"]), f(inp["beta"]).reshape(B * T, -1),
                            kin.flat_cu(inp), inp["scale"], w.C, h0=inp["h0"].double().numpy(), dO=f(inp["dO"]),
                            dS_final=inp["dS_final"].double().numpy(), bf16_operands=True)
    from tests.kda_cases import chunk_errors, gpu_on_heads
    got = gpu_on_heads(inp, out)
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        g_ce = chunk_errors(got[key], ref[key], kin.flat_cu(inp), w.C)
        m_ce = chunk_errors(model[key], ref[key], kin.flat_cu(inp), w.C)
        print(f"[strong decay C=16] {key}@chunk gpu {g_ce.max():.2e} model {m_ce.max():.2e}", flush=True)
        assert np.all(g_ce <= np.maximum(TOL["bf16"], 2 * m_ce + 1e-3)), key


@pytest.mark.parametrize("channels", ["all", "upper_half", "one"])
def test_strong_decay_c64(oracle_mod, channels):
    """Per-token gates in [-5, -0.5] with C = 64: a chunk-local cumsum reaches -100 to -320,
    where e^{-G} alone is beyond fp32 (and e^{G} below it). The kernels refer each 16-row
    block to its first row wherever a wave's columns need it, so no factor they form exceeds
    e^{85}; every output is finite and within the bf16 tolerance per tensor. The strong gates
    cover every channel, the upper half of the channels (waves with and without block
    references in one chunk) or a single channel. Per (chunk, head) the error is held to
    three times the tolerance."""
    w = small_workload("strong_decay_c64", B=2, T=150, H=2, HV=4, C=64, has_h0=True, has_dsf=True)
    inp = kin.make_inputs(w, seed=23)
    gen = torch.Generator().manual_seed(24)
    strong = -(0.5 + 4.5 * torch.rand(inp["g"].shape, generator=gen))
    if channels == "all":
        inp["g"] = strong
    elif channels == "upper_half":
        inp["g"][..., 64:] = strong[..., 64:]
    else:
        inp["g"][..., 37] = strong[..., 37]
    assert float(inp["g"].min()) >= -5.0
    out = run_gpu(inp)
    for key in GRADS + ["o", "final_state"]:
        assert out.get(key) is not None and np.isfinite(out[key]).all(), key
    ref = run_oracle(oracle_mod, inp)
    errs, bad = compare(inp, out, ref)
    _report(f"strong decay C=64 {channels}", errs)
    assert not {k: v for k, v in bad.items() if "@chunk" not in k}, bad
    assert all(v <= 3 * TOL["bf16"] for k, v in errs.items() if "@chunk" in k), errs


def test_strong_decay_some_chunks_packed_gva(oracle_mod):
    """Strong gates ([-5, -0.5]) in the tokens of a few chunks only, on packed ragged sequences
    with grouped heads at C = 64: chunk-heads with and without block references side by side in
    one launch, and a strong chunk next to a sequence boundary."""
    inp = _small_inputs("gva3_varlen")
    cu = [int(x) for x in inp["cu_seqlens"]]
    gen = torch.Generator().manual_seed(31)
    strong = -(0.5 + 4.5 * torch.rand(inp["g"].shape, generator=gen))
    g = inp["g"].clone()
    # the second chunk of every sequence, and the last 40 tokens of the first
    for a, b in zip(cu[:-1], cu[1:]):
        g[:, a + 64:min(a + 128, b)] = strong[:, a + 64:min(a + 128, b)]
    g[:, max(cu[0], cu[1] - 40):cu[1]] = strong[:, max(cu[0], cu[1] - 40):cu[1]]
    inp["g"] = g
    out = run_gpu(inp)
    for key in GRADS + ["o", "final_state"]:
        assert np.isfinite(out[key]).all(), key
    ref = run_oracle(oracle_mod, inp)
    errs, bad = compare(inp, out, ref)
    _report("strong decay some chunks, packed GVA", errs)
    assert not {k: v for k, v in bad.items() if "@chunk" not in k}, bad
    assert all(v <= 3 * TOL["bf16"] for k, v in errs.items() if "@chunk" in k), errs


def test_strong_decay_fp32_c16(oracle_mod):
    """fp32 path (K = V = C = 16) with per-token gates in [-5.5, -4.5]: chunk-local cumsums reach
    -72 to -88, so some chunks take the block reference (one block per chunk) and some do not.
    Every output is held to the fp32 tolerance, except dg, which under this decay is mostly the
    cancellation of pair terms: it is held to three times (plus 1e-6) what the chunk form
    predicts with fp32-rounded operands, per tensor and per (chunk, head)."""
    w = small_workload("strong_fp32", B=2, T=70, H=1, HV=2, K=16, V=16, C=16, dtype="f32",
                       has_h0=True, has_dsf=True)
    inp = kin.make_inputs(w, seed=41)
    gen = torch.Generator().manual_seed(42)
    inp["g"] = -(4.5 + 1.0 * torch.rand(inp["g"].shape, generator=gen))
    out = run_gpu(inp)
    for key in GRADS + ["o", "final_state"]:
        assert np.isfinite(out[key]).all(), key
    ref = run_oracle(oracle_mod, inp)
    errs, bad = compare(inp, out, ref)
    _report("strong decay fp32 C=16", errs)
    assert not {k: v for k, v in bad.items() if not k.startswith("dg")}, bad
    from tests.kda_cases import chunk_errors, gpu_on_heads
    B, T = inp["B"], inp["T"]
    f = lambda t: t.float().numpy().astype(np.float64).reshape(B * T, *t.shape[2:])
    model = chunked_fwd_bwd(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["g"]), f(inp["beta"]).reshape(B * T, -1),
                            kin.flat_cu(inp), inp["scale"], w.C, h0=inp["h0"].double().numpy(), dO=f(inp["dO"]),
                            dS_final=inp["dS_final"].double().numpy(), f32_operands=True)
    got = gpu_on_heads(inp, out)
    m_t = rel_l2(model["dg"], ref["dg"])
    g_ce = chunk_errors(got["dg"], ref["dg"], kin.flat_cu(inp), w.C)
    m_ce = chunk_errors(model["dg"], ref["dg"], kin.flat_cu(inp), w.C)
    print(f"[strong decay fp32 C=16] dg gpu {errs['dg']:.2e} model {m_t:.2e}; per chunk gpu {g_ce.max():.2e} "
          f"model {m_ce.max():.2e}", flush=True)
    assert errs["dg"] <= max(TOL["f32"], 3 * m_t + 1e-6)
    assert np.all(g_ce <= np.maximum(TOL["f32"], 3 * m_ce + 1e-6))


@pytest.mark.parametrize("name", ["dense_ragged", "gva_ragged"])
def test_error_matches_bf16_model(oracle_mod, name):
    """The kernels lose no more precision than a bf16 implementation should: each gradient's
    error against the oracle is within twice (plus 1e-3) what the chunked reference predicts
    when every product operand and kept tensor is rounded to bf16."""
    from oracle.chunked import chunked_fwd_bwd
    inp = _small_inputs(name)
    out = run_gpu(inp)
    ref = run_oracle(oracle_mod, inp)
    B, T = inp["B"], inp["T"]
    f = lambda t: t.float().numpy().astype(np.float64).reshape(B * T, *t.shape[2:])
    model = chunked_fwd_bwd(f(inp["q"]), f(inp["k"]), f(inp["v"]), f(inp["g"]), f(inp["beta"]).reshape(B * T, -1),
                            kin.flat_cu(inp), inp["scale"], 64, h0=inp["h0"].double().numpy(), dO=f(inp["dO"]),
                            dS_final=inp["dS_final"].double().numpy(), bf16_operands=True)
    errs, bad = compare(inp, out, ref)
    assert not bad, bad
    for key in GRADS:
        predicted = rel_l2(model[key], ref[key])
        print(f"[bf16 model {name}] {key}: gpu {errs[key]:.2e} model {predicted:.2e}", flush=True)
        assert errs[key] <= 2 * predicted + 1e-3, (key, errs[key], predicted)


@pytest.mark.parametrize("case", ["beta_one", "no_decay", "beta_one_no_decay"])
def test_boundary_gates(oracle_mod, case):
    """The method's boundary settings: beta = 1 (each write replaces the key's component of the
    state) and g = 0 (no decay), alone and together, on ragged chunks with h0 and dS_final."""
    inp = _small_inputs("dense_ragged")
    if "beta_one" in case:
        inp["beta"] = torch.ones_like(inp["beta"])
    if "no_decay" in case:
        inp["g"] = torch.zeros_like(inp["g"])
    out = run_gpu(inp)
    ref = run_oracle(oracle_mod, inp)
    errs, bad = compare(inp, out, ref)
    _report(case, errs)
    assert not bad, bad


def _random_case(i):
    """Seeded random geometry: precision, chunk size, heads and grouping, dense or packed
    lengths (empty and one-token sequences included), initial state and final-state gradient,
    beta or its logits."""
    rng = np.random.default_rng(500 + i)
    f32 = rng.random() < 0.25
    dims = dict(K=16, V=16, C=16, dtype="f32") if f32 else dict(K=128, V=128, C=int(rng.choice([16, 64])),
                                                                   dtype="bf16")
    H = int(rng.integers(1, 4))
    HV = H * int(rng.integers(1, 5))
    has_h0, has_dsf = bool(rng.random() < 0.7), bool(rng.random() < 0.7)
    if rng.random() < 0.5:
        w = small_workload(f"rand{i}", B=int(rng.integers(1, 4)), T=int(rng.integers(1, 260)), H=H, HV=HV,
                           has_h0=has_h0, has_dsf=has_dsf, **dims)
        inp = kin.make_inputs(w, seed=600 + i)
    else:
        lens = [int(x) for x in rng.integers(0, 200, size=int(rng.integers(1, 6)))]
        lens[int(rng.integers(0, len(lens)))] = int(rng.choice([0, 1, 64, 65]))
        if sum(lens) == 0:
            lens[0] = 7
        cu = [0]
        for ln in lens:
            cu.append(cu[-1] + ln)
        w = small_workload(f"rand{i}", varlen=len(lens), total=cu[-1], len_lo=0, len_hi=cu[-1], H=H, HV=HV,
                           has_h0=has_h0, has_dsf=has_dsf, **dims)
        inp = kin.make_inputs(w, seed=600 + i)
        inp["cu_seqlens"] = cu
    logits = bool(rng.random() < 0.3)
    if logits:
        inp["beta"] = torch.from_numpy(rng.normal(0.0, 1.5, size=tuple(inp["beta"].shape)).astype(np.float32))
    return inp, logits


@pytest.mark.parametrize("i", range(12))
def test_random_geometries(oracle_mod, i):
    inp, logits = _random_case(i)
    w = inp["workload"]
    print(f"[rand {i}] {w.dtype} C={w.C} H={w.H} HV={w.HV} cu={inp['cu_seqlens']} B={inp['B']} T={inp['T']} "
          f"h0={inp['h0'] is not None} dsf={inp['dS_final'] is not None} logits={logits}", flush=True)
    out = run_gpu(inp, beta_logits=logits)
    ref = run_oracle(oracle_mod, inp, beta_logits=logits)
    errs, bad = compare(inp, out, ref)
    _report(f"rand {i}", errs)
    assert not bad, bad


@pytest.mark.parametrize("i", range(8))
def test_random_geometries_strong_gates(oracle_mod, i):
    """Random bf16 geometries (as above, C = 16 or 64, dense or packed) with per-token gates in
    [-5.5, -0.5] on a random set of channels over a random token range: chunk-heads, waves and
    columns with and without block references mixed at random. Per tensor within 2e-2, per
    (chunk, head) within three times that (dg under strong decay is mostly cancellation)."""
    inp, logits = _random_case(100 + i)
    while inp["workload"].dtype != "bf16":
        i += 1000
        inp, logits = _random_case(100 + i)
    w = inp["workload"]
    rng = np.random.default_rng(900 + i)
    g = inp["g"].clone()
    ntok = g.shape[1]
    a = int(rng.integers(0, max(1, ntok)))
    b = int(rng.integers(a, ntok + 1))
    chans = torch.from_numpy(rng.random(w.K) < rng.uniform(0.05, 1.0))
    strong = -(0.5 + 5.0 * torch.from_numpy(rng.random(tuple(g.shape)).astype(np.float32)))
    sel = torch.zeros_like(g, dtype=torch.bool)
    sel[:, a:b, :, :] = chans
    g = torch.where(sel, strong, g)
    inp["g"] = g
    print(f"[rand strong {i}] C={w.C} H={w.H} HV={w.HV} cu={inp['cu_seqlens']} B={inp['B']} T={inp['T']} "
          f"tokens {a}:{b} channels {int(chans.sum())}", flush=True)
    out = run_gpu(inp, beta_logits=logits)
    for key in GRADS + ["o", "final_state"]:
        if out.get(key) is not None:
            assert np.isfinite(out[key]).all(), key
    ref = run_oracle(oracle_mod, inp, beta_logits=logits)
    errs, bad = compare(inp, out, ref)
    _report(f"rand strong {i}", errs)
    assert not {k: v for k, v in bad.items() if "@chunk" not in k}, bad
    assert all(v <= 3 * TOL["bf16"] for k, v in errs.items() if "@chunk" in k), errs
