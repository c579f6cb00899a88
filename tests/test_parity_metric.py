"""The parity metric itself (CPU): a localized error that the whole-tensor relative L2 error
lets through is caught by the per-(chunk, head) check in tests/kda_cases.compare. The
planted mistakes are in a copy of the oracle's own output; no GPU is involved."""
import numpy as np

from chunked_gated_delta_09_amd import inputs as kin
from tests.kda_cases import chunk_errors, compare, run_oracle, small_workload


def _as_gpu_layout(inp, ref):
    """The oracle's outputs arranged as the library returns them ([B, T, heads, ...])."""
    B, T = inp["B"], inp["T"]
    w = inp["workload"]
    out = {}
    for key, rkey, heads in (("dq", "dq", w.H), ("dk", "dk", w.H), ("dv", "dv", w.HV), ("dg", "dg", w.HV),
                             ("o", "o", w.HV)):
        out[key] = ref[rkey].reshape(B, T, heads, -1).copy()
    out["dbeta"] = ref["dbeta"].reshape(B, T, w.HV).copy()
    out["dh0"] = ref["dh0"].copy()
    out["final_state"] = ref["S_T"].copy()
    return out


def test_localized_errors_fail_per_chunk_only(oracle_mod):
    # 256 chunks of 64 tokens on one head: one wrong row is ~1/128 of a tensor's norm, five
    # wrong rows ~1/57
    w = small_workload("metric", B=1, T=16384, H=1, HV=1, K=16, V=16, C=64, dtype="f32", has_h0=True,
                       has_dsf=True)
    inp = kin.make_inputs(w, seed=11)
    ref = run_oracle(oracle_mod, inp)
    exact = _as_gpu_layout(inp, ref)
    errs, bad = compare(inp, exact, ref, tol=2e-2)
    assert not bad and max(errs.values()) == 0.0

    # one token's dq row doubled: the tensor passes 2e-2, its chunk does not
    one_row = _as_gpu_layout(inp, ref)
    one_row["dq"][0, 5000] *= 2.0
    errs, bad = compare(inp, one_row, ref, tol=2e-2)
    assert errs["dq"] < 2e-2, errs["dq"]
    assert set(bad) == {"dq@chunk"}, bad

    # the last 5 rows of the sequence (the end of its last chunk) of dv zeroed: same outcome
    tail = _as_gpu_layout(inp, ref)
    tail["dv"][0, -5:] = 0.0
    errs, bad = compare(inp, tail, ref, tol=2e-2)
    assert errs["dv"] < 2e-2, errs["dv"]
    assert set(bad) == {"dv@chunk"}, bad


def test_chunk_errors_floor_and_shape():
    """Chunks follow the sequence boundaries (a chunk never straddles two sequences); a chunk
    whose reference is zero is judged against the tensor's scale, not divided by zero."""
    rng = np.random.default_rng(0)
    ref = rng.normal(size=(100, 2, 3))
    ref[0:10, 0] = 0.0  # the first chunk of head 0 has a zero reference
    x = ref.copy()
    x[0:10, 0] = 1e-9
    cu = [0, 10, 100]  # sequences of 10 and 90 tokens, chunks of 64: 1 + 2 chunks
    ce = chunk_errors(x, ref, cu, 64)
    assert ce.shape == (3, 2)
    assert np.all(np.isfinite(ce)) and ce.max() < 1e-8
    assert ce[1:, :].max() == 0.0
