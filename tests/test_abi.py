"""C ABI checks that need no GPU: the library loads, exports every function that
include/kda.h declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import chunked_gated_delta_09_amd as kda
from chunked_gated_delta_09_amd import inputs as kin

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    """Every kda_* function declared in the headers under include/."""
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, f)).read(), flags=re.S)
            names |= set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return kda.load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"kda_fwd_states", "kda_chunk_bwd", "kda_last_error"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def _dims(**kw):
    base = dict(B=2, T=2048, H=8, HV=8, K=128, V=128, C=64, scale=None, dtype="bf16")
    base.update(kw)
    d, keep = kda.make_dims(**base)
    return d, keep


def test_chunk_counts_and_workspace_sizes(lib):
    d, _ = _dims()
    assert kda.num_chunks(d) == 64
    wsb = kda.bwd_workspace_bytes(d)
    # kr, -w^T, W, dS, (kr dS)^T in bf16 and e^gam in fp32, per chunk-head
    per = 64 * 128 * 2 * 2 + 128 * 128 * 2 * 2 + 128 * 64 * 2 + 128 * 4
    assert wsb >= 64 * 8 * per
    d, keep = kda.make_dims(1, 300, 2, 2, 128, 128, 64, cu_seqlens=[0, 70, 70, 71, 300])
    assert kda.num_chunks(d) == 2 + 0 + 1 + 4
    d, _ = kda.make_dims(1, 64, 1, 1, 16, 16, 16, dtype="f32")
    assert kda.num_chunks(d) == 4


def _call_bwd(lib, d, ptr=1):
    p = ctypes.c_void_p(ptr) if ptr else None
    return lib.kda_chunk_bwd(ctypes.byref(d), p, p, p, p, p, p, p, p, None, p, p, p, p, p, None, p, 1 << 40, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(H=3, HV=8), -1, "multiple of H"),
    (dict(K=64, V=64), -2, "unsupported"),
    (dict(C=32), -2, "unsupported"),
    (dict(dtype="f32"), -2, "unsupported"),
    (dict(T=-1), -1, "positive"),
    (dict(H=0), -1, "positive"),
    (dict(B=1 << 20, T=1 << 11, H=8, HV=256), -1, "too many chunk-heads"),
])
def test_validation_errors(lib, kw, status, msg):
    d, _ = _dims(**kw)
    assert _call_bwd(lib, d) == status
    assert msg in lib.kda_last_error().decode()
    assert kda.num_chunks(d) == -1 and kda.bwd_workspace_bytes(d) == 0


def test_beta_logits_flag_validated(lib):
    d, _ = _dims()
    d.beta_logits = 2
    assert _call_bwd(lib, d) == -1
    assert "beta_logits" in lib.kda_last_error().decode()
    d.beta_logits = 1
    assert kda.num_chunks(d) > 0


class _FakeDev:
    """Stands in for a device tensor: validation fails before the pointer is used."""

    def data_ptr(self):
        return 256


def test_varlen_validation(lib):
    d, keep = kda.make_dims(1, 100, 1, 1, 128, 128, 64, cu_seqlens=[0, 60, 100])
    assert _call_bwd(lib, d) == -1
    assert "both given or both NULL" in lib.kda_last_error().decode()
    d, keep = kda.make_dims(1, 100, 1, 1, 128, 128, 64, cu_seqlens=[0, 60, 50, 100], cu_seqlens_dev=_FakeDev())
    assert _call_bwd(lib, d) == -1
    assert "non-decreasing" in lib.kda_last_error().decode()
    d, keep = kda.make_dims(1, 100, 1, 1, 128, 128, 64, cu_seqlens=[0, 60, 90], cu_seqlens_dev=_FakeDev())
    assert _call_bwd(lib, d) == -1
    assert "must equal T" in lib.kda_last_error().decode()
    d, keep = kda.make_dims(2, 100, 1, 1, 128, 128, 64, cu_seqlens=[0, 60, 100], cu_seqlens_dev=_FakeDev())
    assert _call_bwd(lib, d) == -1
    assert "B = 1" in lib.kda_last_error().decode()


def test_null_pointers_and_small_workspace(lib):
    d, _ = _dims()
    assert lib.kda_chunk_bwd(ctypes.byref(d), *([None] * 15), None, 0, None) == -1
    assert "is NULL" in lib.kda_last_error().decode()
    p = ctypes.c_void_p(256)
    assert lib.kda_chunk_bwd(ctypes.byref(d), p, p, p, p, p, p, p, p, None, p, p, p, p, p, None, p, 1024, None) == -1
    assert "workspace too small" in lib.kda_last_error().decode()
    assert lib.kda_fwd_states(ctypes.byref(d), None, p, p, p, p, None, p, p, None, p, p, 1 << 40, None) == -1
    assert "q (needed for o)" in lib.kda_last_error().decode()


def test_saved_mode_validation(lib):
    """The saved-operand entry points check their extra buffer (and the save's need for q and
    o) before any HIP call."""
    d, _ = _dims()
    need = kda.saved_bytes(d)
    # kr, -w^T, Q'^T in bf16 and e^gam in fp32 per chunk-head, 64 chunks x 8 heads
    assert need >= 64 * 8 * (3 * 64 * 128 * 2 + 128 * 4)
    p = ctypes.c_void_p(256)
    big = 1 << 40
    args = [p] * 7  # q, k, v, g, beta, states, inv
    outs = [p, None, p, p, p, p, p, None]  # dO, dS_final, dq, dk, dv, dg, dbeta, dh0
    assert lib.kda_chunk_bwd_saved(ctypes.byref(d), *args, None, need, *outs, p, big, None) == -1
    assert "saved is NULL" in lib.kda_last_error().decode()
    assert lib.kda_chunk_bwd_saved(ctypes.byref(d), *args, p, need - 1, *outs, p, big, None) == -1
    assert "saved buffer too small" in lib.kda_last_error().decode()
    assert lib.kda_chunk_bwd_saved(ctypes.byref(d), *args, ctypes.c_void_p(257), need, *outs, p, big, None) == -1
    assert "256-byte aligned" in lib.kda_last_error().decode()
    # forward: q and o required, then the buffer
    fargs = [p, p, p, p, None, p, p, None]  # k, v, g, beta, h0, states, inv, final_state
    assert lib.kda_fwd_states_save(ctypes.byref(d), p, *fargs, None, p, need, p, big, None) == -1
    assert "o (the save" in lib.kda_last_error().decode()
    assert lib.kda_fwd_states_save(ctypes.byref(d), None, *fargs, p, p, need, p, big, None) == -1
    assert "q" in lib.kda_last_error().decode()
    assert lib.kda_fwd_states_save(ctypes.byref(d), p, *fargs, p, p, 16, p, big, None) == -1
    assert "saved buffer too small" in lib.kda_last_error().decode()
    bad, _ = _dims(C=32)
    assert kda.saved_bytes(bad) == 0


def test_workload_table_is_consistent():
    for wid, w in kin.WORKLOADS.items():
        if w.varlen:
            assert w.total > 0
        else:
            assert w.B > 0 and w.T > 0
        assert w.HV % w.H == 0


def test_entry_points_reject_host_tensors():
    """The product path has no CPU fallback: host tensors are refused before any launch."""
    import torch
    from chunked_gated_delta_09_amd.autograd import kda_chunk
    q = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16)
    v = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16)
    g = torch.zeros(1, 64, 1, 128)
    beta = torch.zeros(1, 64, 1)
    with pytest.raises(ValueError, match="GPU tensor"):
        kda.fwd_states(q, q, v, g, beta)
    with pytest.raises(ValueError, match="GPU tensor"):
        kda_chunk(q, q, v, g, beta)
