"""Host-side logic of bench.py (no GPU): the one-GPU guard and the roofline accounting."""
import importlib.util
import math
import os
import subprocess
import sys

from chunked_gated_delta_09_amd import inputs as kin

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def _per_token_head_bytes(K, V, C, es, group):
    """Bytes per token-head counted from the operation's inputs and outputs: q, k and their
    gradients are shared by the `group` value heads of a q/k head; g, dg are fp32 per channel;
    beta, dbeta fp32 per token; the chunk's state S_in (K x V) and inverse (C x C) are spread
    over its C tokens."""
    reads = (2 * K * es) / group + 2 * V * es + 4 * K + 4 + (K * V + C * C) * es / C
    writes = (2 * K * es) / group + V * es + 4 * K + 4
    return reads + writes


def test_algorithmic_bytes_match_the_per_token_head_count():
    bench = _bench()
    for wid in (1, 2, 4):
        w = kin.WORKLOADS[wid]
        inp = kin.make_inputs(w, wid=wid)
        th = inp["B"] * inp["T"] * w.HV
        per_seq = w.HV * w.K * w.V * (4 + (2 if inp["dS_final"] is not None else 0))  # dh0 fp32, dS_final bf16
        expect = th * _per_token_head_bytes(w.K, w.V, w.C, 2, w.HV // w.H) + inp["N"] * per_seq
        assert bench.algorithmic_bytes(w, inp) == round(expect), wid
    # the figure quoted for the bench workload (B=2, T=2048, H=8): 3,464 B per token-head
    w1 = kin.WORKLOADS[1]
    assert _per_token_head_bytes(w1.K, w1.V, w1.C, 2, 1) == 3464
    assert bench.algorithmic_bytes(w1, kin.make_inputs(w1, wid=1)) == 115_081_216


def test_algorithmic_flops_count():
    bench = _bench()
    w = kin.WORKLOADS[1]
    inp = kin.make_inputs(w, wid=1)
    # seven C x K x V products and ten triangular C x C x D products (C^2 D / 2 MACs each) per
    # chunk, 2 flop per MAC
    per_chunk = 2 * 7 * w.C * w.K * w.V + 10 * w.C * w.C * w.K
    chunks = inp["B"] * math.ceil(inp["T"] / w.C) * w.HV
    assert bench.algorithmic_flops(w, inp) == per_chunk * chunks


def test_recorded_traffic_follows_the_sources(tmp_path):
    bench = _bench()
    w = kin.WORKLOADS[1]
    t = bench.recorded_traffic(w.name)
    # either the record matches the current sources (a positive byte count) or it is withheld
    assert t is None or t > bench.algorithmic_bytes(w, kin.make_inputs(w, wid=1))
    assert bench.recorded_traffic("no_such_workload") is None
    # a record is used only with a line for every kernel of the call and the current sources
    sha = bench.sources_sha256()
    rec = tmp_path / "rec.md"
    lines = [f"bench-traffic: workload={w.name} kernel={k} bytes={b} sources-sha256={sha}"
             for k, b in zip(bench.BWD_KERNELS, (10, 20, 30))]
    rec.write_text("\n".join(lines[:2]) + "\n")
    assert bench.recorded_traffic(w.name, "call", record=str(rec)) is None
    assert bench.recorded_traffic(w.name, "bwd_scan", record=str(rec)) == 20
    rec.write_text("\n".join(lines) + "\n")
    assert bench.recorded_traffic(w.name, "call", record=str(rec)) == 60
    rec.write_text("\n".join(x.replace(sha, "0" * 64) for x in lines) + "\n")
    assert bench.recorded_traffic(w.name, "call", record=str(rec)) is None


def test_forward_algorithmic_bytes():
    """kda_fwd_states with o: reads q, k, v (bf16), g, beta (fp32), h0; writes the chunk states
    (K x V per chunk), inverses (C x C), o and the fp32 final state."""
    bench = _bench()
    w = kin.WORKLOADS[1]
    inp = kin.make_inputs(w, wid=1)
    th = inp["B"] * inp["T"] * w.HV
    per_th = 2 * w.K * 2 + w.V * 2 + 4 * w.K + 4 + (w.K * w.V + w.C * w.C) * 2 / w.C + w.V * 2
    per_seq = w.HV * w.K * w.V * (2 + 4)
    assert per_th == 2180
    assert bench.fwd_algorithmic_bytes(w, inp) == round(th * per_th + inp["N"] * per_seq)


def test_saved_read_bytes_is_the_librarys_save():
    """The saved-operand backward's extra algorithmic bytes are the save it reads: kr, -w^T and
    Q'^T (C x K bf16 each) and e^gam (K fp32) per chunk-head, 48.5 KB at K = 128, C = 64; the
    library's own size query for the same dims agrees (its sub-buffers are 256-byte aligned,
    which these sizes already are)."""
    import chunked_gated_delta_09_amd as kda
    bench = _bench()
    for wid in (1, 4):
        w = kin.WORKLOADS[wid]
        inp = kin.make_inputs(w, wid=wid)
        per_chunk_head = 3 * w.C * w.K * 2 + w.K * 4
        assert per_chunk_head == 49664
        assert bench.saved_read_bytes(w, inp) == bench.num_chunks(w, inp) * w.HV * per_chunk_head
        dims, keep = kda.make_dims(inp["B"], inp["T"], w.H, w.HV, w.K, w.V, w.C, inp["scale"], w.dtype,
                                   inp["cu_seqlens"])
        assert kda.saved_bytes(dims) == bench.saved_read_bytes(w, inp)
    assert bench.saved_read_bytes(kin.WORKLOADS[1], kin.make_inputs(kin.WORKLOADS[1], wid=1)) == 25427968


def test_scan_forms_w_follows_the_slice_rule():
    """The reverse scan forms W itself when a workgroup holds 4 or more of the 16-column value
    slices (the fewest slices per workgroup that keep the grid near 256 workgroups): 16 (sequence,
    head) pairs x 8 slices fit one per workgroup (workloads 1, 2), 256 pairs need 8 per workgroup
    (the packed workload 3), 128 need 4 (workload 4); never on the fp32 path."""
    bench = _bench()
    expect = {0: False, 1: False, 2: False, 3: True, 4: True}
    for wid, want in expect.items():
        w = kin.WORKLOADS[wid]
        assert bench.scan_forms_w(w, kin.make_inputs(w, wid=wid)) is want, wid
