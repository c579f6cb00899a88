// C ABI of the KDA chunk library: argument validation (before any HIP call), the chunk
// table, workspace layout and the launch sequence of each entry point.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "kda.h"
#include "kda_measure.h"
#include "kda_launch.h"

#define KDA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_err;
thread_local void* const* g_events = nullptr;
thread_local int g_nevents = 0;

// Records the measurement events around the i-th launch of a call (kda_measure.h).
struct LaunchCounter {
  hipStream_t st;
  int i = 0;
  explicit LaunchCounter(hipStream_t s) : st(s) {}
  void before() {
    if (g_events != nullptr && 2 * i + 1 < g_nevents) (void)hipEventRecord(static_cast<hipEvent_t>(g_events[2 * i]), st);
  }
  void after() {
    if (g_events != nullptr && 2 * i + 1 < g_nevents)
      (void)hipEventRecord(static_cast<hipEvent_t>(g_events[2 * i + 1]), st);
    ++i;
  }
};

kda_status fail(kda_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int dtype = 0, K = 0, V = 0, C = 0;
  size_t es = 0;      // element size of the dims dtype
  int64_t NT = 0;     // total chunks
  bool varlen = false;
};

kda_status validate(const kda_dims* d, Plan& p, bool launching) {
  if (d == nullptr) return fail(KDA_EINVAL, "dims is NULL");
  if (d->B <= 0 || d->H <= 0 || d->HV <= 0 || d->K <= 0 || d->V <= 0 || d->C <= 0 || d->N <= 0 || d->T < 0)
    return fail(KDA_EINVAL, "dims must be positive (B=%d T=%d H=%d HV=%d K=%d V=%d C=%d N=%d)", d->B, d->T, d->H,
                d->HV, d->K, d->V, d->C, d->N);
  if (d->HV % d->H != 0) return fail(KDA_EINVAL, "HV (%d) must be a multiple of H (%d)", d->HV, d->H);
  if (d->dtype != KDA_F32 && d->dtype != KDA_BF16) return fail(KDA_EINVAL, "unknown dtype %d", d->dtype);
  if (d->beta_logits != 0 && d->beta_logits != 1) return fail(KDA_EINVAL, "beta_logits must be 0 or 1, got %d", d->beta_logits);
  if (!std::isfinite(d->scale)) return fail(KDA_EINVAL, "scale must be finite");
  const bool ok = (d->dtype == KDA_F32 && d->K == 16 && d->V == 16 && d->C == 16) ||
                  (d->dtype == KDA_BF16 && d->K == 128 && d->V == 128 && (d->C == 64 || d->C == 16));
  if (!ok)
    return fail(KDA_EUNSUPPORTED,
                "unsupported (dtype=%s, K=%d, V=%d, C=%d); supported: (f32,16,16,16), (bf16,128,128,64), "
                "(bf16,128,128,16)",
                d->dtype == KDA_F32 ? "f32" : "bf16", d->K, d->V, d->C);
  // Size queries read only the host copy; launches need both copies.
  if (launching && (d->cu_seqlens_dev == nullptr) != (d->cu_seqlens_host == nullptr))
    return fail(KDA_EINVAL, "cu_seqlens_dev and cu_seqlens_host must be both given or both NULL");
  p.dtype = d->dtype;
  p.K = d->K;
  p.V = d->V;
  p.C = d->C;
  p.es = d->dtype == KDA_F32 ? 4 : 2;
  p.varlen = d->cu_seqlens_host != nullptr;
  if (p.varlen) {
    if (d->B != 1) return fail(KDA_EINVAL, "packed sequences (cu_seqlens given) need B = 1, got %d", d->B);
    const int32_t* cu = d->cu_seqlens_host;
    if (cu[0] != 0) return fail(KDA_EINVAL, "cu_seqlens[0] must be 0, got %d", cu[0]);
    int64_t nt = 0;
    for (int n = 0; n < d->N; ++n) {
      if (cu[n + 1] < cu[n])
        return fail(KDA_EINVAL, "cu_seqlens must be non-decreasing (cu[%d]=%d > cu[%d]=%d)", n, cu[n], n + 1,
                    cu[n + 1]);
      nt += (cu[n + 1] - cu[n] + d->C - 1) / d->C;
    }
    if (cu[d->N] != d->T) return fail(KDA_EINVAL, "cu_seqlens[N] (%d) must equal T (%d)", cu[d->N], d->T);
    p.NT = nt;
  } else {
    if (d->N != d->B) return fail(KDA_EINVAL, "dense batches need N == B (N=%d, B=%d)", d->N, d->B);
    p.NT = (int64_t)d->B * ((d->T + d->C - 1) / d->C);
  }
  if (p.NT > (int64_t)1 << 30) return fail(KDA_EINVAL, "too many chunks (%lld)", (long long)p.NT);
  // the chunk kernels launch one workgroup per (chunk, head) on a one-dimensional grid,
  // rounded up to whole runs of 8 q/k groups
  if (p.NT * d->HV + 8 * (int64_t)(d->HV / d->H) > (int64_t)INT32_MAX)
    return fail(KDA_EINVAL, "too many chunk-heads (%lld chunks x %d value heads)", (long long)p.NT, d->HV);
  return KDA_OK;
}

// Workspace offsets (bytes, 256-aligned).
struct FwdLayout {
  size_t choff, negw, krT, uT, eg, total;
};
struct BwdLayout {
  size_t choff, kr, nwT, bcT, eg, dS, yT, total;
};
// The forward's save for the backward (kda_fwd_states_save / kda_chunk_bwd_saved).
struct SavedLayout {
  size_t kr, nwT, qpT, eg, total;
};

// Elements per chunk-head of the scan's K x C operand: the bf16 path stores it in
// fragment order, padded to whole 32-wide contraction steps.
size_t p2_elems(const Plan& p) {
  if (p.dtype == KDA_BF16) return (size_t)(p.K / 16) * ((p.C / 16 + 1) / 2) * 64 * 8;
  return (size_t)p.K * p.C;
}

FwdLayout fwd_layout(const kda_dims* d, const Plan& p) {
  FwdLayout L;
  const size_t nth = (size_t)p.NT * d->HV;
  size_t o = 0;
  L.choff = o; o = align_up(o + sizeof(int32_t) * (d->N + 1));
  L.negw = o; o = align_up(o + nth * p.C * p.K * p.es);
  L.krT = o; o = align_up(o + nth * p2_elems(p) * p.es);
  L.uT = o; o = align_up(o + nth * p.V * p.C * p.es);
  L.eg = o; o = align_up(o + nth * p.K * sizeof(float));
  L.total = o;
  return L;
}

BwdLayout bwd_layout(const kda_dims* d, const Plan& p) {
  BwdLayout L;
  const size_t nth = (size_t)p.NT * d->HV;
  size_t o = 0;
  L.choff = o; o = align_up(o + sizeof(int32_t) * (d->N + 1));
  L.kr = o; o = align_up(o + nth * p.C * p.K * p.es);
  L.nwT = o; o = align_up(o + nth * p2_elems(p) * p.es);
  L.bcT = o; o = align_up(o + nth * p.V * p.K * p.es);
  L.eg = o; o = align_up(o + nth * p.K * sizeof(float));
  L.dS = o; o = align_up(o + nth * p.K * p.V * p.es);
  L.yT = o; o = align_up(o + nth * p.V * p.C * p.es);
  L.total = o;
  return L;
}

SavedLayout saved_layout(const kda_dims* d, const Plan& p) {
  SavedLayout L;
  const size_t nth = (size_t)p.NT * d->HV;
  size_t o = 0;
  L.kr = o; o = align_up(o + nth * p.C * p.K * p.es);
  L.nwT = o; o = align_up(o + nth * p2_elems(p) * p.es);
  L.qpT = o; o = align_up(o + nth * p2_elems(p) * p.es);
  L.eg = o; o = align_up(o + nth * p.K * sizeof(float));
  L.total = o;
  return L;
}

kda::SavedWs saved_ws(void* saved, const SavedLayout& L) {
  char* b = static_cast<char*>(saved);
  kda::SavedWs sv;
  sv.kr = b + L.kr;
  sv.nwT = b + L.nwT;
  sv.qpT = b + L.qpT;
  sv.eg = reinterpret_cast<float*>(b + L.eg);
  return sv;
}

kda_status check_saved(const void* saved, size_t bytes, size_t need) {
  if (saved == nullptr && need > 0) return fail(KDA_EINVAL, "saved is NULL (%zu bytes needed)", need);
  if (bytes < need) return fail(KDA_EINVAL, "saved buffer too small: %zu bytes given, %zu needed", bytes, need);
  if (reinterpret_cast<uintptr_t>(saved) % kAlign != 0) return fail(KDA_EINVAL, "saved must be 256-byte aligned");
  return KDA_OK;
}

kda::Shape make_shape(const kda_dims* d, const Plan& p, void* ws, size_t choff_off) {
  kda::Shape s;
  s.T = d->T;
  s.H = d->H;
  s.HV = d->HV;
  s.N = d->N;
  s.NT = (int)p.NT;
  s.scale = d->scale;
  s.cu = p.varlen ? d->cu_seqlens_dev : nullptr;
  s.choff = p.varlen ? reinterpret_cast<const int32_t*>(static_cast<char*>(ws) + choff_off) : nullptr;
  s.hv0 = 0;
  s.nhv = d->HV;
  s.beta_logits = d->beta_logits;
  return s;
}

kda_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (ws == nullptr && need > 0) return fail(KDA_EINVAL, "workspace is NULL (%zu bytes needed)", need);
  if (ws_bytes < need) return fail(KDA_EINVAL, "workspace too small: %zu bytes given, %zu needed", ws_bytes, need);
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return fail(KDA_EINVAL, "workspace must be 256-byte aligned");
  return KDA_OK;
}

#define KDA_REQUIRE(ptr, name) \
  if ((ptr) == nullptr) return fail(KDA_EINVAL, "%s is NULL", name)

#define KDA_HIP(call)                                                                  \
  do {                                                                                 \
    lc.before();                                                                       \
    const hipError_t e_ = (call);                                                      \
    lc.after();                                                                        \
    if (e_ != hipSuccess) return fail(KDA_EHIP, "%s: %s", #call, hipGetErrorString(e_)); \
  } while (0)

}  // namespace

namespace kda {

// Validation and workspace size of a kda_chunk_bwd call, for entry points that supply the
// workspace themselves (the message of a failed check is left for kda_last_error).
kda_status bwd_plan(const kda_dims* dims, size_t* ws_bytes) {
  Plan p;
  const kda_status st = validate(dims, p, true);
  if (st != KDA_OK) return st;
  *ws_bytes = bwd_layout(dims, p).total;
  return KDA_OK;
}

kda_status set_error(kda_status st, const char* msg) { return fail(st, "%s", msg); }

}  // namespace kda

KDA_EXPORT int64_t kda_num_chunks(const kda_dims* dims) {
  Plan p;
  if (validate(dims, p, false) != KDA_OK) return -1;
  return p.NT;
}

KDA_EXPORT size_t kda_fwd_workspace_bytes(const kda_dims* dims) {
  Plan p;
  if (validate(dims, p, false) != KDA_OK) return 0;
  return fwd_layout(dims, p).total;
}

KDA_EXPORT size_t kda_bwd_workspace_bytes(const kda_dims* dims) {
  Plan p;
  if (validate(dims, p, false) != KDA_OK) return 0;
  return bwd_layout(dims, p).total;
}

KDA_EXPORT size_t kda_saved_bytes(const kda_dims* dims) {
  Plan p;
  if (validate(dims, p, false) != KDA_OK) return 0;
  return saved_layout(dims, p).total;
}

KDA_EXPORT const char* kda_last_error(void) { return g_err.c_str(); }

KDA_EXPORT void kda_set_kernel_events(void* const* events, int count) {
  g_events = count > 0 ? events : nullptr;
  g_nevents = count > 0 ? count : 0;
}

namespace {

kda_status fwd_impl(const kda_dims* dims, const void* q, const void* k, const void* v, const float* g,
                    const float* beta, const void* h0, void* states, void* inv, float* final_state, void* o,
                    void* saved, size_t saved_bytes, bool save, void* workspace, size_t ws_bytes, void* stream) {
  Plan p;
  kda_status st = validate(dims, p, true);
  if (st != KDA_OK) return st;
  if (p.NT > 0) {
    KDA_REQUIRE(k, "k");
    KDA_REQUIRE(v, "v");
    KDA_REQUIRE(g, "g");
    KDA_REQUIRE(beta, "beta");
    KDA_REQUIRE(states, "states");
    KDA_REQUIRE(inv, "inv");
    if (o != nullptr) KDA_REQUIRE(q, "q (needed for o)");
    if (save) {
      KDA_REQUIRE(q, "q");
      KDA_REQUIRE(o, "o (the save is written by the output kernel)");
    }
  }
  const FwdLayout L = fwd_layout(dims, p);
  st = check_ws(workspace, ws_bytes, L.total);
  if (st != KDA_OK) return st;
  const SavedLayout SL = saved_layout(dims, p);
  if (save) {
    st = check_saved(saved, saved_bytes, SL.total);
    if (st != KDA_OK) return st;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  LaunchCounter lc(hs);
  char* ws = static_cast<char*>(workspace);
  const kda::Shape s = make_shape(dims, p, workspace, L.choff);
  kda::FwdWs fw;
  fw.negw = ws + L.negw;
  fw.krT = ws + L.krT;
  fw.uT = ws + L.uT;
  fw.eg = reinterpret_cast<float*>(ws + L.eg);
  kda::SavedWs sv{};
  if (save) sv = saved_ws(saved, SL);
  const kda::SavedWs* svp = save ? &sv : nullptr;
  if (p.varlen) KDA_HIP(kda::launch_chunk_offsets(dims->cu_seqlens_dev, dims->N, p.C, reinterpret_cast<int32_t*>(ws + L.choff), hs));
  KDA_HIP(kda::launch_fwd_prep(p.dtype, p.C, s, k, v, g, beta, inv, fw, hs, svp));
  KDA_HIP(kda::launch_scan_fwd(p.dtype, p.C, s, fw, h0, states, final_state, hs));
  if (o != nullptr) KDA_HIP(kda::launch_fwd_out(p.dtype, p.C, s, q, k, v, g, beta, states, inv, o, hs, svp));
  return KDA_OK;
}

}  // namespace

KDA_EXPORT kda_status kda_fwd_states(const kda_dims* dims, const void* q, const void* k, const void* v,
                                     const float* g, const float* beta, const void* h0, void* states, void* inv,
                                     float* final_state, void* o, void* workspace, size_t ws_bytes, void* stream) {
  return fwd_impl(dims, q, k, v, g, beta, h0, states, inv, final_state, o, nullptr, 0, false, workspace, ws_bytes,
                  stream);
}

KDA_EXPORT kda_status kda_fwd_states_save(const kda_dims* dims, const void* q, const void* k, const void* v,
                                          const float* g, const float* beta, const void* h0, void* states, void* inv,
                                          float* final_state, void* o, void* saved, size_t saved_bytes,
                                          void* workspace, size_t ws_bytes, void* stream) {
  return fwd_impl(dims, q, k, v, g, beta, h0, states, inv, final_state, o, saved, saved_bytes, true, workspace,
                  ws_bytes, stream);
}

namespace {

kda_status bwd_impl(const kda_dims* dims, const void* q, const void* k, const void* v, const float* g,
                    const float* beta, const void* states, const void* inv, const void* saved, size_t saved_bytes,
                    bool use_saved, const void* dO, const void* dS_final, void* dq, void* dk, void* dv, float* dg,
                    float* dbeta, float* dh0, void* workspace, size_t ws_bytes, void* stream) {
  Plan p;
  kda_status st = validate(dims, p, true);
  if (st != KDA_OK) return st;
  if (p.NT > 0) {
    KDA_REQUIRE(q, "q");
    KDA_REQUIRE(k, "k");
    KDA_REQUIRE(v, "v");
    KDA_REQUIRE(g, "g");
    KDA_REQUIRE(beta, "beta");
    KDA_REQUIRE(states, "states");
    KDA_REQUIRE(inv, "inv");
    KDA_REQUIRE(dO, "dO");
    KDA_REQUIRE(dq, "dq");
    KDA_REQUIRE(dk, "dk");
    KDA_REQUIRE(dv, "dv");
    KDA_REQUIRE(dg, "dg");
    KDA_REQUIRE(dbeta, "dbeta");
  }
  const BwdLayout L = bwd_layout(dims, p);
  st = check_ws(workspace, ws_bytes, L.total);
  if (st != KDA_OK) return st;
  const SavedLayout SL = saved_layout(dims, p);
  if (use_saved) {
    st = check_saved(saved, saved_bytes, SL.total);
    if (st != KDA_OK) return st;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  LaunchCounter lc(hs);
  char* ws = static_cast<char*>(workspace);
  const kda::Shape s = make_shape(dims, p, workspace, L.choff);
  kda::BwdWs bw;
  bw.kr = ws + L.kr;
  bw.nwT = ws + L.nwT;
  bw.bcT = ws + L.bcT;
  bw.eg = reinterpret_cast<float*>(ws + L.eg);
  bw.dS = ws + L.dS;
  bw.yT = ws + L.yT;
  if (p.varlen) KDA_HIP(kda::launch_chunk_offsets(dims->cu_seqlens_dev, dims->N, p.C, reinterpret_cast<int32_t*>(ws + L.choff), hs));
  if (use_saved) {
    // the scan reads the forward's kr, -w^T and e^gam; W comes from the saved Q'^T, formed
    // by the scan itself or by a small kernel into the workspace
    const kda::SavedWs sv = saved_ws(const_cast<void*>(saved), SL);
    bw.kr = sv.kr;
    bw.nwT = sv.nwT;
    bw.eg = sv.eg;
    if (kda::scan_wq(p.dtype, s, p.V)) {
      bw.bcT = sv.qpT;
    } else {
      KDA_HIP(kda::launch_bwd_w(p.dtype, p.C, s, dO, sv, bw, hs));
    }
  } else {
    KDA_HIP(kda::launch_bwd_prep(p.dtype, p.C, s, q, k, g, beta, inv, dO, bw, hs));
  }
  KDA_HIP(kda::launch_scan_bwd(p.dtype, p.C, s, bw, dO, dS_final, dh0, hs));
  KDA_HIP(kda::launch_bwd_grad(p.dtype, p.C, s, q, k, v, g, beta, states, inv, dO, bw, dq, dk, dv, dg, dbeta, hs));
  return KDA_OK;
}

}  // namespace

KDA_EXPORT kda_status kda_chunk_bwd(const kda_dims* dims, const void* q, const void* k, const void* v,
                                    const float* g, const float* beta, const void* states, const void* inv,
                                    const void* dO, const void* dS_final, void* dq, void* dk, void* dv, float* dg,
                                    float* dbeta, float* dh0, void* workspace, size_t ws_bytes, void* stream) {
  return bwd_impl(dims, q, k, v, g, beta, states, inv, nullptr, 0, false, dO, dS_final, dq, dk, dv, dg, dbeta, dh0,
                  workspace, ws_bytes, stream);
}

KDA_EXPORT kda_status kda_chunk_bwd_saved(const kda_dims* dims, const void* q, const void* k, const void* v,
                                          const float* g, const float* beta, const void* states, const void* inv,
                                          const void* saved, size_t saved_bytes, const void* dO,
                                          const void* dS_final, void* dq, void* dk, void* dv, float* dg,
                                          float* dbeta, float* dh0, void* workspace, size_t ws_bytes,
                                          void* stream) {
  return bwd_impl(dims, q, k, v, g, beta, states, inv, saved, saved_bytes, true, dO, dS_final, dq, dk, dv, dg, dbeta,
                  dh0, workspace, ws_bytes, stream);
}

KDA_EXPORT kda_status kda_bwd_state_grads(const kda_dims* dims, const void* workspace, size_t ws_bytes,
                                          float* dstates, void* stream) {
  Plan p;
  kda_status st = validate(dims, p, true);
  if (st != KDA_OK) return st;
  if (p.NT > 0) KDA_REQUIRE(dstates, "dstates");
  const BwdLayout L = bwd_layout(dims, p);
  st = check_ws(const_cast<void*>(workspace), ws_bytes, L.total);
  if (st != KDA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  LaunchCounter lc(hs);
  char* ws = static_cast<char*>(const_cast<void*>(workspace));
  const kda::Shape s = make_shape(dims, p, ws, L.choff);
  kda::BwdWs bw{};
  bw.dS = ws + L.dS;
  KDA_HIP(kda::launch_dstates_out(p.dtype, p.C, s, bw, dstates, hs));
  return KDA_OK;
}
