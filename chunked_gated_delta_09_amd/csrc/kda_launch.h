// Host-side launchers of the KDA kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

// Problem geometry shared by every kernel.
struct Shape {
  int T;                 // tokens per sequence (dense) or total tokens (packed)
  int H, HV;             // q/k heads, value heads
  int N;                 // sequences
  int NT;                // total chunks
  float scale;
  const int32_t* cu;     // device cu_seqlens, or nullptr when dense
  const int32_t* choff;  // device first-chunk table [N+1], or nullptr when dense
  int hv0, nhv;          // value heads of this launch: hv0 .. hv0 + nhv - 1 (a multiple of HV / H)
  int beta_logits;       // beta holds logits: kernels apply a sigmoid; dbeta is w.r.t. the logits
};

// Per-chunk workspace tensors of the forward (all [NT, HV, ...]).
struct FwdWs {
  void* negw;  // [C][K]   -w, w = INV diag(beta) (k e^G)
  void* krT;   // [K][C]   (k e^(gam-G))^T
  void* uT;    // [V][C]   u^T, u = INV diag(beta) v
  float* eg;   // [K]      e^gam
};

// Per-chunk tensors the forward can save for the backward (all [NT, HV, ...]; bf16 path in the
// reverse scan's fragment order, ScanFrag): what the backward's prep kernel would otherwise
// recompute from q, k, g, beta and INV.
struct SavedWs {
  void* kr;    // [C][K]   k e^(gam-G)
  void* nwT;   // [K][C]   -w^T
  void* qpT;   // [K][C]   Q'^T, Q' = qd - Mqk w
  float* eg;   // [K]      e^gam
};

// Per-chunk workspace tensors of the backward (all [NT, HV, ...]).
struct BwdWs {
  void* kr;    // [C][K]   k e^(gam-G)
  void* nwT;   // [K][C]   -w^T
  void* bcT;   // [V][K]   W = Q'^T dO, transposed (Q' = qd - Mqk w); or, where the scan forms W
               //          itself (scan_wq), Q'^T [K][C] in the scan's fragment order (a
               //          chunk-head every ScanFrag::P2_ELEMS elements)
  float* eg;   // [K]      e^gam
  void* dS;    // [K][V]   gradient w.r.t. each chunk's S_out
  void* yT;    // (kr dS)^T: bf16 in the reverse scan's lane-major order (tile m of slice vt at
               //          ScanFrag::seed(vt, m, C/16, lane)), fp32 [V][C]
};

// Value slices (16 columns each) per workgroup of the bf16 scans: the fewest that keep the
// grid within about one workgroup per CU.
inline int scan_slices(const Shape& s, int V) {
  const int slices = s.N * s.nhv * (V / 16);
  int nc = 1;
  while (nc < V / 16 && slices / nc > 256) nc *= 2;
  return nc;
}
// The bf16 reverse scan forms W = Q'^T dO itself when a workgroup holds 4 or more slices (its
// step is then bound by operand reads, and W's bytes exceed those of Q'^T and dO); with fewer
// it reads W as precomputed seed tiles (its step is a dependency chain that extra products
// would lengthen).
inline bool scan_wq(int dtype, const Shape& s, int V) { return dtype != 0 && scan_slices(s, V) >= 4; }

// dtype: 0 = fp32 (K = V = C = 16), 1 = bf16 (K = V = 128, C in {16, 64}).
hipError_t launch_chunk_offsets(const int32_t* cu, int N, int C, int32_t* choff, hipStream_t st);
// sv: where to save the backward's chunk operands (nullptr: not saved).
hipError_t launch_fwd_prep(int dtype, int C, const Shape& s, const void* k, const void* v, const float* g,
                           const float* beta, void* inv, const FwdWs& ws, hipStream_t st,
                           const SavedWs* sv = nullptr);
hipError_t launch_fwd_out(int dtype, int C, const Shape& s, const void* q, const void* k, const void* v,
                          const float* g, const float* beta, const void* states, const void* inv, void* o,
                          hipStream_t st, const SavedWs* sv = nullptr);
hipError_t launch_scan_fwd(int dtype, int C, const Shape& s, const FwdWs& ws, const void* h0, void* states,
                           float* final_state, hipStream_t st);
hipError_t launch_bwd_prep(int dtype, int C, const Shape& s, const void* q, const void* k, const float* g,
                           const float* beta, const void* inv, const void* dO, const BwdWs& ws, hipStream_t st);
hipError_t launch_scan_bwd(int dtype, int C, const Shape& s, const BwdWs& ws, const void* dO, const void* dSf,
                           float* dh0, hipStream_t st);
// W = Q'^T dO from the saved Q'^T into ws.bcT, in the scan's seed order (the part of the
// backward prep kernel that needs dO).
hipError_t launch_bwd_w(int dtype, int C, const Shape& s, const void* dO, const SavedWs& sv, const BwdWs& ws,
                        hipStream_t st);
hipError_t launch_bwd_grad(int dtype, int C, const Shape& s, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const void* states, const void* inv, const void* dO,
                           const BwdWs& ws, void* dq, void* dk, void* dv, float* dg, float* dbeta, hipStream_t st);

hipError_t launch_dstates_out(int dtype, int C, const Shape& s, const BwdWs& ws, float* out, hipStream_t st);

// C-ABI helpers (kda_api.cpp): validation + workspace size of a kda_chunk_bwd call, and the
// thread-local error message behind kda_last_error.
kda_status bwd_plan(const kda_dims* dims, size_t* ws_bytes);
kda_status set_error(kda_status st, const char* msg);

}  // namespace kda
