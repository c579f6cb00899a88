// Sequential chunk scans of KDA for gfx950. The fp32 path (small K, V, C) reads its
// operands in plain row-major order; the bf16 path reads them in fragment order.
//
// Both directions are one affine step per chunk on a K x V fp32 matrix X:
//   Y    = Z + P1 X                 (C x V, contraction over K)
//   X'   = diag(e^gam) X + W + P2 Y (K x V, contraction over C)
// Forward (FLA chunk_gated_delta_rule_fwd_h; FlashKDA page, the state update
// S_new = S*exp(gT) + kr^T@U): X = S, P1 = -w, Z = u, P2 = kr^T, W = 0, so Y = U and
// X' = S_out. Backward (FLA chunk_gated_delta_rule_bwd_dhu; FlashKDA page steps 2-3):
// X = dS (gradient w.r.t. S_out), P1 = kr, Z = 0 so Y = kr dS, P2 = -w^T and
// W = (qd - Mqk w)^T dO, giving X' = dS_in = diag(e^gam) dS + qd^T dO - w^T (Mqk^T dO + kr dS).
//
// The columns of X evolve independently, so one wavefront owns a 16-column slice of one
// (sequence, head) and walks its chunks in order, keeping X in fp32 registers as MFMA
// accumulator tiles. The accumulator tiles of X and Y are fed back as B operands with
// the contraction index permuted (rows 16t + 4*grp + i of tile t map to lane group grp,
// slot i), and the A operands are loaded in the same permuted order, so neither X nor Y
// round-trips through LDS.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <class T, int K, int V, int C, bool FWD>
__global__ __launch_bounds__(64) void scan_kernel(Shape s, const T* __restrict__ P1, const T* __restrict__ P2,
                                                   const T* __restrict__ Zi, const T* __restrict__ Wi,
                                                   const float* __restrict__ eg, const T* __restrict__ X0,
                                                   T* __restrict__ Xout, T* __restrict__ Yout,
                                                   float* __restrict__ Xfin) {
  typedef Mma<T> M;
  constexpr int KT = K / 16, CT = C / 16;
  const int vt = blockIdx.x, h = s.hv0 + blockIdx.y, nseq = blockIdx.z;
  const int lane = threadIdx.x, n = lane & 15, grp = lane >> 4;
  const int vcol = 16 * vt + n;
  int c0, nc;
  seq_range(nseq, s.cu, s.choff, s.T, C, c0, nc);
  if (c0 + nc > s.NT) nc = max(0, s.NT - c0);

  f32x4 X[KT];
  if (X0 != nullptr) {
    const T* x0 = X0 + ((long)nseq * s.HV + h) * K * V;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) X[t][j] = to_f(x0[(16 * t + 4 * grp + j) * V + vcol]);
  } else {
#pragma unroll
    for (int t = 0; t < KT; ++t) X[t] = zero4();
  }

  for (int ii = 0; ii < nc; ++ii) {
    const int c = FWD ? c0 + ii : c0 + nc - 1 - ii;
    const long ch = (long)c * s.HV + h;
    // X entering this step: S_in (forward) or the gradient w.r.t. S_out (backward).
    T* xo = Xout + ch * K * V;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) xo[(16 * t + 4 * grp + j) * V + vcol] = from_f<T>(X[t][j]);

    // Y = Z + P1 X
    f32x4 Y[CT];
    if (Zi != nullptr) {
#pragma unroll
      for (int m = 0; m < CT; ++m) Y[m] = ld4f(Zi + ch * V * C + vcol * C + 16 * m + 4 * grp);
    } else {
#pragma unroll
      for (int m = 0; m < CT; ++m) Y[m] = zero4();
    }
    const T* p1 = P1 + ch * C * K;
    if constexpr (M::PER == 8) {
      static_assert(KT % 2 == 0, "bf16 scan pairs row tiles of X");
#pragma unroll
      for (int p = 0; p < KT / 2; ++p) {
        bf16x8 b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          b[i] = (bf16)X[2 * p][i];
          b[4 + i] = (bf16)X[2 * p + 1][i];
        }
#pragma unroll
        for (int m = 0; m < CT; ++m) {
          const T* row = p1 + (16 * m + n) * K + 32 * p + 4 * grp;
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 16);
          const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          Y[m] = M::mma(a, b, Y[m]);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int m = 0; m < CT; ++m)
            Y[m] = M::mma(to_f(p1[(16 * m + n) * K + 16 * t + 4 * grp + j]), X[t][j], Y[m]);
    }
    if (Yout != nullptr) {
#pragma unroll
      for (int m = 0; m < CT; ++m) st4(Yout + ch * V * C + vcol * C + 16 * m + 4 * grp, Y[m]);
    }

    // X' = W + P2 Y, then X = diag(e^gam) X + X'
    f32x4 Xn[KT];
    if (Wi != nullptr) {
#pragma unroll
      for (int t = 0; t < KT; ++t) Xn[t] = ld4f(Wi + ch * V * K + vcol * K + 16 * t + 4 * grp);
    } else {
#pragma unroll
      for (int t = 0; t < KT; ++t) Xn[t] = zero4();
    }
    const T* p2 = P2 + ch * K * C;
    if constexpr (M::PER == 8) {
#pragma unroll
      for (int q = 0; q < (CT + 1) / 2; ++q) {
        bf16x8 b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          b[i] = (bf16)Y[2 * q][i];
          b[4 + i] = 2 * q + 1 < CT ? (bf16)Y[2 * q + 1 < CT ? 2 * q + 1 : 0][i] : (bf16)0.0f;
        }
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          const T* row = p2 + (16 * t + n) * C + 32 * q + 4 * grp;
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row);
          bf16x4 hi = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
          if (2 * q + 1 < CT) hi = *reinterpret_cast<const bf16x4*>(row + 16);
          const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          Xn[t] = M::mma(a, b, Xn[t]);
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < CT; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int t = 0; t < KT; ++t)
            Xn[t] = M::mma(to_f(p2[(16 * t + n) * C + 16 * m + 4 * grp + j]), Y[m][j], Xn[t]);
    }
    const float* e = eg + ch * K;
#pragma unroll
    for (int t = 0; t < KT; ++t) X[t] = ld4f(e + 16 * t + 4 * grp) * X[t] + Xn[t];
  }

  if (Xfin != nullptr) {
    float* xf = Xfin + ((long)nseq * s.HV + h) * K * V;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) xf[(16 * t + 4 * grp + j) * V + vcol] = X[t][j];
  }
}


// bf16 path: the per-chunk operands are stored in fragment order (ScanFrag), so each wave
// load is a contiguous 1 KB block, and the next chunk's operands are loaded into registers
// while the current chunk is computed (the index is clamped, so the loads are
// unconditional and always in flight). A second wave keeps the operands TOUCH_AHEAD chunks
// further on moving into L2: one 4-byte load per 128-byte line, the lines shared by the
// column slices of a head split between their workgroups, each load delivered into a
// scratch word of LDS so that it holds no register and is never waited for. The two waves
// meet at one barrier per chunk, which keeps the touches a fixed distance ahead.
//
// Backward direction: a column slice covers the columns ScanCols::col(vt, n) (not 16
// consecutive ones), and the per-chunk dS leaves exactly as this wave holds it, 4 values
// per lane and row tile in seed order (one 8-byte store per row tile); the gradient kernel
// transposes it, and the column choice makes the transposed values of two slices one
// contiguous B fragment.
template <int K, int V, int C, bool FWD>
__global__ __launch_bounds__(128) void scan_bf16_kernel(Shape s, const bf16* __restrict__ P1,
                                                        const bf16* __restrict__ P2, const bf16* __restrict__ Zs,
                                                        const bf16* __restrict__ Ws, const float* __restrict__ eg,
                                                        const bf16* __restrict__ X0, bf16* __restrict__ Xout,
                                                        bf16* __restrict__ Yout, float* __restrict__ Xfin) {
  typedef ScanFrag<K, V, C> F;
  typedef Mma<bf16> M;
  constexpr int KT = F::KT, CT = F::CT, KP = F::KP, CQ = F::CQ, VT = V / 16;
  static_assert(KT % 2 == 0, "the bf16 scan pairs row tiles of X");
  // Workgroups are dealt round-robin to the 8 XCDs by linear id, so ids i, i+8, i+16, ...
  // share an XCD (and its L2). All VT column slices of one (sequence, head) get ids of one
  // residue class mod 8: the slices' shared per-chunk operands are then fetched from HBM
  // once per XCD and served from L2 to the others.
  const int wid = blockIdx.x;
  const int xcd = wid % 8, r = wid / 8;
  const int pair = (r / VT) * 8 + xcd;  // (sequence, head) index
  const int vt = r % VT;
  if (pair >= s.N * s.nhv) return;
  const int h = s.hv0 + pair % s.nhv, nseq = pair / s.nhv;
  const int lane = threadIdx.x & 63, n = lane & 15, grp = lane >> 4;
  const int vcol = FWD ? 16 * vt + n : ScanCols::col(vt, n);
  int c0, nc;
  seq_range(nseq, s.cu, s.choff, s.T, C, c0, nc);
  if (c0 + nc > s.NT) nc = max(0, s.NT - c0);
  constexpr int TOUCH_AHEAD = 4;

  if (threadIdx.x >= 64) {
    // prefetch wave: lanes 0..31 cover this slice's share of the lines of P1 and P2,
    // lanes 32..63 the lines of this slice's own seed tiles; a second load covers e^gam.
    constexpr int SHARED_LINES = (F::P1_ELEMS + F::P2_ELEMS) * 2 / 128;
    constexpr int SEED_LINES = (FWD ? C : K) * 16 * 2 / 128;
    static_assert(SHARED_LINES <= 32 * VT && SEED_LINES <= 32, "one touch covers at most 64 lines per wave");
    __shared__ int sink[64];
    const int tl = min(32 * vt + (lane & 31), SHARED_LINES - 1);
    const int tl2 = max(0, min(lane - 32, SEED_LINES - 1));
    auto touch = [&](int c) {
      const long ch = (long)c * s.HV + h;
      const bf16* a;
      if (lane < 32) {
        a = tl < F::P1_ELEMS / 64 ? P1 + ch * F::P1_ELEMS + 64 * tl : P2 + ch * F::P2_ELEMS + 64 * (tl - F::P1_ELEMS / 64);
      } else {
        a = (FWD ? Zs + ch * C * V + F::seed(vt, 0, CT, 0) : Ws + ch * K * V + F::seed(vt, 0, KT, 0)) + 64 * tl2;
      }
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)a,
                                       (__attribute__((address_space(3))) void*)sink, 4, 0, 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(eg + ch * K + 32 * (lane % ((K + 31) / 32))),
                                       (__attribute__((address_space(3))) void*)sink, 4, 0, 0);
    };
    for (int d = 1; d < TOUCH_AHEAD && d < nc; ++d) touch(FWD ? c0 + d : c0 + nc - 1 - d);
    for (int ii = 0; ii < nc; ++ii) {
      __builtin_amdgcn_s_barrier();
      if (ii + TOUCH_AHEAD < nc) touch(FWD ? c0 + ii + TOUCH_AHEAD : c0 + nc - 1 - ii - TOUCH_AHEAD);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }

  struct Ops {  // double-buffered: the next chunk's are loaded during the current step
    bf16x8 a1[CT][KP];
    bf16x8 a2[KT][CQ];
  };
  struct Small {  // loaded at the start of their own step, ahead of the next chunk's Ops
    bf16x4 w[KT];
    bf16x4 z[CT];
    f32x4 e[KT];
  };
  auto load = [&](int c, Ops& o) {
    const long ch = (long)c * s.HV + h;
    const bf16x8* p1 = reinterpret_cast<const bf16x8*>(P1 + ch * F::P1_ELEMS) + lane;
#pragma unroll
    for (int m = 0; m < CT; ++m)
#pragma unroll
      for (int p = 0; p < KP; ++p) o.a1[m][p] = p1[(m * KP + p) * 64];
    const bf16x8* p2 = reinterpret_cast<const bf16x8*>(P2 + ch * F::P2_ELEMS) + lane;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int q = 0; q < CQ; ++q) o.a2[t][q] = p2[(t * CQ + q) * 64];
  };
  auto load_small = [&](int c, Small& o) {
    const long ch = (long)c * s.HV + h;
    if constexpr (!FWD) {
#pragma unroll
      for (int t = 0; t < KT; ++t) o.w[t] = *reinterpret_cast<const bf16x4*>(Ws + ch * K * V + F::seed(vt, t, KT, lane));
    }
    if constexpr (FWD) {
#pragma unroll
      for (int m = 0; m < CT; ++m) o.z[m] = *reinterpret_cast<const bf16x4*>(Zs + ch * C * V + F::seed(vt, m, CT, lane));
    }
#pragma unroll
    for (int t = 0; t < KT; ++t) o.e[t] = *reinterpret_cast<const f32x4*>(eg + ch * K + 16 * t + 4 * grp);
  };

  f32x4 X[KT];
  if (X0 != nullptr) {
    const bf16* x0 = X0 + ((long)nseq * s.HV + h) * K * V;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) X[t][j] = (float)x0[(16 * t + 4 * grp + j) * V + vcol];
  } else {
#pragma unroll
    for (int t = 0; t < KT; ++t) X[t] = zero4();
  }

  // One chunk step with operands `cur`; the loads of the next chunk into `nxt` are issued
  // first. The loop below alternates two buffers, so no register copy ever waits on a load
  // still in flight.
  auto step = [&](int ii, const Ops& cur, Ops& nxt) {
    __builtin_amdgcn_s_barrier();
    if (!FWD && ii < 63) KDA_TS(1, ii);
    const int c = FWD ? c0 + ii : c0 + nc - 1 - ii;
    Small sm;
    load_small(c, sm);
    {
      const int in = min(ii + 1, nc - 1);
      load(FWD ? c0 + in : c0 + nc - 1 - in, nxt);
    }
    const long ch = (long)c * s.HV + h;

    bf16x8 bx[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bx[p][i] = (bf16)X[2 * p][i];
        bx[p][4 + i] = (bf16)X[2 * p + 1][i];
      }
    if constexpr (FWD) {
      bf16* xo = Xout + ch * K * V;
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) xo[(16 * t + 4 * grp + j) * V + vcol] = bx[t / 2][4 * (t % 2) + j];
    } else {
      bf16* xo = Xout + ch * K * V;
#pragma unroll
      for (int t = 0; t < KT; ++t)
        *reinterpret_cast<bf16x4*>(xo + F::seed(vt, t, KT, lane)) =
            bf16x4{bx[t / 2][4 * (t % 2)], bx[t / 2][4 * (t % 2) + 1], bx[t / 2][4 * (t % 2) + 2], bx[t / 2][4 * (t % 2) + 3]};
    }

    // Y = Z + P1 X
    f32x4 Y[CT];
#pragma unroll
    for (int m = 0; m < CT; ++m) {
      if constexpr (FWD) {
        Y[m] = f32x4{(float)sm.z[m][0], (float)sm.z[m][1], (float)sm.z[m][2], (float)sm.z[m][3]};
      } else {
        Y[m] = zero4();
      }
    }
#pragma unroll
    for (int p = 0; p < KP; ++p)
#pragma unroll
      for (int m = 0; m < CT; ++m) Y[m] = M::mma(cur.a1[m][p], bx[p], Y[m]);
    if constexpr (!FWD) {
#pragma unroll
      for (int m = 0; m < CT; ++m) st4(Yout + ch * V * C + vcol * C + 16 * m + 4 * grp, Y[m]);
    }

    // X' = W + P2 Y;  X = diag(e^gam) X + X'
    f32x4 Xn[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      if constexpr (!FWD) {
        Xn[t] = f32x4{(float)sm.w[t][0], (float)sm.w[t][1], (float)sm.w[t][2], (float)sm.w[t][3]};
      } else {
        Xn[t] = zero4();
      }
    }
#pragma unroll
    for (int q = 0; q < CQ; ++q) {
      const bool pair = 2 * q + 1 < CT;
      bf16x8 b;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[i] = (bf16)Y[2 * q][i];
        b[4 + i] = pair ? (bf16)Y[pair ? 2 * q + 1 : 2 * q][i] : (bf16)0.0f;
      }
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        bf16x8 a = cur.a2[t][q];
        if (!pair) {
#pragma unroll
          for (int i = 4; i < 8; ++i) a[i] = (bf16)0.0f;
        }
        Xn[t] = M::mma(a, b, Xn[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < KT; ++t) X[t] = sm.e[t] * X[t] + Xn[t];
    // Issue order: this step's small loads first, then one load of the next chunk's
    // fragments after each MFMA, so that the address unit works while the matrix pipe does
    // (issued as one burst, the loads would hold up the MFMAs behind them).
    constexpr int NSMALL = KT + (FWD ? CT : KT), NMMA = CT * KP + KT * CQ;
    static_assert(NMMA == CT * KP + KT * CQ, "one next-chunk load per MFMA");
    __builtin_amdgcn_sched_group_barrier(0x020, NSMALL, 0);
#pragma unroll
    for (int i = 0; i < NMMA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
  };

  if (nc > 0) {
    Ops ping, pong;
    load(FWD ? c0 : c0 + nc - 1, ping);
    for (int ii = 0; ii < nc; ii += 2) {
      step(ii, ping, pong);
      if (ii + 1 < nc) step(ii + 1, pong, ping);
    }
  }

  if (Xfin != nullptr) {
    float* xf = Xfin + ((long)nseq * s.HV + h) * K * V;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) xf[(16 * t + 4 * grp + j) * V + vcol] = X[t][j];
  }
}

template <class T, int K, int V, int C, bool FWD>
static hipError_t scan_t(const Shape& s, const void* P1, const void* P2, const void* Zi, const void* Wi,
                         const float* eg, const void* X0, void* Xout, void* Yout, float* Xfin, hipStream_t st) {
  if (s.N == 0) return hipSuccess;
  if constexpr (sizeof(T) == 2) {
    const int pairs = s.N * s.nhv;
    const int grid = ((pairs + 7) / 8) * 8 * (V / 16);
    hipLaunchKernelGGL((scan_bf16_kernel<K, V, C, FWD>), dim3(grid), dim3(128), 0, st, s,
                       static_cast<const bf16*>(P1), static_cast<const bf16*>(P2), static_cast<const bf16*>(Zi),
                       static_cast<const bf16*>(Wi), eg, static_cast<const bf16*>(X0), static_cast<bf16*>(Xout),
                       static_cast<bf16*>(Yout), Xfin);
  } else {
    hipLaunchKernelGGL((scan_kernel<T, K, V, C, FWD>), dim3(V / 16, s.nhv, s.N), dim3(64), 0, st, s,
                       static_cast<const T*>(P1), static_cast<const T*>(P2), static_cast<const T*>(Zi),
                       static_cast<const T*>(Wi), eg, static_cast<const T*>(X0), static_cast<T*>(Xout),
                       static_cast<T*>(Yout), Xfin);
  }
  return hipGetLastError();
}

hipError_t launch_scan_fwd(int dtype, int C, const Shape& s, const FwdWs& ws, const void* h0, void* states,
                           float* final_state, hipStream_t st) {
  if (dtype == 0)
    return scan_t<float, 16, 16, 16, true>(s, ws.negw, ws.krT, ws.uT, nullptr, ws.eg, h0, states, nullptr,
                                           final_state, st);
  if (C == 64)
    return scan_t<bf16, 128, 128, 64, true>(s, ws.negw, ws.krT, ws.uT, nullptr, ws.eg, h0, states, nullptr,
                                            final_state, st);
  return scan_t<bf16, 128, 128, 16, true>(s, ws.negw, ws.krT, ws.uT, nullptr, ws.eg, h0, states, nullptr,
                                          final_state, st);
}

hipError_t launch_scan_bwd(int dtype, int C, const Shape& s, const BwdWs& ws, const void* dSf, float* dh0,
                           hipStream_t st) {
  if (dtype == 0)
    return scan_t<float, 16, 16, 16, false>(s, ws.kr, ws.nwT, nullptr, ws.bcT, ws.eg, dSf, ws.dS, ws.yT, dh0, st);
  if (C == 64)
    return scan_t<bf16, 128, 128, 64, false>(s, ws.kr, ws.nwT, nullptr, ws.bcT, ws.eg, dSf, ws.dS, ws.yT, dh0,
                                             st);
  return scan_t<bf16, 128, 128, 16, false>(s, ws.kr, ws.nwT, nullptr, ws.bcT, ws.eg, dSf, ws.dS, ws.yT, dh0, st);
}

}  // namespace kda
