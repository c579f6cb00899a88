// Backward chunk kernels of KDA for gfx950.
//
// Chunk algebra of the backward (FlashKDA backward page, steps 1-3 and the dMqk / dqd /
// dki / dkd / dbeta products; FLA chunk_kda_bwd page, kernels dAv and wy_dqkg_fused, the
// intra-chunk step, the GVA reduction and the reverse chunk-local cumsum of dg). With
// dS the gradient w.r.t. a chunk's S_out:
//   dU = Mqk^T dO + kr dS;  dvc = INV^T dU;  dv = diag(beta) dvc
//   dS_in = diag(e^gam) dS + qd^T dO - kd^T diag(beta) dvc
//   dMqk = tril(dO U^T);  dL = -strict_tril(dvc U^T)
//   dqd = dO S_in^T + dMqk ki;  dkd = diag(beta)(dL ki - dvc S_in^T)
//   dki = dMqk^T qd + (diag(beta) dL)^T kd;  dkr = U dS^T
//   dbeta = rowsum(dvc o (v - kd S_in)) + rowsum(kd o (dL ki))
//   dq = scale e^G dqd;  dk = e^G dkd + e^-G dki + e^(gam-G) dkr
//   dG = q o dq + k o (e^G dkd - e^-G dki - e^(gam-G) dkr)
//   dG[last] += e^gam o rowsum(dS o S_in) + sum_j kr_j o dkr_j;  dg = reverse cumsum of dG.
//
// bwd_prep_kernel writes what the reverse scan needs per chunk (kr, -w^T, e^gam and
// W = (qd - Mqk w)^T dO, so that dS_in = diag(e^gam) dS + W - w^T (kr dS)); the scan then
// leaves dS and kr dS per chunk; bwd_grad_kernel forms every gradient of one chunk with
// all C x C triangles kept in LDS. The triangle products take q, k referenced to R per
// column and 16-row block (choose_refs in kda_device.h: R = 0 where |G| stays small), so
// e^(G_i - G_j) never passes through an out-of-range e^(-G).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

#ifdef KDA_PHASE_TIMING
__device__ unsigned long long kda_phase_ts[3][8][64];
extern "C" __attribute__((visibility("default"))) int kda_phase_ts_read(void* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(kda_phase_ts), sizeof(kda_phase_ts), 0, hipMemcpyDeviceToHost);
}
#endif

// LDS plan of the bwd prep kernel, small enough for two workgroups per CU. Later buffers
// overlay earlier ones that a barrier has retired (with QPT the kernel ends at Q'^T, written
// straight to global memory):
//   QL, KiL (phases 0-2: scale q e^(G - R), k e^(R - G), block-referenced) -> dO^T (phase 3)
//   beta kd^T (phases 0-1a)        -> Q'^T (phases 2-3)
//   INV (phases 0-1a)              -> Mqk (phases 1b-2)
//   W^T (phases 1a-2)
template <class T, int K, int V, int C>
struct BwdPrepLds {
  static constexpr int NW = 8;
  static constexpr int P = pad_of<T>();
  static constexpr int LDK = K + P, LDC = C + P;
  static constexpr size_t oQd = 0;
  static constexpr size_t oKi = oQd + sizeof(T) * C * LDK;
  static constexpr size_t oDoT = 0;
  static constexpr size_t oBKdT = oKi + sizeof(T) * C * LDK;
  static constexpr size_t oQpT = oBKdT;
  static constexpr size_t oINV = oBKdT + sizeof(T) * K * LDC;
  static constexpr size_t oMqk = oINV;
  static constexpr size_t oWT = oINV + sizeof(T) * C * LDC;
  static constexpr size_t oBeta = oWT + sizeof(T) * K * LDC;
  static constexpr size_t oRt = oBeta + sizeof(float) * C;  // R of each 16-row block per channel
  static constexpr size_t oD = oRt + sizeof(float) * (C / 16) * K;  // ratios of consecutive R
  static constexpr size_t oFlag = oD + sizeof(float) * (C / 16 - 1) * K;  // per-wave reference mode
  static constexpr size_t total = oFlag + sizeof(int) * NW;
  static_assert(sizeof(T) * V * LDC <= oBKdT, "dO^T overlays QL and KiL");
  static_assert(C > 64 || total <= 80 * 1024, "two workgroups per CU");
};

// One workgroup per (chunk, value head); two fit on a CU (LDS plan above, at most 128
// VGPRs), so one's loads overlap the other's products. QPT: the scan forms W = Q'^T dO
// itself, so this kernel writes Q'^T in the scan's K x C fragment order instead of W, and
// reads no dO.
template <class T, int K, int V, int C, bool QPT>
__global__ __launch_bounds__(512, 4) void bwd_prep_kernel(Shape s, const T* __restrict__ qp, const T* __restrict__ kp,
                                                        const float* __restrict__ gp, const float* __restrict__ bp,
                                                        const T* __restrict__ invp, const T* __restrict__ dOp,
                                                        BwdWs ws) {
  typedef BwdPrepLds<T, K, V, C> Lay;
  constexpr int NW = Lay::NW, NTH = 64 * NW, RT = C / 16, KT = K / 16, VT = V / 16;
  constexpr int NCK = (KT + NW - 1) / NW, NCV = (VT + NW - 1) / NW, NI = (C * C + NTH - 1) / NTH;
  constexpr int LDK = Lay::LDK, LDC = Lay::LDC;
  __shared__ __align__(16) unsigned char smem[Lay::total];
  T* QL = reinterpret_cast<T*>(smem + Lay::oQd);
  T* KiL = reinterpret_cast<T*>(smem + Lay::oKi);
  float* Rt = reinterpret_cast<float*>(smem + Lay::oRt);
  float* D = reinterpret_cast<float*>(smem + Lay::oD);
  int* wflag = reinterpret_cast<int*>(smem + Lay::oFlag);
  T* BKdT = reinterpret_cast<T*>(smem + Lay::oBKdT);
  T* DoT = reinterpret_cast<T*>(smem + Lay::oDoT);
  T* INVt = reinterpret_cast<T*>(smem + Lay::oINV);
  T* Mqk = reinterpret_cast<T*>(smem + Lay::oMqk);
  T* WT = reinterpret_cast<T*>(smem + Lay::oWT);
  T* QpT = reinterpret_cast<T*>(smem + Lay::oQpT);
  float* betas = reinterpret_cast<float*>(smem + Lay::oBeta);

  // heads of one chunk are neighbouring workgroups (together they read whole token rows), a
  // q/k group's on one XCD
  const int task = group_task(blockIdx.x, s.HV / s.H, s.NT * s.nhv);
  if (task < 0) return;
  const int c = task / s.nhv, h = s.hv0 + task % s.nhv;
  const int hq = h / (s.HV / s.H);
  const Geo geo = chunk_geo(c, s.cu, s.choff, s.N, s.T, C);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, grp = lane >> 4;
  const long ch = (long)c * s.HV + h;
  const int len = geo.len;
  if (len <= 0) return;
  const int qs = s.H * K, gs = s.HV * K, vs = s.HV * V;
  const T* __restrict__ qc = qp + (geo.bos * s.H + hq) * K;
  const T* __restrict__ kc = kp + (geo.bos * s.H + hq) * K;
  const float* __restrict__ gc = gp + (geo.bos * s.HV + h) * K;
  const T* __restrict__ dOc = dOp + (geo.bos * s.HV + h) * V;
  const float* __restrict__ bc = bp + geo.bos * s.HV + h;
  const T* __restrict__ invc = invp + ch * C * C;
  T* __restrict__ krg = reinterpret_cast<T*>(ws.kr) + ch * C * K;
  float* __restrict__ egc = ws.eg + ch * K;

  KDA_TS(0, 0);
  // ---- every global load of the chunk, issued before any use
  const float beta_raw = beta_of(bc[min(tid % C, len - 1) * s.HV], s.beta_logits);
  float G[NCK][RT][4], qv[NCK][RT][4], kv[NCK][RT][4];
#pragma unroll
  for (int ci = 0; ci < NCK; ++ci) {
    const int kt = wave + ci * NW;
    if (kt < KT) {
      col_load<float, RT>(G[ci], gc, gs, 16 * kt + n, grp, len);
      col_load<T, RT>(qv[ci], qc, qs, 16 * kt + n, grp, len);
      col_load<T, RT>(kv[ci], kc, qs, 16 * kt + n, grp, len);
    }
  }
  typedef T vecT __attribute__((ext_vector_type(16 / sizeof(T))));
  constexpr int VEC = 16 / (int)sizeof(T), NIV = (C * C / VEC + NTH - 1) / NTH;
  vecT iv[NIV];
#pragma unroll
  for (int i = 0; i < NIV; ++i) iv[i] = *reinterpret_cast<const vecT*>(invc + min(tid + i * NTH, C * C / VEC - 1) * VEC);
  if (tid < C) betas[tid] = tid < len ? beta_raw : 0.f;
  __syncthreads();

  // ---- gate cumsum and the decayed keys / queries
  bool strong_w = false;  // this wave's columns take block references
#pragma unroll
  for (int ci = 0; ci < NCK; ++ci) {
    const int kt = wave + ci * NW;
    if (kt < KT) {
      const int col = 16 * kt + n;
      const float gam = col_prefix<RT>(G[ci], lane);  // the column total is gam
      float R[RT];
      strong_w = choose_refs<RT>(G[ci], R, lane) || strong_w;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 bk, ql4, ki4, kr4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 16 * rt + 4 * grp + j;
          const float e = __expf(G[ci][rt][j]);
          ql4[j] = s.scale * qv[ci][rt][j] * __expf(G[ci][rt][j] - R[rt]);
          ki4[j] = kv[ci][rt][j] * __expf(R[rt] - G[ci][rt][j]);
          bk[j] = betas[row] * kv[ci][rt][j] * e;
          kr4[j] = kv[ci][rt][j] * __expf(gam - G[ci][rt][j]);
        }
        if (grp == 0) {
          Rt[rt * K + col] = R[rt];
          if (rt + 1 < RT) D[rt * K + col] = __expf(R[rt + 1] - R[rt]);
        }
        store_rows<T>(QL, LDK, 16 * rt, 16 * kt, ql4, lane, 1 << 30);
        store_rows<T>(KiL, LDK, 16 * rt, 16 * kt, ki4, lane, 1 << 30);
        if constexpr (sizeof(T) == 2) {
          // row layout (this lane: row 16rt + n, columns 16kt + 4grp ..): one 8-byte piece
          st4(krg + ScanFrag<K, V, C>::p1(16 * rt + n, 16 * kt + 4 * grp), to_rows_bf16(kr4[0], kr4[1], kr4[2], kr4[3], lane));
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) krg[(16 * rt + 4 * grp + j) * K + col] = kr4[j];
        }
        st4(BKdT + col * LDC + 16 * rt + 4 * grp, bk);
      }
      if (grp == 0) egc[col] = __expf(gam);
    }
  }
  if (lane == 0) wflag[wave] = strong_w;
  // dO (first used by W at the end): issued once g, q and k have arrived, so that the
  // opening burst of the two workgroups of a CU is smaller and dO lands during the products
  T dor[NCV][RT][4];
  if constexpr (!QPT) {
#pragma unroll
    for (int cv = 0; cv < NCV; ++cv) {
      const int vt = min(wave + cv * NW, VT - 1);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) dor[cv][rt][j] = dOc[min(16 * rt + 4 * grp + j, len - 1) * vs + 16 * vt + n];
    }
  }
#pragma unroll
  for (int i = 0; i < NIV; ++i) {
    const int pid = tid + i * NTH;
    if (pid < C * C / VEC) {
      const int r = (pid * VEC) / C, c0 = (pid * VEC) % C;
      vecT m;
#pragma unroll
      for (int t = 0; t < VEC; ++t) m[t] = (r < len && c0 + t < len) ? iv[i][t] : from_f<T>(r == c0 + t ? 1.f : 0.f);
      st_2x8(INVt + r * LDC + c0, m);
    }
  }
  __syncthreads();

  KDA_TS(0, 1);
  // w = INV diag(beta) kd: kept transposed in LDS, stored negated and transposed for the scan.
  T* __restrict__ nwT = reinterpret_cast<T*>(ws.nwT) + ch * (sizeof(T) == 2 ? ScanFrag<K, V, C>::P2_ELEMS : K * C);
  constexpr int BNK = KT % 2 == 0 ? 2 : 1;
  block_gemm<T, RT, KT, BNK, NW, C>(
      INVt, LDC, 1 << 30, BKdT, LDC, [](int mt, int, int& kb, int& ke) { ke = min(C, round_up<T>(16 * (mt + 1))); },
      [&](int, int mt, int nt0, f32x4(&acc)[BNK]) {
#pragma unroll
        for (int jb = 0; jb < BNK; ++jb) {
          const int col = 16 * (nt0 + jb) + n;
          st4(WT + col * LDC + 16 * mt + 4 * grp, acc[jb]);
          if constexpr (sizeof(T) == 2) {
            st4(nwT + ScanFrag<K, V, C>::p2(col, 16 * mt + 4 * grp), -acc[jb]);
          } else {
            st4(nwT + col * C + 16 * mt + 4 * grp, -acc[jb]);
          }
        }
      }, wave, lane);
  __syncthreads();  // INV and beta kd^T retired
  // Mqk = tril(qd ki^T), row-major, from the block-referenced q and keys.
  const bool scl = any_flag<NW>(wflag);  // some column takes block references
  tri_tiles<T, RT, NW, K>(
      QL, LDK, KiL, LDK, D, K, scl,
      [&](int mt, int nt0, f32x4 acc) {
        f32x4 m4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 16 * mt + 4 * grp + j, col = 16 * nt0 + n;
          m4[j] = col <= row ? acc[j] : 0.f;
        }
        store_rows<T>(Mqk, LDC, 16 * mt, 16 * nt0, m4, lane, 1 << 30);
      }, wave, lane);
  __syncthreads();
  KDA_TS(0, 2);
  // Q' = qd - Mqk w, transposed (qd = QL e^R, rows of block mt).
  block_gemm<T, RT, KT, BNK, NW, C>(
      Mqk, LDC, 1 << 30, WT, LDC, [](int mt, int, int& kb, int& ke) { ke = min(C, round_up<T>(16 * (mt + 1))); },
      [&](int, int mt, int nt0, f32x4(&acc)[BNK]) {
#pragma unroll
        for (int jb = 0; jb < BNK; ++jb) {
          const int col = 16 * (nt0 + jb) + n;
          f32x4 qp4;
          const float eR = scl ? __expf(Rt[mt * K + col]) : 1.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) qp4[j] = to_f(QL[(16 * mt + 4 * grp + j) * LDK + col]) * eR - acc[jb][j];
          if constexpr (QPT) {
            static_assert(sizeof(T) == 2 && ScanFrag<K, V, C>::P2_ELEMS <= V * K, "Q'^T fits the W buffer");
            st4(reinterpret_cast<T*>(ws.bcT) + ch * ScanFrag<K, V, C>::P2_ELEMS + ScanFrag<K, V, C>::p2(col, 16 * mt + 4 * grp), qp4);
          } else {
            st4(QpT + col * LDC + 16 * mt + 4 * grp, qp4);
          }
        }
      }, wave, lane);
  if constexpr (QPT) return;
  __syncthreads();  // QL, KiL, Mqk, W^T retired
  // dO^T over QL and KiL
#pragma unroll
  for (int cv = 0; cv < NCV; ++cv) {
    const int vt = wave + cv * NW;
    if (vt < VT) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 d4;
#pragma unroll
        for (int j = 0; j < 4; ++j) d4[j] = 16 * rt + 4 * grp + j < len ? to_f(dor[cv][rt][j]) : 0.f;
        st4(DoT + (16 * vt + n) * LDC + 16 * rt + 4 * grp, d4);
      }
    }
  }
  __syncthreads();
  KDA_TS(0, 3);
  // W = Q'^T dO, stored transposed [V][K].
  T* __restrict__ bcT = reinterpret_cast<T*>(ws.bcT) + ch * V * K;
  constexpr int BNV = VT % 2 == 0 ? 2 : 1;
  block_gemm<T, KT, VT, BNV, NW, C>(QpT, LDC, 1 << 30, DoT, LDC, FullRange(),
                                    [&](int, int mt, int nt0, f32x4(&acc)[BNV]) {
#pragma unroll
                                      for (int jb = 0; jb < BNV; ++jb)
                                        if constexpr (sizeof(T) == 2) {
                                          // column v = 16(nt0 + jb) + n goes to its scan slice and lane
                                          const int v = 16 * (nt0 + jb) + n;
                                          st4(bcT + ScanFrag<K, V, C>::seed(ScanCols::slice(v), mt, KT,
                                                                            ScanCols::lane_col(v) + 16 * grp),
                                              acc[jb]);
                                        } else {
                                          st4(bcT + (16 * (nt0 + jb) + n) * K + 16 * mt + 4 * grp, acc[jb]);
                                        }
                                    }, wave, lane);
  KDA_TS(0, 4);
}

// LDS plan of the gradient kernel. Phase-2 temporaries alias buffers that are written
// later; every alias is separated from its predecessor's last read by a barrier.
//   region A [0, endA): Qd, Kd, Ki, S_in^T (phase 1-2)  |  Qd^T, Kd^T, Ki^T, U, -dvc (phase 2-3)
//   region B [endA, endB): vcorr^T then dU^T, INV, INV^T  |  dMqk, dMqk^T, dL, (beta dL)^T
//   then Mqk^T, beta, dbeta partials, dO^T
template <class T, int K, int V, int C>
struct GradLds {
  static constexpr int NW = 8;
  static constexpr int P = pad_of<T>();
  static constexpr int LDK = K + P, LDC = C + P, LDV = V + P;
  static constexpr size_t szCK = sizeof(T) * C * LDK, szKC = sizeof(T) * K * LDC, szCV = sizeof(T) * C * LDV;
  static constexpr size_t szVC = sizeof(T) * V * LDC, szVK = sizeof(T) * V * LDK, szCC = sizeof(T) * C * LDC;
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t oQd = 0, oKd = szCK, oKi = 2 * szCK, oSinT = 3 * szCK;
  static constexpr size_t oQdT = 0, oKdT = szKC, oKiT = 2 * szKC, oU = 3 * szKC, oNdv = 3 * szKC + szCV;
  static constexpr size_t endA = mx(3 * szCK + szVK, 3 * szKC + 2 * szCV);
  static constexpr size_t oVcT = endA, oDuT = endA;
  static constexpr size_t oINV = endA + szVC, oINVT = oINV + szCC;
  static constexpr size_t oDMqk = endA, oDMqkT = endA + szCC, oDL = endA + 2 * szCC, oDLT = endA + 3 * szCC;
  static constexpr size_t endB = mx(endA + szVC + 2 * szCC, endA + 4 * szCC);
  static constexpr size_t oMqkT = endB;
  static constexpr size_t oBeta = oMqkT + szCC;
  static constexpr size_t oRt = oBeta + sizeof(float) * C;  // R of each 16-row block per channel
  static constexpr size_t oD = oRt + sizeof(float) * (C / 16) * K;  // ratios of consecutive R
  static constexpr size_t oFlag = oD + sizeof(float) * (C / 16 - 1) * K;  // per-wave reference mode
  static constexpr size_t oDbp = oFlag + sizeof(int) * NW;
  static constexpr size_t oDoT = oDbp + sizeof(float) * 2 * NW * C;  // dbeta partials: dvc part, then phase-3 part
  // dg leaves through the dO slot in passes of SR rows of K fp32 (row stride K + 4)
  static constexpr int SR = C < 32 ? C : 32;
  static constexpr size_t total = mx(oDoT + szVC, oDoT + sizeof(float) * SR * (K + 4));
  static_assert(total <= 160 * 1024, "gradient kernel exceeds the LDS of one CU");
};

// One workgroup per (chunk, q/k head); the value heads of the group are processed in
// turn and their dq, dk contributions summed in registers. Each phase issues all of its
// global loads before using any of them; q, k and the gate cumsum G stay in registers
// for the whole value head, and dO is read from HBM once (as 16-byte row vectors) and
// staged in LDS transposed (for dU) and then row-major (for dMqk and dq).
template <class T, int K, int V, int C, bool GVA>
__global__ __launch_bounds__(512) void bwd_grad_kernel(Shape s, const T* __restrict__ qp, const T* __restrict__ kp,
                                                        const T* __restrict__ vp, const float* __restrict__ gp,
                                                        const float* __restrict__ bp, const T* __restrict__ states,
                                                        const T* __restrict__ invp, const T* __restrict__ dOp,
                                                        BwdWs ws, T* __restrict__ dqp, T* __restrict__ dkp,
                                                        T* __restrict__ dvp, float* __restrict__ dgp,
                                                        float* __restrict__ dbp) {
  typedef GradLds<T, K, V, C> Lay;
  typedef Mma<T> M;
  typedef T vecT __attribute__((ext_vector_type(16 / sizeof(T))));
  constexpr int NW = Lay::NW, NTH = 64 * NW, RT = C / 16, KT = K / 16, VT = V / 16;
  constexpr int NCT = (KT + NW - 1) / NW, NCV = (VT + NW - 1) / NW, NI = (C * C + NTH - 1) / NTH;
  constexpr int VEC = 16 / (int)sizeof(T), NVEC = C * V / VEC, NDV = (NVEC + NTH - 1) / NTH;
  constexpr int LDK = Lay::LDK, LDC = Lay::LDC, LDV = Lay::LDV;
  constexpr int BN1 = VT % 2 == 0 ? 2 : 1;
  static_assert(NW >= VT / BN1, "the blocks of one wave in the C x V walk lie in different row tiles");
  constexpr int NIT1 = (RT * (VT / BN1) + NW - 1) / NW;
  constexpr int NITC = (RT * RT + NW - 1) / NW;
  constexpr int NKV = V / M::KS;
  __shared__ __align__(16) unsigned char smem[Lay::total];
  T* QL = reinterpret_cast<T*>(smem + Lay::oQd);
  T* Kd = reinterpret_cast<T*>(smem + Lay::oKd);
  T* KiL = reinterpret_cast<T*>(smem + Lay::oKi);
  T* SinT = reinterpret_cast<T*>(smem + Lay::oSinT);
  T* QLT = reinterpret_cast<T*>(smem + Lay::oQdT);
  T* BKLT = reinterpret_cast<T*>(smem + Lay::oKdT);
  T* KiLT = reinterpret_cast<T*>(smem + Lay::oKiT);
  T* U = reinterpret_cast<T*>(smem + Lay::oU);
  T* Ndv = reinterpret_cast<T*>(smem + Lay::oNdv);
  T* VcT = reinterpret_cast<T*>(smem + Lay::oVcT);
  T* DuT = reinterpret_cast<T*>(smem + Lay::oDuT);
  T* INVt = reinterpret_cast<T*>(smem + Lay::oINV);
  T* INVTt = reinterpret_cast<T*>(smem + Lay::oINVT);
  T* DMqk = reinterpret_cast<T*>(smem + Lay::oDMqk);
  T* DMqkT = reinterpret_cast<T*>(smem + Lay::oDMqkT);
  T* DL = reinterpret_cast<T*>(smem + Lay::oDL);
  T* DLT = reinterpret_cast<T*>(smem + Lay::oDLT);
  T* MqkT = reinterpret_cast<T*>(smem + Lay::oMqkT);
  float* betas = reinterpret_cast<float*>(smem + Lay::oBeta);
  float* Rt = reinterpret_cast<float*>(smem + Lay::oRt);
  float* D = reinterpret_cast<float*>(smem + Lay::oD);
  int* wflag = reinterpret_cast<int*>(smem + Lay::oFlag);
  float* dbpart = reinterpret_cast<float*>(smem + Lay::oDbp);
  T* DoT = reinterpret_cast<T*>(smem + Lay::oDoT);  // dO^T, then dO row-major (same slot)
  T* DoR = DoT;

  // heads of one chunk are neighbouring workgroups: together they read whole token rows
  const int nhq = s.nhv / (s.HV / s.H);
  const int c = blockIdx.x / nhq, hq = s.hv0 / (s.HV / s.H) + blockIdx.x % nhq;
  const int Gq = s.HV / s.H;
  const Geo geo = chunk_geo(c, s.cu, s.choff, s.N, s.T, C);
  if (geo.len <= 0) return;
  const long bos = geo.bos;
  const int qs = s.H * K, gs = s.HV * K, vs = s.HV * V;
  const T* __restrict__ qc = qp + (bos * s.H + hq) * K;
  const T* __restrict__ kc = kp + (bos * s.H + hq) * K;
  T* __restrict__ dqc = dqp + (bos * s.H + hq) * K;
  T* __restrict__ dkc = dkp + (bos * s.H + hq) * K;

  // Grouped heads sum dq, dk over the group in registers; otherwise they are stored
  // directly from phase 3.
  constexpr int NACC = GVA ? NCT : 1;
  float dqa[NACC][RT][4], dka[NACC][RT][4];
#pragma unroll
  for (int ci = 0; ci < NACC; ++ci)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) dqa[ci][rt][j] = dka[ci][rt][j] = 0.f;

  for (int e = 0; e < Gq; ++e) {
    const int h = hq * Gq + e;
    const long ch = (long)c * s.HV + h;
    // Per-iteration opaque copies: keep lane-dependent addresses and row masks from being
    // hoisted out of this loop (which would hold hundreds of them live across its body).
    const int tid = opaque_v(threadIdx.x);
    const int lane = tid & 63, n = lane & 15, grp = lane >> 4;
    const int wave = opaque_s(__builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
    const int len = opaque_s(__builtin_amdgcn_readfirstlane(geo.len));
    const T* __restrict__ Sin = states + ch * K * V;
    const T* __restrict__ dSo = reinterpret_cast<const T*>(ws.dS) + ch * K * V;
    const T* __restrict__ yT = reinterpret_cast<const T*>(ws.yT) + ch * V * C;
    const T* __restrict__ dOc = dOp + (bos * s.HV + h) * V;
    const T* __restrict__ vc = vp + (bos * s.HV + h) * V;
    const float* __restrict__ gc = gp + (bos * s.HV + h) * K;
    const float* __restrict__ bc = bp + bos * s.HV + h;
    const T* __restrict__ invc = invp + ch * C * C;
    T* __restrict__ dvc_out = dvp + (bos * s.HV + h) * V;
    float* __restrict__ dgc = dgp + (bos * s.HV + h) * K;
    float* __restrict__ dbc = dbp + bos * s.HV + h;

    KDA_TS(2, 0);
    // ---- phase 1: every global load of this value head, issued before any use
    // beta: loaded with the rest, written to LDS once everything is in flight
    const float beta_raw = beta_of(bc[min(tid % C, len - 1) * s.HV], s.beta_logits);
    for (int i = tid; i < NW * C; i += NTH) dbpart[i] = 0.f;  // dvc part (written sparsely)
    float Gr[NCT][RT][4], qv[NCT][RT][4], kv[NCT][RT][4];
    ColTile<float, RT> tg[NCT];
    ColTile<T, RT> tq[NCT], tk[NCT];
#pragma unroll
    for (int ci = 0; ci < NCT; ++ci) {
      const int kt = min(wave + ci * NW, KT - 1);  // clamped: loads stay unconditional
      tg[ci].load(gc, gs, 16 * kt, lane, len);
      tq[ci].load(qc, qs, 16 * kt, lane, len);
      tk[ci].load(kc, qs, 16 * kt, lane, len);
    }
    // S_in, INV and dO as 16-byte row pieces. bf16 (BLK): piece i of this lane is in 16 x 32
    // block b = wave + i*NW of the matrix (blocks down the rows first), row 16(b % row
    // tiles) + n, columns 32(b / row tiles) + 8grp .. +7, so each block can be written
    // transposed into LDS by store_T_block. Otherwise piece i of thread tid covers elements
    // VEC*pid .. of a row, pid = tid + i*NTH (S_in: lanes on consecutive rows).
    constexpr bool BLK = sizeof(T) == 2 && C % 32 == 0 && V % 32 == 0 && K % 16 == 0;
    constexpr int NBS = KT * (V / 32), NBI = RT * (C / 32), NBD = RT * (V / 32);
    auto blk_rc = [&](int b, int rtiles, int& r, int& c) {
      r = 16 * (b % rtiles) + n;
      c = 32 * (b / rtiles) + 8 * grp;
    };
    constexpr int NSV = (K * V / VEC + NTH - 1) / NTH;
    // with one column tile per wave, the row pieces of S_in this wave loads here (blocks
    // wave + i NW: rows 16 wave + n, columns 32 i + 8 grp) are the B fragments of its phase-3
    // products, kept in registers instead of loading S_in a second time
    constexpr bool SIN_REUSE = BLK && NCT == 1 && KT == NW && NSV == V / M::KS;
    vecT sv[NSV];
#pragma unroll
    for (int i = 0; i < NSV; ++i) {
      if constexpr (BLK) {
        int r, c;
        blk_rc(min(wave + i * NW, NBS - 1), KT, r, c);
        sv[i] = *reinterpret_cast<const vecT*>(Sin + r * V + c);
      } else {
        const int pid = min(tid + i * NTH, K * V / VEC - 1);
        sv[i] = *reinterpret_cast<const vecT*>(Sin + (pid % K) * V + (pid / K) * VEC);
      }
    }
    constexpr int NIV = (C * C / VEC + NTH - 1) / NTH;
    vecT iv[NIV];
#pragma unroll
    for (int i = 0; i < NIV; ++i) {
      if constexpr (BLK) {
        int r, c;
        blk_rc(min(wave + i * NW, NBI - 1), RT, r, c);
        iv[i] = *reinterpret_cast<const vecT*>(invc + r * C + c);
      } else {
        iv[i] = *reinterpret_cast<const vecT*>(invc + min(tid + i * NTH, C * C / VEC - 1) * VEC);
      }
    }

    // ---- phase 1 compute: column tiles of g, q, k and v into the column-owner layout; gate
    // cumsum, block references R, block-referenced q and keys and decayed keys (row-major),
    // S_in^T
    if (tid < C) betas[tid] = tid < len ? beta_raw : 0.f;
#pragma unroll
    for (int ci = 0; ci < NCT; ++ci) {
      if (wave + ci * NW < KT) {
        tg[ci].get(Gr[ci], lane, len);
        tq[ci].get(qv[ci], lane, len);
        tk[ci].get(kv[ci], lane, len);
      }
    }
    // v, dO and (kr dS)^T are first used after the first barrier: issued once the first tiles
    // have arrived, so that the opening burst of every CU is smaller and these land during
    // phase 1
    // v at the places of the C x V accumulator tiles this wave owns in the block walk of
    // kd S_in and INV^T dU (same walk: RT x VT tiles in blocks of 1 x BN1)
    typedef T t4 __attribute__((ext_vector_type(4)));
    t4 vraw[NIT1][BN1];
    ColTile<T, 1> tv[NIT1][BN1];
#pragma unroll
    for (int it = 0; it < NIT1; ++it) {
      const int blk = min(wave + it * NW, RT * (VT / BN1) - 1);
      const int mt = blk / (VT / BN1), nt0 = (blk % (VT / BN1)) * BN1;
#pragma unroll
      for (int jb = 0; jb < BN1; ++jb) tv[it][jb].load(vc, vs, 16 * (nt0 + jb), lane, len, 16 * mt);
    }
    vecT dov[NDV];
#pragma unroll
    for (int i = 0; i < NDV; ++i) {
      int row, c;
      if constexpr (BLK) {
        blk_rc(min(wave + i * NW, NBD - 1), RT, row, c);
      } else {
        const int vi = min(tid + i * NTH, NVEC - 1);
        row = vi / (V / VEC);
        c = (vi % (V / VEC)) * VEC;
      }
      dov[i] = *reinterpret_cast<const vecT*>(dOc + min(row, len - 1) * vs + c);
      if (row >= len) dov[i] = vecT{};
    }
    // (kr dS)^T at the places of the dU tiles this wave owns (same block walk), for the dU
    // epilogue
    t4 yraw[NIT1][BN1];
#pragma unroll
    for (int it = 0; it < NIT1; ++it) {
      const int blk = min(wave + it * NW, RT * (VT / BN1) - 1);
      const int mt = blk / (VT / BN1), nt0 = (blk % (VT / BN1)) * BN1;
#pragma unroll
      for (int jb = 0; jb < BN1; ++jb) {
        const int v = 16 * (nt0 + jb) + n;
        if constexpr (sizeof(T) == 2)  // the bf16 scan's order: value column v at lane column lane_col(v) of slice slice(v)
          yraw[it][jb] = *reinterpret_cast<const t4*>(yT + ScanFrag<K, V, C>::seed(ScanCols::slice(v), mt, RT, ScanCols::lane_col(v) + 16 * grp));
        else
          yraw[it][jb] = *reinterpret_cast<const t4*>(yT + v * C + 16 * mt + 4 * grp);
      }
    }
    float gam[NCT];
    bool strong_c[NCT];  // column tile ci takes block references
#pragma unroll
    for (int ci = 0; ci < NCT; ++ci) {
      const int kt = wave + ci * NW;
      gam[ci] = 0.f;
      strong_c[ci] = false;
      if (kt < KT) {
        const int col = 16 * kt + n;
        gam[ci] = col_prefix<RT>(Gr[ci], lane);  // the column total is gam
        float R[RT];
        strong_c[ci] = choose_refs<RT>(Gr[ci], R, lane);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          f32x4 q4, kd4, ki4;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float G = Gr[ci][rt][j];
            q4[j] = s.scale * qv[ci][rt][j] * __expf(G - R[rt]);
            kd4[j] = kv[ci][rt][j] * __expf(G);
            ki4[j] = kv[ci][rt][j] * __expf(R[rt] - G);
          }
          if (grp == 0) {
            Rt[rt * K + col] = R[rt];
            if (rt + 1 < RT) D[rt * K + col] = __expf(R[rt + 1] - R[rt]);
          }
          if constexpr (sizeof(T) == 2) {
            // row layout (this lane: row 16rt + n, columns 16kt + 4grp ..): 8-byte writes
            const int off = (16 * rt + n) * LDK + 16 * kt + 4 * grp;
            st4(QL + off, to_rows_bf16(q4[0], q4[1], q4[2], q4[3], lane));
            st4(Kd + off, to_rows_bf16(kd4[0], kd4[1], kd4[2], kd4[3], lane));
            st4(KiL + off, to_rows_bf16(ki4[0], ki4[1], ki4[2], ki4[3], lane));
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int row = 16 * rt + 4 * grp + j;
              QL[row * LDK + col] = from_f<T>(q4[j]);
              Kd[row * LDK + col] = from_f<T>(kd4[j]);
              KiL[row * LDK + col] = from_f<T>(ki4[j]);
            }
          }
        }
      }
    }
    {
      int f = 0;
#pragma unroll
      for (int ci = 0; ci < NCT; ++ci) f |= strong_c[ci];
      if (lane == 0) wflag[wave] = f;
    }
#pragma unroll
    for (int i = 0; i < NSV; ++i) {
      if constexpr (BLK) {
        const int b = wave + i * NW;
        if (b < NBS) store_T_block(SinT, LDK, 16 * (b % KT), 32 * (b / KT), sv[i], lane);
      } else {
        const int pid = tid + i * NTH;
        if (pid < K * V / VEC) {
          const int row = pid % K, c0 = (pid / K) * VEC;
#pragma unroll
          for (int t = 0; t < VEC; ++t) SinT[(c0 + t) * LDK + row] = sv[i][t];
        }
      }
    }
    __syncthreads();
    KDA_TS(2, 1);
    // INV and INV^T (read first by U = INV vcorr, after the next barrier)
#pragma unroll
    for (int i = 0; i < NIV; ++i) {
      if constexpr (BLK) {
        const int b = wave + i * NW;
        if (b < NBI) {
          int r, c0;
          blk_rc(b, RT, r, c0);
          vecT m;
#pragma unroll
          for (int t = 0; t < VEC; ++t) m[t] = (r < len && c0 + t < len) ? iv[i][t] : from_f<T>(r == c0 + t ? 1.f : 0.f);
          st_2x8(INVt + r * LDC + c0, m);
          store_T_block(INVTt, LDC, 16 * (b % RT), 32 * (b / RT), m, lane);
        }
      } else {
        const int pid = tid + i * NTH;
        if (pid < C * C / VEC) {
          const int r = (pid * VEC) / C, c0 = (pid * VEC) % C;
#pragma unroll
          for (int t = 0; t < VEC; ++t) {
            const int cc = c0 + t;
            const T val = (r < len && cc < len) ? iv[i][t] : from_f<T>(r == cc ? 1.f : 0.f);
            INVt[r * LDC + cc] = val;
            INVTt[cc * LDC + r] = val;
          }
        }
      }
    }

    // ---- Mqk = tril(qd ki^T) -> Mqk^T, from the block-referenced q and keys
    tri_tiles<T, RT, NW, K>(
        QL, LDK, KiL, LDK, D, K, any_flag<NW>(wflag),
        [&](int mt, int nt0, f32x4 acc) {
          f32x4 m4;
#pragma unroll
          for (int j = 0; j < 4; ++j) m4[j] = (16 * nt0 + n <= 16 * mt + 4 * grp + j) ? acc[j] : 0.f;
          st4(MqkT + (16 * nt0 + n) * LDC + 16 * mt + 4 * grp, m4);
        }, wave, lane);
#pragma unroll
    for (int it = 0; it < NIT1; ++it) {
      const int blk = min(wave + it * NW, RT * (VT / BN1) - 1);
      const int mt = blk / (VT / BN1);
#pragma unroll
      for (int jb = 0; jb < BN1; ++jb) {
        float x[1][4];
        tv[it][jb].get(x, lane, len, 16 * mt);
#pragma unroll
        for (int j = 0; j < 4; ++j) vraw[it][jb][j] = from_f<T>(x[0][j]);
      }
    }
    // ---- kd S_in -> vcorr^T = (beta (v - kd S_in))^T
    block_gemm<T, RT, VT, BN1, NW, K>(Kd, LDK, 1 << 30, SinT, LDK, FullRange(),
                                      [&](int it, int mt, int nt0, f32x4(&acc)[BN1]) {
#pragma unroll
                                        for (int jb = 0; jb < BN1; ++jb) {
                                          const int col = 16 * (nt0 + jb) + n;
                                          f32x4 r, b4;
#pragma unroll
                                          for (int j = 0; j < 4; ++j) {
                                            const int row = 16 * mt + 4 * grp + j;
                                            r[j] = to_f(vraw[it][jb][j]) - acc[jb][j];
                                            b4[j] = betas[row] * r[j];
                                          }
                                          st4(VcT + col * LDC + 16 * mt + 4 * grp, b4);
                                        }
                                      }, wave, lane);
    __syncthreads();

    KDA_TS(2, 2);
    // ---- block-referenced q^T, (beta k)^T (decayed) and k^T (inverse decay), region A over
    // the dead QL/Kd/KiL/S_in^T; dO^T
#pragma unroll
    for (int ci = 0; ci < NCT; ++ci) {
      const int kt = wave + ci * NW;
      if (kt < KT) {
        const int col = 16 * kt + n;
        // LDS reads first: a read issued after the stores below would wait for them
        f32x4 b4s[RT];
        float Rs[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          b4s[rt] = *reinterpret_cast<const f32x4*>(betas + 16 * rt + 4 * grp);
          Rs[rt] = strong_c[ci] ? Rt[rt * K + col] : 0.f;
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float Rr = Rs[rt];
          const f32x4 b4 = b4s[rt];
          f32x4 q4, kd4, ki4;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float eGR = __expf(Gr[ci][rt][j] - Rr);
            q4[j] = s.scale * qv[ci][rt][j] * eGR;
            kd4[j] = b4[j] * (kv[ci][rt][j] * eGR);
            ki4[j] = kv[ci][rt][j] * __expf(Rr - Gr[ci][rt][j]);
          }
          st4(QLT + col * LDC + 16 * rt + 4 * grp, q4);
          st4(BKLT + col * LDC + 16 * rt + 4 * grp, kd4);
          st4(KiLT + col * LDC + 16 * rt + 4 * grp, ki4);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NDV; ++i) {
      if constexpr (BLK) {
        const int b = wave + i * NW;
        if (b < NBD) store_T_block(DoT, LDC, 16 * (b % RT), 32 * (b / RT), dov[i], lane);
      } else {
        const int vi = tid + i * NTH;
        if (vi < NVEC) {
          const int row = vi / (V / VEC), c8 = vi % (V / VEC);
#pragma unroll
          for (int t = 0; t < VEC; ++t) DoT[(c8 * VEC + t) * LDC + row] = dov[i][t];
        }
      }
    }
    // ---- U = INV vcorr (row-major)
    block_gemm<T, RT, VT, BN1, NW, C>(
        INVt, LDC, 1 << 30, VcT, LDC, [](int mt, int, int& kb, int& ke) { ke = min(C, round_up<T>(16 * (mt + 1))); },
        [&](int, int mt, int nt0, f32x4(&acc)[BN1]) {
#pragma unroll
          for (int jb = 0; jb < BN1; ++jb) store_rows<T>(U, LDV, 16 * mt, 16 * (nt0 + jb), acc[jb], lane, 1 << 30);
        }, wave, lane);
    __syncthreads();

    KDA_TS(2, 3);
    // ---- dU = Mqk^T dO + kr dS -> dU^T
    block_gemm<T, RT, VT, BN1, NW, C>(
        MqkT, LDC, 1 << 30, DoT, LDC, [](int mt, int, int& kb, int& ke) { kb = round_dn<T>(16 * mt); },
        [&](int it, int mt, int nt0, f32x4(&acc)[BN1]) {
#pragma unroll
          for (int jb = 0; jb < BN1; ++jb) {
            const f32x4 y = {to_f(yraw[it][jb][0]), to_f(yraw[it][jb][1]), to_f(yraw[it][jb][2]), to_f(yraw[it][jb][3])};
            st4(DuT + (16 * (nt0 + jb) + n) * LDC + 16 * mt + 4 * grp, acc[jb] + y);
          }
        }, wave, lane);
    __syncthreads();

    KDA_TS(2, 4);
    // ---- dO row-major (into the dead dO^T slot); dvc = INV^T dU -> -dvc, dv, dbeta part 1
#pragma unroll
    for (int i = 0; i < NDV; ++i) {
      if constexpr (BLK) {
        const int b = wave + i * NW;
        if (b < NBD) {
          int r, c;
          blk_rc(b, RT, r, c);
          st_2x8(DoR + r * LDV + c, dov[i]);
        }
      } else {
        const int vi = tid + i * NTH;
        if (vi < NVEC) {
          const int row = vi / (V / VEC), c8 = vi % (V / VEC);
          st_2x8(DoR + row * LDV + c8 * VEC, dov[i]);
        }
      }
    }
    block_gemm<T, RT, VT, BN1, NW, C>(
        INVTt, LDC, 1 << 30, DuT, LDC, [](int mt, int, int& kb, int& ke) { kb = round_dn<T>(16 * mt); },
        [&](int it, int mt, int nt0, f32x4(&acc)[BN1]) {
          float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int jb = 0; jb < BN1; ++jb) {
            f32x4 ndv, dvb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int row = 16 * mt + 4 * grp + j;
              const float dvc = acc[jb][j];
              ndv[j] = -dvc;
              dvb[j] = betas[row] * dvc;
              part[j] += dvc * to_f(vraw[it][jb][j]);
            }
            store_rows<T>(Ndv, LDV, 16 * mt, 16 * (nt0 + jb), ndv, lane, 1 << 30);
            store_rows<T>(dvc_out, vs, 16 * mt, 16 * (nt0 + jb), dvb, lane, len);
          }
          // row sums over the 16 columns; lane n < 4 writes row 4grp + n of the tile (each
          // block of a wave has its own row tile, so these are plain writes)
          float pw = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p = row_allsum16(part[j]);
            pw = n == j ? p : pw;
          }
          if (n < 4) dbpart[wave * C + 16 * mt + 4 * grp + n] = pw;
        }, wave, lane);
    __syncthreads();

    KDA_TS(2, 5);
    // The S_in and dS fragments of phase 3 (column tile kt of this wave): issued here so that
    // they arrive during the two products below. dS: the bf16 scan leaves its column slices'
    // tiles as it holds them (4 rows per lane); those of slices 2kk and 2kk+1, transposed by
    // an MFMA against the identity, form the B fragment of columns 32kk.. (done at the point
    // of use in phase 3).
    typedef short s4i __attribute__((ext_vector_type(4)));
    typename M::frag bs[NCT][NKV], bd[NCT][NKV];
    s4i dsr[NCT][NKV][2];
#pragma unroll
    for (int ci = 0; ci < NCT; ++ci) {
      const int kt = min(wave + ci * NW, KT - 1);
#pragma unroll
      for (int kk = 0; kk < NKV; ++kk) {
        // bf16: phase 1 loaded exactly these pieces (rows 16 wave + n, columns 32 kk + 8 grp)
        if constexpr (SIN_REUSE) bs[ci][kk] = sv[kk];
        else bs[ci][kk] = frag_ld16<T>(Sin, V, 16 * kt, kk * M::KS, lane);
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int b = 0; b < 2; ++b)
            dsr[ci][kk][b] = *reinterpret_cast<const s4i*>(dSo + ScanFrag<K, V, C>::seed(2 * kk + b, kt, KT, lane));
        } else {
          bd[ci][kk] = frag_ld16<T>(dSo, V, 16 * kt, kk * M::KS, lane);
        }
      }
    }
    // ---- dMqk = tril(dO U^T); dL = strict_tril(-dvc U^T), in one pass over the 16 x 16
    // tiles: the two products share the U fragments, and tiles above the diagonal load
    // nothing (their zeros are still written: phase 3 reads whole 32-wide steps)
    {
      constexpr int NB = RT * RT, NITM = (NB + NW - 1) / NW, NKV2 = V / M::KS;
#pragma unroll
      for (int it = 0; it < NITM; ++it) {
        const int blk = wave + it * NW;
        if (blk < NB) {
          const int mt = blk / RT, nt0 = blk % RT;
          f32x4 am = zero4(), al = zero4();
          if (nt0 <= mt) {
            typename M::frag fo[NKV2], fn[NKV2], fu[NKV2];
#pragma unroll
            for (int k = 0; k < NKV2; ++k) {
              fu[k] = frag_ld<T>(U, LDV, 16 * nt0, k * M::KS, lane);
              fo[k] = frag_ld<T>(DoR, LDV, 16 * mt, k * M::KS, lane);
              fn[k] = frag_ld<T>(Ndv, LDV, 16 * mt, k * M::KS, lane);
            }
#pragma unroll
            for (int k = 0; k < NKV2; ++k) {
              am = M::mma(fo[k], fu[k], am);
              al = M::mma(fn[k], fu[k], al);
            }
          }
          f32x4 m4, l4;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = 16 * mt + 4 * grp + j, col = 16 * nt0 + n;
            m4[j] = col <= row ? am[j] : 0.f;
            l4[j] = col < row ? al[j] : 0.f;
          }
          store_rows<T>(DMqk, LDC, 16 * mt, 16 * nt0, m4, lane, 1 << 30);
          st4(DMqkT + (16 * nt0 + n) * LDC + 16 * mt + 4 * grp, m4);
          store_rows<T>(DL, LDC, 16 * mt, 16 * nt0, l4, lane, 1 << 30);
          st4(DLT + (16 * nt0 + n) * LDC + 16 * mt + 4 * grp, l4);
        }
      }
    }
    __syncthreads();

    KDA_TS(2, 6);
    // ---- phase 3: per column tile of K, the C x K gradients of this value head
    float dGk[NCT][RT][4];
    float dbz_sum[RT][4];  // dbeta part 2 row sums of this wave's column tiles
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) dbz_sum[rt][j] = 0.f;
    // 16 x 16 identity as the B operand of a 16x16x16 bf16 MFMA (lane: column n, rows 4grp..)
    s4i ident4;
#pragma unroll
    for (int j = 0; j < 4; ++j) ident4[j] = (4 * grp + j == n) ? (short)0x3f80 : (short)0;
#pragma unroll
    for (int ci = 0; ci < NCT; ++ci) {
      const int kt = wave + ci * NW;
      if (kt < KT) {
        const int col = 16 * kt + n;
        f32x4 aq[RT], akd[RT], ai[RT], ar[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) aq[rt] = akd[rt] = ai[rt] = ar[rt] = zero4();
        // ai = dMqk^T qd + dL^T diag(beta) kd relative to R_rt (LDS only: runs while the S_in /
        // dS fragments arrive). Each lane's contraction values lie in one 16-row block blk;
        // the rows of blocks after rt take e^(R_blk - R_rt) <= 1.
        float Rc[RT];  // block references of this lane's column
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) Rc[rt] = strong_c[ci] ? Rt[rt * K + col] : 0.f;
        // this lane's contraction values at step kk lie in block kk/16 (lane groups whose
        // offset PER grp stays below 16) or kk/16 + 1: the reference of its block, clamped
        // to [lo, hi] (indices known at compile time once the loops are unrolled)
        auto pick = [&](int b) {  // Rc[b] as a select chain (no dynamic register indexing)
          float r = Rc[0];
#pragma unroll
          for (int i = 1; i < RT; ++i) r = b == i ? Rc[i] : r;
          return r;
        };
        auto ref_of = [&](int kk, int lo, int hi) {
          const int b0 = min(max(kk >> 4, lo), hi), b1 = min(max((kk + M::KS - 1) >> 4, lo), hi);
          float r0 = pick(b0), r1 = pick(b1);
          asm volatile("" : "+v"(r0), "+v"(r1));  // a select of values, not of array slots
          return ((kk & 15) + M::PER * grp >= 16) ? r1 : r0;
        };
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float Rr = Rc[rt];
#pragma unroll
          for (int kk = round_dn<T>(16 * rt); kk < C; kk += M::KS) {
            typename M::frag bq = frag_ld<T>(QLT, LDC, 16 * kt, kk, lane, C, 1 << 30);
            typename M::frag bk = frag_ld<T>(BKLT, LDC, 16 * kt, kk, lane, C, 1 << 30);
            if (strong_c[ci] && kk + M::KS > 16 * (rt + 1)) {
              const float f = __expf(ref_of(kk, rt, RT - 1) - Rr);
              bq = scale_frag<T>(bq, f);
              bk = scale_frag<T>(bk, f);
            }
            ai[rt] = M::mma(frag_ld<T>(DMqkT, LDC, 16 * rt, kk, lane, C, 1 << 30), bq, ai[rt]);
            ai[rt] = M::mma(frag_ld<T>(DLT, LDC, 16 * rt, kk, lane, C, 1 << 30), bk, ai[rt]);
          }
        }
        float rsum = 0.f;  // this lane's share of sum_v dS[k][v] S_in[k][v], k = col
#pragma unroll
        for (int kk = 0; kk < NKV; ++kk) {
          if constexpr (sizeof(T) == 2) {
            const f32x4 d0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(dsr[ci][kk][0], ident4, zero4(), 0, 0, 0);
            const f32x4 d1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(dsr[ci][kk][1], ident4, zero4(), 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              bd[ci][kk][i] = (bf16)d0[i];
              bd[ci][kk][4 + i] = (bf16)d1[i];
            }
          }
          if constexpr (M::PER == 8) {
#pragma unroll
            for (int i = 0; i < 8; ++i) rsum += (float)bs[ci][kk][i] * (float)bd[ci][kk][i];
          } else {
            rsum += bs[ci][kk] * bd[ci][kk];
          }
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            aq[rt] = M::mma(frag_ld<T>(DoR, LDV, 16 * rt, kk * M::KS, lane), bs[ci][kk], aq[rt]);
            akd[rt] = M::mma(frag_ld<T>(Ndv, LDV, 16 * rt, kk * M::KS, lane), bs[ci][kk], akd[rt]);
            ar[rt] = M::mma(frag_ld<T>(U, LDV, 16 * rt, kk * M::KS, lane), bd[ci][kk], ar[rt]);
          }
        }
        rsum = col_allsum(rsum);
        // aq, akd relative to R_rt: with block references the state terms above take the
        // factor e^(R_rt) (to 0 where it underflows: their true size is below fp32's range);
        // then the triangle products dMqk ki, dL ki, the keys of blocks before rt taking
        // e^(R_rt - R_blk) <= 1
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          if (strong_c[ci]) {
            const float eR = __expf(Rc[rt]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              aq[rt][j] *= eR;
              akd[rt][j] *= eR;
            }
          }
          const int klo = min(C, round_up<T>(16 * (rt + 1)));
#pragma unroll
          for (int kk = 0; kk < klo; kk += M::KS) {
            typename M::frag b = frag_ld<T>(KiLT, LDC, 16 * kt, kk, lane, C, 1 << 30);
            if (strong_c[ci] && kk < 16 * rt) b = scale_frag<T>(b, __expf(Rc[rt] - ref_of(kk, 0, rt)));
            aq[rt] = M::mma(frag_ld<T>(DMqk, LDC, 16 * rt, kk, lane, C, 1 << 30), b, aq[rt]);
            akd[rt] = M::mma(frag_ld<T>(DL, LDC, 16 * rt, kk, lane, C, 1 << 30), b, akd[rt]);
          }
        }
        const float g_last = gam[ci];
        float dG[RT][4];
        float krd = 0.f;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          float dbz[4];
          f32x4 dq4, dk4;
          const float Rr = Rc[rt];
          // dG = q dq + k (dk_d - dk_i - dk_r), its triangle terms taken as the row factors
          // times aq, akd, ai with the factors as rounded into the MFMA operands (read back
          // from them: this lane's 4 rows of its column). A pair (i, j) of the diagonal block
          // then enters dG_i and dG_j as the same product of the same values and cancels in
          // the chunk's reverse cumsum to fp32 precision; under strong decay most of dG is
          // such pairs, and the fp32 factors would leave bf16-sized residues.
          typedef T t4r __attribute__((ext_vector_type(4)));
          const t4r qlr = *reinterpret_cast<const t4r*>(QLT + col * LDC + 16 * rt + 4 * grp);
          const t4r bklr = *reinterpret_cast<const t4r*>(BKLT + col * LDC + 16 * rt + 4 * grp);
          const t4r kilr = *reinterpret_cast<const t4r*>(KiLT + col * LDC + 16 * rt + 4 * grp);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = 16 * rt + 4 * grp + j;
            const float G = Gr[ci][rt][j];
            const float eGR = __expf(G - Rr), eRG = __expf(Rr - G), erG = __expf(g_last - G);
            const float kl = kv[ci][rt][j] * eGR;
            dG[rt][j] = to_f(qlr[j]) * aq[rt][j] + to_f(bklr[j]) * akd[rt][j] - to_f(kilr[j]) * ai[rt][j];
            const float dq_e = s.scale * eGR * aq[rt][j];
            const float dk_d = eGR * betas[row] * akd[rt][j], dk_i = eRG * ai[rt][j], dk_r = erG * ar[rt][j];
            dq4[j] = dq_e;
            dk4[j] = dk_d + dk_i + dk_r;
            if constexpr (GVA) {
              dqa[ci][rt][j] += dq_e;
              dka[ci][rt][j] += dk4[j];
            }
            dG[rt][j] -= kv[ci][rt][j] * dk_r;
            krd += kv[ci][rt][j] * dk_r;
            dbz[j] = kl * akd[rt][j];  // dbeta part 2: rowsum(kd o akd)
          }
          if constexpr (!GVA) {
            store_rows<T>(dqc, qs, 16 * rt, 16 * kt, dq4, lane, len);
            store_rows<T>(dkc, qs, 16 * rt, 16 * kt, dk4, lane, len);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) dbz_sum[rt][j] += row_allsum16(dbz[j]);
        }
        krd = col_allsum(krd);
        // dgam enters at the chunk's last valid row
        const int rl = len - 1;
        if (grp == (rl & 15) >> 2) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (rt == (rl >> 4) && j == (rl & 3)) dG[rt][j] += __expf(g_last) * rsum + krd;
        }
        col_suffix<RT>(dG, lane);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int j = 0; j < 4; ++j) dGk[ci][rt][j] = dG[rt][j];
      }
    }
    // dg leaves through LDS (the dO slot, dead after the products above) as whole rows:
    // 16-byte stores, consecutive lanes on consecutive columns.
    {
      constexpr int SR = Lay::SR;  // rows per pass
      constexpr int LDG = K + 4;
      float* stg = reinterpret_cast<float*>(smem + Lay::oDoT);
#pragma unroll
      for (int pass = 0; pass < C / SR; ++pass) {
        __syncthreads();
#pragma unroll
        for (int ci = 0; ci < NCT; ++ci) {
          const int kt = wave + ci * NW;
          if (kt < KT) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
              if (rt * 16 >= pass * SR && rt * 16 < (pass + 1) * SR) {
#pragma unroll
                for (int j = 0; j < 4; ++j) stg[(16 * rt + 4 * grp + j - pass * SR) * LDG + 16 * kt + n] = dGk[ci][rt][j];
              }
          }
        }
        __syncthreads();
        for (int i = tid; i < SR * K / 4; i += NTH) {
          const int r = i / (K / 4), c4 = (i % (K / 4)) * 4;
          const int row = pass * SR + r;
          // nontemporal: nothing later in the call reads dg, and full rows leave as whole
          // lines, so the marking keeps them from pushing the inputs that workgroups still
          // to come will read out of the L2 and the Infinity Cache without adding traffic
          // (the 8-byte row pieces of dq, dk and dv would leave as partial lines: plain
          // stores, merged in L2, for those)
          if (row < len) __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(stg + r * LDG + c4), reinterpret_cast<f32x4*>(dgc + row * gs + c4));
        }
      }
    }
    {
      // lane n of group grp writes row 16(n/4) + 4grp + n%4 (plain write, every row once)
      float v = 0.f;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int j = 0; j < 4; ++j) v = (n == 4 * rt + j) ? dbz_sum[rt][j] : v;
      if (n < 4 * RT) dbpart[NW * C + wave * C + 16 * (n >> 2) + 4 * grp + (n & 3)] = v;
    }
    __syncthreads();
    KDA_TS(2, 7);
    if (tid < len) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) acc += dbpart[w * C + tid];
#pragma unroll
      for (int w = 0; w < NW; ++w) acc += dbpart[NW * C + w * C + tid];
      if (s.beta_logits) acc *= betas[tid] * (1.f - betas[tid]);  // d sigmoid / d logit
      dbc[tid * s.HV] = acc;
    }
    __syncthreads();
  }

  KDA_TS(2, 8);
  if constexpr (!GVA) {
    KDA_TS(2, 9);
    return;
  }
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, grp = lane >> 4;
  const int len = geo.len;
#pragma unroll
  for (int ci = 0; ci < NACC; ++ci) {
    const int kt = wave + ci * NW;
    if (kt < KT) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        store_rows<T>(dqc, qs, 16 * rt, 16 * kt, f32x4{dqa[ci][rt][0], dqa[ci][rt][1], dqa[ci][rt][2], dqa[ci][rt][3]}, lane, len);
        store_rows<T>(dkc, qs, 16 * rt, 16 * kt, f32x4{dka[ci][rt][0], dka[ci][rt][1], dka[ci][rt][2], dka[ci][rt][3]}, lane, len);
      }
    }
  }
  KDA_TS(2, 9);
}

// W = Q'^T dO for the saved path (kda_chunk_bwd_saved): the tail of the prep kernel, with
// Q'^T read back from the forward's save in the scan's fragment order. One workgroup per
// (chunk, value head); dO^T staged in LDS; wave w owns the K rows 16w .. of W. It also pulls
// the chunk's saved kr, -w^T and e^gam into the caches (copies to a scratch LDS block that
// nothing reads): the reverse scan that follows is a chain of dependent steps whose operand
// copies otherwise come from HBM.
template <class T, int K, int V, int C>
__global__ __launch_bounds__(512) void bwd_w_kernel(Shape s, const T* __restrict__ dOp, SavedWs saved, BwdWs ws) {
  constexpr int NW = 8, RT = C / 16, KT = K / 16, VT = V / 16, NCV = (VT + NW - 1) / NW;
  constexpr int LDC = C + pad_of<T>();
  __shared__ __align__(16) T DoT[V * LDC];
  __shared__ __align__(16) unsigned char land[sizeof(T) == 2 ? NW * 1024 : 16];
  const int task = group_task(blockIdx.x, s.HV / s.H, s.NT * s.nhv);
  if (task < 0) return;
  const int c = task / s.nhv, h = s.hv0 + task % s.nhv;
  const Geo geo = chunk_geo(c, s.cu, s.choff, s.N, s.T, C);
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long ch = (long)c * s.HV + h;
  const int len = geo.len;
  if (len <= 0) return;
  const int vs = s.HV * V;
  const T* __restrict__ dOc = dOp + (geo.bos * s.HV + h) * V;
  typedef ScanFrag<K, V, C> SF;
  // this wave's A fragments of Q'^T (K tile `wave`), requested first
  bf16x8 af[sizeof(T) == 2 ? SF::CQ : 1];
  if constexpr (sizeof(T) == 2) {
    static_assert(KT == NW, "one K tile per wave");
    const bf16x8* src = reinterpret_cast<const bf16x8*>(saved.qpT) + ch * (SF::P2_ELEMS / 8) + lane;
#pragma unroll
    for (int q = 0; q < SF::CQ; ++q) af[q] = src[(wave * SF::CQ + q) * 64];
    // the scan's operands of this chunk-head: 1 KB blocks of kr and -w^T shared out over the
    // waves, and e^gam
    constexpr int NB1 = SF::P1_ELEMS / 512, NB2 = SF::P2_ELEMS / 512, PER = (NB1 + NB2 + NW - 1) / NW;
    const bf16* kr = reinterpret_cast<const bf16*>(saved.kr) + ch * SF::P1_ELEMS + 8 * lane;
    const bf16* nw = reinterpret_cast<const bf16*>(saved.nwT) + ch * SF::P2_ELEMS + 8 * lane;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int b = wave * PER + i;
      if (b < NB1) copy16_to_lds(kr + 512 * b, land + 1024 * wave);
      else if (b < NB1 + NB2) copy16_to_lds(nw + 512 * (b - NB1), land + 1024 * wave);
    }
    if (wave == 0) copy16_to_lds(saved.eg + ch * K + 4 * (lane % (K / 4)), land);
  }
  // dO^T (rows past the chunk's end as zero): row pieces moved to the column-owner layout
  ColTile<T, RT> td[NCV];
#pragma unroll
  for (int cv = 0; cv < NCV; ++cv) td[cv].load(dOc, vs, 16 * min(wave + cv * NW, VT - 1), lane, len);
#pragma unroll
  for (int cv = 0; cv < NCV; ++cv) {
    float x[RT][4];
    td[cv].get(x, lane, len);
    const int vt = wave + cv * NW;
    if (vt < VT) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        st4(DoT + (16 * vt + n) * LDC + 16 * rt + 4 * grp, f32x4{x[rt][0], x[rt][1], x[rt][2], x[rt][3]});
    }
  }
  __syncthreads();
  T* __restrict__ bcT = reinterpret_cast<T*>(ws.bcT) + ch * V * K;
  if constexpr (sizeof(T) == 2) {
    const int kt = wave;
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int q = 0; q < SF::CQ; ++q) {
        // B: dO rows in the fragment order's contraction order (32q + 4grp .. +3, then
        // 32q + 16 + 4grp .. +3) of column 16vt + n; the second half is absent when C = 16
        const bool pair2 = 2 * q + 1 < RT;
        const T* br = DoT + (16 * vt + n) * LDC + 32 * q + 4 * grp;
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(br);
        bf16x4 hi = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
        if (pair2) hi = *reinterpret_cast<const bf16x4*>(br + 16);
        const bf16x8 b = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        bf16x8 a = af[q];
        if (!pair2) {  // the fragment order pads C = 16 to a 32-wide step: unwritten there
#pragma unroll
          for (int i = 4; i < 8; ++i) a[i] = (bf16)0.0f;
        }
        acc = Mma<T>::mma(a, b, acc);
      }
      // column v = 16vt + n goes to its scan slice and lane
      const int v = 16 * vt + n;
      st4(bcT + SF::seed(ScanCols::slice(v), kt, KT, ScanCols::lane_col(v) + 16 * grp), acc);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the cache pulls have landed
  } else {
    const T* __restrict__ qps = reinterpret_cast<const T*>(saved.qpT) + ch * K * C;
    for (int e = tid; e < K * V; e += 64 * NW) {
      const int k = e / V, v = e % V;
      float acc = 0.f;
      for (int j = 0; j < C; ++j) acc += to_f(qps[k * C + j]) * to_f(DoT[v * LDC + j]);
      bcT[v * K + k] = from_f<T>(acc);
    }
  }
}

hipError_t launch_bwd_w(int dtype, int C, const Shape& s, const void* dO, const SavedWs& sv, const BwdWs& ws,
                        hipStream_t st) {
  if (s.NT == 0) return hipSuccess;
  const dim3 grid(group_grid(s.NT * s.nhv, s.HV / s.H)), block(512);
  if (dtype == 0)
    hipLaunchKernelGGL((bwd_w_kernel<float, 16, 16, 16>), grid, block, 0, st, s, static_cast<const float*>(dO), sv, ws);
  else if (C == 64)
    hipLaunchKernelGGL((bwd_w_kernel<bf16, 128, 128, 64>), grid, block, 0, st, s, static_cast<const bf16*>(dO), sv, ws);
  else
    hipLaunchKernelGGL((bwd_w_kernel<bf16, 128, 128, 16>), grid, block, 0, st, s, static_cast<const bf16*>(dO), sv, ws);
  return hipGetLastError();
}

template <class T, int K, int V, int C>
static hipError_t bwd_prep_t(const Shape& s, const void* q, const void* k, const float* g, const float* beta,
                             const void* inv, const void* dO, const BwdWs& ws, hipStream_t st) {
  if (s.NT == 0) return hipSuccess;
  const dim3 grid(group_grid(s.NT * s.nhv, s.HV / s.H)), block(64 * BwdPrepLds<T, K, V, C>::NW);
  if constexpr (sizeof(T) == 2) {
    if (scan_wq(1, s, V)) {
      hipLaunchKernelGGL((bwd_prep_kernel<T, K, V, C, true>), grid, block, 0, st, s, static_cast<const T*>(q),
                         static_cast<const T*>(k), g, beta, static_cast<const T*>(inv), static_cast<const T*>(dO), ws);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((bwd_prep_kernel<T, K, V, C, false>), grid, block, 0, st, s, static_cast<const T*>(q),
                     static_cast<const T*>(k), g, beta, static_cast<const T*>(inv), static_cast<const T*>(dO), ws);
  return hipGetLastError();
}

hipError_t launch_bwd_prep(int dtype, int C, const Shape& s, const void* q, const void* k, const float* g,
                           const float* beta, const void* inv, const void* dO, const BwdWs& ws, hipStream_t st) {
  if (dtype == 0) return bwd_prep_t<float, 16, 16, 16>(s, q, k, g, beta, inv, dO, ws, st);
  if (C == 64) return bwd_prep_t<bf16, 128, 128, 64>(s, q, k, g, beta, inv, dO, ws, st);
  return bwd_prep_t<bf16, 128, 128, 16>(s, q, k, g, beta, inv, dO, ws, st);
}

template <class T, int K, int V, int C>
static hipError_t bwd_grad_t(const Shape& s, const void* q, const void* k, const void* v, const float* g,
                             const float* beta, const void* states, const void* inv, const void* dO, const BwdWs& ws,
                             void* dq, void* dk, void* dv, float* dg, float* dbeta, hipStream_t st) {
  if (s.NT == 0) return hipSuccess;
  const dim3 grid(s.NT * (s.nhv / (s.HV / s.H))), block(64 * GradLds<T, K, V, C>::NW);
  if (s.HV > s.H) {
    hipLaunchKernelGGL((bwd_grad_kernel<T, K, V, C, true>), grid, block, 0, st, s, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), g, beta, static_cast<const T*>(states),
                       static_cast<const T*>(inv), static_cast<const T*>(dO), ws, static_cast<T*>(dq),
                       static_cast<T*>(dk), static_cast<T*>(dv), dg, dbeta);
  } else {
    hipLaunchKernelGGL((bwd_grad_kernel<T, K, V, C, false>), grid, block, 0, st, s, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), g, beta, static_cast<const T*>(states),
                       static_cast<const T*>(inv), static_cast<const T*>(dO), ws, static_cast<T*>(dq),
                       static_cast<T*>(dk), static_cast<T*>(dv), dg, dbeta);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_grad(int dtype, int C, const Shape& s, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, const void* states, const void* inv, const void* dO,
                           const BwdWs& ws, void* dq, void* dk, void* dv, float* dg, float* dbeta, hipStream_t st) {
  if (dtype == 0) return bwd_grad_t<float, 16, 16, 16>(s, q, k, v, g, beta, states, inv, dO, ws, dq, dk, dv, dg,
                                                       dbeta, st);
  if (C == 64)
    return bwd_grad_t<bf16, 128, 128, 64>(s, q, k, v, g, beta, states, inv, dO, ws, dq, dk, dv, dg, dbeta, st);
  return bwd_grad_t<bf16, 128, 128, 16>(s, q, k, v, g, beta, states, inv, dO, ws, dq, dk, dv, dg, dbeta, st);
}

}  // namespace kda
