// Forward chunk kernels of KDA for gfx950: the packed-sequence chunk table, the per-chunk
// preparation (gate cumsum, WY/UT inverse, w, u, kr) and the chunk output o.
//
// Chunk algebra (FlashKDA backward page, the forward workspace and the forward it
// differentiates; FLA chunk_kda_bwd page, recompute_w_u_fwd and chunk_gated_delta_rule_fwd_h):
// with G the chunk-local inclusive cumsum of g and gam = G at the chunk's last row,
//   kd = k e^G, ki = k e^-G, kr = k e^(gam-G), qd = scale q e^G,
//   INV = (I + strict_tril(diag(beta) kd ki^T))^-1,  w = INV diag(beta) kd,  u = INV diag(beta) v,
//   U = u - w S_in,  S_out = diag(e^gam) S_in + kr^T U,  o = qd S_in + tril(qd ki^T) U.
// The triangles kd ki^T and qd ki^T are formed from referenced rows (k e^(G - R), k e^(R - G),
// scale q e^(G - R)): R = 0 for the columns whose |G| stays small, else the cumsum at the first
// row of each 16-row block, so that every operand stays in range whatever the gates
// (choose_refs, tri_tiles in kda_device.h).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// choff[0] = 0, choff[n+1] = choff[n] + ceil(len_n / C).
__global__ __launch_bounds__(1024) void chunk_offsets_kernel(const int32_t* __restrict__ cu, int N, int C,
                                                             int32_t* __restrict__ choff) {
  __shared__ int buf[1024];
  __shared__ int carry;
  const int t = threadIdx.x;
  if (t == 0) {
    carry = 0;
    choff[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < N; base += 1024) {
    const int i = base + t;
    int val = 0;
    if (i < N) val = (cu[i + 1] - cu[i] + C - 1) / C;
    buf[t] = val;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int add = t >= off ? buf[t - off] : 0;
      __syncthreads();
      buf[t] += add;
      __syncthreads();
    }
    if (i < N) choff[i + 1] = carry + buf[t];
    __syncthreads();
    if (t == 1023) carry += buf[1023];
    __syncthreads();
  }
}

// LDS plan of the forward prep kernel (two workgroups per CU). Later buffers overlay
// earlier ones that a barrier has retired:
//   KL, KiL (until L)                -> X (fp32 inverse) and INV (bf16 / fp32 operand)
//   L (fp32, until the inverse)      -> diag(beta) v^T
//   diag(beta) kd^T (whole kernel); R of each 16-row block per channel (until L)
template <class T, int K, int V, int C>
struct FwdPrepLds {
  static constexpr int P = pad_of<T>();
  static constexpr int LDK = K + P, LDC = C + P, LDL = C + 4;
  static constexpr size_t mx(size_t a, size_t b) { return a > b ? a : b; }
  static constexpr size_t oKd = 0;
  static constexpr size_t oKi = oKd + sizeof(T) * C * LDK;
  static constexpr size_t oX = 0;
  static constexpr size_t oINV = oX + sizeof(float) * C * LDL;
  static constexpr size_t endA = mx(oKi + sizeof(T) * C * LDK, oINV + sizeof(T) * C * LDC);
  static constexpr size_t oBKdT = endA;
  static constexpr size_t oL = oBKdT + sizeof(T) * K * LDC;
  static constexpr size_t oBVT = oL;
  static constexpr size_t oBeta = oL + mx(sizeof(float) * C * LDL, sizeof(T) * V * LDC);
  static constexpr size_t oD = oBeta + sizeof(float) * C;  // ratios of consecutive block references
  static constexpr size_t oFlag = oD + sizeof(float) * (C / 16 - 1) * K;  // per-wave reference mode
  static constexpr size_t total = oFlag + sizeof(int) * 8;
  static_assert(total <= 80 * 1024 || C > 64, "two workgroups per CU");
};

// (I + L)^-1 of a unit lower-triangular C x C matrix (L strictly lower, fp32 in LDS with row
// stride LDL), blocked by 16: each diagonal block is inverted by forward substitution (one
// wave, a lane per column), then the blocks below the diagonal follow one block diagonal at
// a time, X_ij = -X_ii * sum_{k=j..i-1} L_ik X_kj, as fp32 16x16x4 MFMA products (a block per
// wave). X (fp32, same stride) receives the inverse; its upper triangle is zero. Whole
// workgroup; begins and ends with every wave's LDS writes visible.
template <int C, int NW>
__device__ __forceinline__ void unit_lower_inverse(const float* __restrict__ L, float* __restrict__ X, int ldl,
                                                   int wave, int lane) {
  constexpr int RT = C / 16;
  static_assert(NW >= RT, "a wave per diagonal block");
  const int n = lane & 15, grp = lane >> 4;
  // diagonal blocks; the rest of the upper triangle is cleared by the same waves
  if (wave < RT) {
    const int b = 16 * wave;
    if (lane < 16) {
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = i == lane ? 1.f : 0.f;
        const float* Lrow = L + (b + i) * ldl + b;
#pragma unroll
        for (int j = 0; j < i; ++j) acc -= Lrow[j] * x[j];
        x[i] = acc;
        X[(b + i) * ldl + b + lane] = acc;
      }
    }
    // blocks above the diagonal in this block row are zero
    for (int cb = wave + 1; cb < RT; ++cb)
#pragma unroll
      for (int j = 0; j < 4; ++j) X[(b + 4 * grp + j) * ldl + 16 * cb + n] = 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int d = 1; d < RT; ++d) {
    const int i = d + wave, j = wave;  // block (i, j) on block diagonal d
    if (i < RT) {
      // S = sum_k L_ik X_kj (standard contraction order)
      f32x4 S = zero4();
      for (int k = j; k < i; ++k)
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4)
          S = __builtin_amdgcn_mfma_f32_16x16x4f32(L[(16 * i + n) * ldl + 16 * k + k0 + grp],
                                                   X[(16 * k + k0 + grp) * ldl + 16 * j + n], S, 0, 0, 0);
      // X_ij = -X_ii S, with the contraction index permuted so that S's accumulator values are
      // the B operand as held: step s covers contraction indices 4g + s (lane group g)
      f32x4 D = zero4();
#pragma unroll
      for (int st = 0; st < 4; ++st)
        D = __builtin_amdgcn_mfma_f32_16x16x4f32(X[(16 * i + n) * ldl + 16 * i + 4 * grp + st], S[st], D, 0, 0, 0);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) X[(16 * i + 4 * grp + jj) * ldl + 16 * j + n] = -D[jj];
    }
    __syncthreads();
  }
}

// One workgroup per (chunk, value head); 512 threads, two workgroups per CU. SAVE: also writes
// the backward's kr, -w^T (the reverse scan's fragment orders) and e^gam to `saved`.
template <class T, int K, int V, int C, bool SAVE>
__global__ __launch_bounds__(512, 2) void fwd_prep_kernel(Shape s, const T* __restrict__ kp, const T* __restrict__ vp,
                                                           const float* __restrict__ gp, const float* __restrict__ bp,
                                                           T* __restrict__ invp, FwdWs ws, SavedWs saved) {
  typedef FwdPrepLds<T, K, V, C> Lay;
  constexpr int NW = 8, RT = C / 16, KT = K / 16, VT = V / 16;
  static_assert(NW <= 8, "one reference-mode flag per wave");
  constexpr int NCK = (KT + NW - 1) / NW, NCV = (VT + NW - 1) / NW;
  constexpr int LDK = Lay::LDK, LDC = Lay::LDC, LDL = Lay::LDL;
  __shared__ __align__(16) unsigned char smem[Lay::total];
  T* KL = reinterpret_cast<T*>(smem + Lay::oKd);   // k e^(G - R), row-major
  T* KiL = reinterpret_cast<T*>(smem + Lay::oKi);  // k e^(R - G), row-major
  float* D = reinterpret_cast<float*>(smem + Lay::oD);
  int* wflag = reinterpret_cast<int*>(smem + Lay::oFlag);
  float* Xf = reinterpret_cast<float*>(smem + Lay::oX);
  T* INVt = reinterpret_cast<T*>(smem + Lay::oINV);
  T* BKdT = reinterpret_cast<T*>(smem + Lay::oBKdT);
  float* Lf = reinterpret_cast<float*>(smem + Lay::oL);
  T* BVT = reinterpret_cast<T*>(smem + Lay::oBVT);
  float* betas = reinterpret_cast<float*>(smem + Lay::oBeta);

  // heads of one chunk are neighbouring workgroups (a q/k group's on one XCD), chunks in
  // reverse order: the first chunks, which the forward scan reads first, are the last ones
  // written
  const int task = group_task(blockIdx.x, s.HV / s.H, s.NT * s.nhv);
  if (task < 0) return;
  const int c = s.NT - 1 - task / s.nhv, h = s.hv0 + task % s.nhv;
  const int hq = h / (s.HV / s.H);
  const Geo geo = chunk_geo(c, s.cu, s.choff, s.N, s.T, C);
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long ch = (long)c * s.HV + h;
  const int len = geo.len;
  if (len <= 0) return;
  const int qs = s.H * K, gs = s.HV * K, vs = s.HV * V;
  const T* __restrict__ kc = kp + (geo.bos * s.H + hq) * K;
  const float* __restrict__ gc = gp + (geo.bos * s.HV + h) * K;
  const T* __restrict__ vc = vp + (geo.bos * s.HV + h) * V;
  const float* __restrict__ bc = bp + geo.bos * s.HV + h;

  // ---- g and k loads, issued before any use (row pieces, moved to the column-owner layout by
  // the tiles' MFMA transposes); v follows once they have arrived
  const float beta_raw = beta_of(bc[min(tid % C, len - 1) * s.HV], s.beta_logits);
  ColTile<float, RT> tg[NCK];
  ColTile<T, RT> tk[NCK], tv[NCV];
#pragma unroll
  for (int ci = 0; ci < NCK; ++ci) {
    const int kt = min(wave + ci * NW, KT - 1);
    tg[ci].load(gc, gs, 16 * kt, lane, len);
    tk[ci].load(kc, qs, 16 * kt, lane, len);
  }
  if (tid < C) betas[tid] = tid < len ? beta_raw : 0.f;
  __syncthreads();

  // ---- gate cumsum; block-referenced keys (row-major), diag(beta) kd^T, kr (scan fragment
  // order), e^gam
  T* __restrict__ krT = reinterpret_cast<T*>(ws.krT) + ch * (sizeof(T) == 2 ? ScanFrag<K, V, C>::P2_ELEMS : K * C);
  bool strong_w = false;  // this wave's columns take block references
#pragma unroll
  for (int ci = 0; ci < NCK; ++ci) {
    const int kt = wave + ci * NW;
    if (kt < KT) {
      float G[RT][4], kv[RT][4];
      tg[ci].get(G, lane, len);
      tk[ci].get(kv, lane, len);
      const int col = 16 * kt + n;
      const float gam = col_prefix<RT>(G, lane);  // the column total is gam
      float R[RT];
      strong_w = choose_refs<RT>(G, R, lane) || strong_w;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 kd4, kl4, ki4, bk, kr4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 16 * rt + 4 * grp + j;
          kd4[j] = kv[rt][j] * __expf(G[rt][j]);
          kl4[j] = kv[rt][j] * __expf(G[rt][j] - R[rt]);
          ki4[j] = kv[rt][j] * __expf(R[rt] - G[rt][j]);
          bk[j] = betas[row] * kd4[j];
          kr4[j] = kv[rt][j] * __expf(gam - G[rt][j]);
        }
        if (grp == 0 && rt + 1 < RT) D[rt * K + col] = __expf(R[rt + 1] - R[rt]);
        store_rows<T>(KL, LDK, 16 * rt, 16 * kt, kl4, lane, 1 << 30);
        store_rows<T>(KiL, LDK, 16 * rt, 16 * kt, ki4, lane, 1 << 30);
        st4(BKdT + col * LDC + 16 * rt + 4 * grp, bk);
        if constexpr (sizeof(T) == 2) {
          st4(krT + ScanFrag<K, V, C>::p2(col, 16 * rt + 4 * grp), kr4);
        } else {
          st4(krT + col * C + 16 * rt + 4 * grp, kr4);
        }
        if constexpr (SAVE) {
          // kr for the reverse scan, [C][K] in its fragment order (row pieces: this lane row
          // 16rt + n, columns 16kt + 4grp ..)
          T* __restrict__ krs = reinterpret_cast<T*>(saved.kr) + ch * C * K;
          if constexpr (sizeof(T) == 2) {
            st4(krs + ScanFrag<K, V, C>::p1(16 * rt + n, 16 * kt + 4 * grp), to_rows_bf16(kr4[0], kr4[1], kr4[2], kr4[3], lane));
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) krs[(16 * rt + 4 * grp + j) * K + col] = kr4[j];
          }
        }
      }
      if (grp == 0) {
        ws.eg[ch * K + col] = __expf(gam);
        if constexpr (SAVE) saved.eg[ch * K + col] = __expf(gam);
      }
    }
  }
  if (lane == 0) wflag[wave] = strong_w;
  // v (first used once INV is known): issued once g and k have arrived, so that the opening
  // burst of the two workgroups of a CU is smaller and v lands during L and the inverse
#pragma unroll
  for (int cv = 0; cv < NCV; ++cv) tv[cv].load(vc, vs, 16 * min(wave + cv * NW, VT - 1), lane, len);
  __syncthreads();

  // ---- L = strict_tril(diag(beta) kd ki^T), fp32, from the block-referenced keys
  tri_tiles<T, RT, NW, K, false>(
      KL, LDK, KiL, LDK, D, K, any_flag<NW>(wflag),
      [&](int mt, int nt0, f32x4 acc) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 16 * mt + 4 * grp + j, col = 16 * nt0 + n;
          Lf[row * LDL + col] = col < row ? betas[row] * acc[j] : 0.f;
        }
      }, wave, lane);
  __syncthreads();  // KL, KiL retired (the epilogue also wrote the upper blocks as zero)

  // ---- INV = (I + L)^-1 (fp32, into the Kd/Ki region)
  unit_lower_inverse<C, NW>(Lf, Xf, LDL, wave, lane);

  // ---- INV to global memory and as the MFMA operand; diag(beta) v^T over L
  float bv[NCV][RT][4];  // diag(beta) v in the column-owner layout
#pragma unroll
  for (int cv = 0; cv < NCV; ++cv) {
    tv[cv].get(bv[cv], lane, len);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[cv][rt][j] *= betas[16 * rt + 4 * grp + j];
  }
  T* __restrict__ inv = invp + ch * C * C;
  for (int i = tid; i < C * C / 4; i += 64 * NW) {
    const int row = (4 * i) / C, col = (4 * i) % C;
    const f32x4 x4 = *reinterpret_cast<const f32x4*>(Xf + row * LDL + col);
    st4(inv + row * C + col, x4);
    st4(INVt + row * LDC + col, x4);
  }
#pragma unroll
  for (int cv = 0; cv < NCV; ++cv) {
    const int vt = wave + cv * NW;
    if (vt < VT) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        st4(BVT + (16 * vt + n) * LDC + 16 * rt + 4 * grp, f32x4{bv[cv][rt][0], bv[cv][rt][1], bv[cv][rt][2], bv[cv][rt][3]});
    }
  }
  __syncthreads();

  // -w, computed as its transpose w^T = (diag(beta) kd)^T INV^T so each lane stores 4
  // consecutive k of one row c.
  T* negw = reinterpret_cast<T*>(ws.negw) + ch * C * K;
  block_gemm<T, KT, RT, 1, NW, C>(
      BKdT, LDC, 1 << 30, INVt, LDC,
      [](int, int nt0, int& kb, int& ke) { ke = min(C, round_up<T>(16 * (nt0 + 1))); },
      [&](int, int mt, int nt0, f32x4(&acc)[1]) {
        if constexpr (sizeof(T) == 2) {
          st4(negw + ScanFrag<K, V, C>::p1(16 * nt0 + n, 16 * mt + 4 * grp), -acc[0]);
        } else {
          st4(negw + (16 * nt0 + n) * K + 16 * mt + 4 * grp, -acc[0]);
        }
        if constexpr (SAVE) {
          // -w^T for the reverse scan, [K][C] in its fragment order: the tile moved to the row
          // layout (this lane: k = 16mt + n, c = 16nt0 + 4grp ..)
          T* __restrict__ nws = reinterpret_cast<T*>(saved.nwT) + ch * (sizeof(T) == 2 ? ScanFrag<K, V, C>::P2_ELEMS : K * C);
          if constexpr (sizeof(T) == 2) {
            st4(nws + ScanFrag<K, V, C>::p2(16 * mt + n, 16 * nt0 + 4 * grp),
                to_rows_bf16(-acc[0][0], -acc[0][1], -acc[0][2], -acc[0][3], lane));
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) nws[(16 * mt + 4 * grp + j) * C + 16 * nt0 + n] = -acc[0][j];
          }
        }
      }, wave, lane);
  // u = INV diag(beta) v, stored transposed [V][C].
  T* uT = reinterpret_cast<T*>(ws.uT) + ch * V * C;
  constexpr int BN = VT % 2 == 0 ? 2 : 1;
  block_gemm<T, RT, VT, BN, NW, C>(
      INVt, LDC, 1 << 30, BVT, LDC,
      [](int mt, int, int& kb, int& ke) { ke = min(C, round_up<T>(16 * (mt + 1))); },
      [&](int, int mt, int nt0, f32x4(&acc)[BN]) {
#pragma unroll
        for (int jb = 0; jb < BN; ++jb)
          if constexpr (sizeof(T) == 2) {
            st4(uT + ScanFrag<K, V, C>::seed(nt0 + jb, mt, RT, lane), acc[jb]);
          } else {
            st4(uT + (16 * (nt0 + jb) + n) * C + 16 * mt + 4 * grp, acc[jb]);
          }
      }, wave, lane);
}

template <class T, int K, int V, int C>
struct FwdOutLds {
  static constexpr int P = pad_of<T>();
  static constexpr int LDK = K + P, LDC = C + P;
  static constexpr size_t oQd = 0;
  static constexpr size_t oKd = oQd + sizeof(T) * C * LDK;
  static constexpr size_t oKi = oKd + sizeof(T) * C * LDK;
  static constexpr size_t oSinT = oKi + sizeof(T) * C * LDK;
  static constexpr size_t oINV = oSinT + sizeof(T) * V * LDK;
  static constexpr size_t oVcT = oINV + sizeof(T) * C * LDC;
  static constexpr size_t oMqk = oVcT + sizeof(T) * V * LDC;
  static constexpr size_t oUT = oMqk + sizeof(T) * C * LDC;
  static constexpr size_t oBeta = oUT + sizeof(T) * V * LDC;
  static constexpr size_t oQL = oBeta + sizeof(float) * C;
  static constexpr size_t oD = oQL + sizeof(T) * C * LDK;  // ratios of consecutive block references
  static constexpr size_t oFlag = oD + sizeof(float) * (C / 16 - 1) * K;  // per-wave reference mode
  static constexpr size_t total = oFlag + sizeof(int) * 8;
  static_assert(total <= 160 * 1024, "output kernel exceeds the LDS of one CU");
};

// o = qd S_in + tril(qd ki^T) U with U = INV diag(beta)(v - kd S_in); one workgroup per
// (chunk, value head), 512 threads. g, q, k, S_in and INV are loaded before any use, v once
// g, q and k have arrived: g, q, k and v as row pieces moved to the column-owner layout by
// MFMA transposes, S_in and INV as 16-byte pieces (bf16: 16 x 32 blocks, written transposed
// into LDS by MFMA transposes). SAVE: also writes the backward's Q'^T = (qd - Mqk w)^T to
// `saved` (the reverse scan's fragment order), from qd and Mqk in LDS and the -w^T that the
// prep kernel saved.
template <class T, int K, int V, int C, bool SAVE>
__global__ __launch_bounds__(512) void fwd_out_kernel(Shape s, const T* __restrict__ qp, const T* __restrict__ kp,
                                                       const T* __restrict__ vp, const float* __restrict__ gp,
                                                       const float* __restrict__ bp, const T* __restrict__ states,
                                                       const T* __restrict__ invp, T* __restrict__ op, SavedWs saved) {
  typedef FwdOutLds<T, K, V, C> Lay;
  typedef T vecT __attribute__((ext_vector_type(16 / sizeof(T))));
  typedef T t4 __attribute__((ext_vector_type(4)));
  constexpr int NW = 8, NTH = 64 * NW, RT = C / 16, KT = K / 16, VT = V / 16;
  static_assert(NW <= 8, "one reference-mode flag per wave");
  constexpr int NCK = (KT + NW - 1) / NW;
  constexpr int VEC = 16 / (int)sizeof(T);
  constexpr int LDK = Lay::LDK, LDC = Lay::LDC;
  constexpr int BN = VT % 2 == 0 ? 2 : 1;
  constexpr int NIT1 = (RT * (VT / BN) + NW - 1) / NW;
  __shared__ __align__(16) unsigned char smem[Lay::total];
  T* Qd = reinterpret_cast<T*>(smem + Lay::oQd);
  T* Kd = reinterpret_cast<T*>(smem + Lay::oKd);
  T* KiL = reinterpret_cast<T*>(smem + Lay::oKi);  // k e^(R - G)
  T* QL = reinterpret_cast<T*>(smem + Lay::oQL);   // scale q e^(G - R)
  float* D = reinterpret_cast<float*>(smem + Lay::oD);
  int* wflag = reinterpret_cast<int*>(smem + Lay::oFlag);
  T* SinT = reinterpret_cast<T*>(smem + Lay::oSinT);
  T* INVt = reinterpret_cast<T*>(smem + Lay::oINV);
  T* VcT = reinterpret_cast<T*>(smem + Lay::oVcT);
  T* Mqk = reinterpret_cast<T*>(smem + Lay::oMqk);
  T* UT = reinterpret_cast<T*>(smem + Lay::oUT);
  float* betas = reinterpret_cast<float*>(smem + Lay::oBeta);

  // heads of one chunk are neighbouring workgroups (a q/k group's on one XCD), chunks in
  // reverse order: the last chunks' states, the last ones the forward scan wrote, are read
  // first
  const int task = group_task(blockIdx.x, s.HV / s.H, s.NT * s.nhv);
  if (task < 0) return;
  const int c = s.NT - 1 - task / s.nhv, h = s.hv0 + task % s.nhv;
  const int hq = h / (s.HV / s.H);
  const Geo geo = chunk_geo(c, s.cu, s.choff, s.N, s.T, C);
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long ch = (long)c * s.HV + h;
  const int len = geo.len;
  if (len <= 0) return;
  const int qs = s.H * K, gs = s.HV * K, vs = s.HV * V;
  const T* __restrict__ qc = qp + (geo.bos * s.H + hq) * K;
  const T* __restrict__ kc = kp + (geo.bos * s.H + hq) * K;
  const float* __restrict__ gc = gp + (geo.bos * s.HV + h) * K;
  const T* __restrict__ vc = vp + (geo.bos * s.HV + h) * V;
  T* __restrict__ oc = op + (geo.bos * s.HV + h) * V;
  const float* __restrict__ bc = bp + geo.bos * s.HV + h;
  const T* __restrict__ Sin = states + ch * K * V;
  const T* __restrict__ invc = invp + ch * C * C;

  // ---- loads
  const float beta_raw = beta_of(bc[min(tid % C, len - 1) * s.HV], s.beta_logits);
  ColTile<float, RT> tg[NCK];
  ColTile<T, RT> tq[NCK], tk[NCK];
#pragma unroll
  for (int ci = 0; ci < NCK; ++ci) {
    const int kt = min(wave + ci * NW, KT - 1);
    tg[ci].load(gc, gs, 16 * kt, lane, len);
    tq[ci].load(qc, qs, 16 * kt, lane, len);
    tk[ci].load(kc, qs, 16 * kt, lane, len);
  }
  // bf16 (BLK): piece i of this lane lies in 16 x 32 block b = wave + i NW of the matrix
  // (blocks down the rows first): row 16(b % row tiles) + n, columns 32(b / row tiles) + 8grp
  // .. +7. Otherwise piece i of thread tid covers VEC elements of a row (S_in: lanes on
  // consecutive rows).
  constexpr bool BLK = sizeof(T) == 2 && C % 32 == 0 && V % 32 == 0 && K % 16 == 0;
  constexpr int NBS = KT * (V / 32), NBI = RT * (C / 32);
  auto blk_rc = [&](int b, int rtiles, int& r, int& cc) {
    r = 16 * (b % rtiles) + n;
    cc = 32 * (b / rtiles) + 8 * grp;
  };
  constexpr int NSV = (K * V / VEC + NTH - 1) / NTH;
  vecT sv[NSV];
#pragma unroll
  for (int i = 0; i < NSV; ++i) {
    if constexpr (BLK) {
      int r, cc;
      blk_rc(min(wave + i * NW, NBS - 1), KT, r, cc);
      sv[i] = *reinterpret_cast<const vecT*>(Sin + r * V + cc);
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
      int r, cc;
      blk_rc(min(wave + i * NW, NBI - 1), RT, r, cc);
      iv[i] = *reinterpret_cast<const vecT*>(invc + r * C + cc);
    } else {
      iv[i] = *reinterpret_cast<const vecT*>(invc + min(tid + i * NTH, C * C / VEC - 1) * VEC);
    }
  }
  if (tid < C) betas[tid] = tid < len ? beta_raw : 0.f;

  // ---- gate cumsum; qd, kd and the block-referenced q, k row-major; S_in^T; INV
  bool strong_w = false;  // this wave's columns take block references
#pragma unroll
  for (int ci = 0; ci < NCK; ++ci) {
    const int kt = wave + ci * NW;
    if (kt < KT) {
      float G[RT][4], qv[RT][4], kv[RT][4];
      tg[ci].get(G, lane, len);
      tq[ci].get(qv, lane, len);
      tk[ci].get(kv, lane, len);
      col_prefix<RT>(G, lane);
      float R[RT];
      strong_w = choose_refs<RT>(G, R, lane) || strong_w;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 q4, ql4, kd4, ki4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float e = __expf(G[rt][j]);
          q4[j] = s.scale * qv[rt][j] * e;
          ql4[j] = s.scale * qv[rt][j] * __expf(G[rt][j] - R[rt]);
          kd4[j] = kv[rt][j] * e;
          ki4[j] = kv[rt][j] * __expf(R[rt] - G[rt][j]);
        }
        if (grp == 0 && rt + 1 < RT) D[rt * K + 16 * kt + n] = __expf(R[rt + 1] - R[rt]);
        store_rows<T>(Qd, LDK, 16 * rt, 16 * kt, q4, lane, 1 << 30);
        store_rows<T>(QL, LDK, 16 * rt, 16 * kt, ql4, lane, 1 << 30);
        store_rows<T>(Kd, LDK, 16 * rt, 16 * kt, kd4, lane, 1 << 30);
        store_rows<T>(KiL, LDK, 16 * rt, 16 * kt, ki4, lane, 1 << 30);
      }
    }
  }
  if (lane == 0) wflag[wave] = strong_w;
  // v at the places of the C x V accumulator tiles this wave owns in the block walk of the
  // products below (RT x VT tiles in blocks of 1 x BN), first used after the barrier below:
  // issued once g, q and k have arrived, so that the opening burst of every CU is smaller and
  // v lands during the stores below
  ColTile<T, 1> tv[NIT1][BN];
#pragma unroll
  for (int it = 0; it < NIT1; ++it) {
    const int blk = min(wave + it * NW, RT * (VT / BN) - 1);
    const int mt = blk / (VT / BN), nt0 = (blk % (VT / BN)) * BN;
#pragma unroll
    for (int jb = 0; jb < BN; ++jb) tv[it][jb].load(vc, vs, 16 * (nt0 + jb), lane, len, 16 * mt);
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
#pragma unroll
  for (int i = 0; i < NIV; ++i) {
    int r, c0;
    bool ok;
    if constexpr (BLK) {
      const int b = wave + i * NW;
      ok = b < NBI;
      blk_rc(b, RT, r, c0);
    } else {
      const int pid = tid + i * NTH;
      ok = pid < C * C / VEC;
      r = (pid * VEC) / C;
      c0 = (pid * VEC) % C;
    }
    if (ok) {
      vecT m;
#pragma unroll
      for (int t = 0; t < VEC; ++t) m[t] = (r < len && c0 + t < len) ? iv[i][t] : from_f<T>(r == c0 + t ? 1.f : 0.f);
      if constexpr (sizeof(T) == 2) {
        st_2x8(INVt + r * LDC + c0, m);
      } else {
#pragma unroll
        for (int t = 0; t < VEC; ++t) INVt[r * LDC + c0 + t] = m[t];
      }
    }
  }
  __syncthreads();
  t4 vraw[NIT1][BN];
#pragma unroll
  for (int it = 0; it < NIT1; ++it) {
    const int blk = min(wave + it * NW, RT * (VT / BN) - 1);
    const int mt = blk / (VT / BN);
#pragma unroll
    for (int jb = 0; jb < BN; ++jb) {
      float x[1][4];
      tv[it][jb].get(x, lane, len, 16 * mt);
#pragma unroll
      for (int j = 0; j < 4; ++j) vraw[it][jb][j] = from_f<T>(x[0][j]);
    }
  }

  // ---- vcorr = diag(beta)(v - kd S_in), stored transposed; Mqk = tril(qd ki^T), row-major
  block_gemm<T, RT, VT, BN, NW, K>(Kd, LDK, 1 << 30, SinT, LDK, FullRange(),
                                   [&](int it, int mt, int nt0, f32x4(&acc)[BN]) {
#pragma unroll
                                     for (int jb = 0; jb < BN; ++jb) {
                                       const int col = 16 * (nt0 + jb) + n;
                                       f32x4 vc4;
#pragma unroll
                                       for (int j = 0; j < 4; ++j)
                                         vc4[j] = betas[16 * mt + 4 * grp + j] * (to_f(vraw[it][jb][j]) - acc[jb][j]);
                                       st4(VcT + col * LDC + 16 * mt + 4 * grp, vc4);
                                     }
                                   }, wave, lane);
  tri_tiles<T, RT, NW, K>(
      QL, LDK, KiL, LDK, D, K, any_flag<NW>(wflag),
      [&](int mt, int nt0, f32x4 acc) {
        f32x4 m4;
#pragma unroll
        for (int j = 0; j < 4; ++j) m4[j] = (16 * nt0 + n <= 16 * mt + 4 * grp + j) ? acc[j] : 0.f;
        store_rows<T>(Mqk, LDC, 16 * mt, 16 * nt0, m4, lane, 1 << 30);
      }, wave, lane);
  __syncthreads();
  // SAVE, bf16: the saved -w^T fragments of this wave's K column tile (16 x 32 steps of the
  // scan's fragment order, which are the B fragments of -w), requested here to land during
  // the products below
  typedef ScanFrag<K, V, C> SF;
  bf16x8 nwf[SAVE && sizeof(T) == 2 ? SF::CQ : 1];
  if constexpr (SAVE && sizeof(T) == 2) {
    static_assert(SF::KT == NW, "one K column tile per wave");
    const bf16x8* src = reinterpret_cast<const bf16x8*>(saved.nwT) + ch * (SF::P2_ELEMS / 8) + lane;
#pragma unroll
    for (int q = 0; q < SF::CQ; ++q) nwf[q] = src[(wave * SF::CQ + q) * 64];
  }
  // ---- U = INV vcorr, stored transposed
  block_gemm<T, RT, VT, BN, NW, C>(
      INVt, LDC, 1 << 30, VcT, LDC, [](int mt, int, int& kb, int& ke) { ke = min(C, round_up<T>(16 * (mt + 1))); },
      [&](int, int mt, int nt0, f32x4(&acc)[BN]) {
#pragma unroll
        for (int jb = 0; jb < BN; ++jb) st4(UT + (16 * (nt0 + jb) + n) * LDC + 16 * mt + 4 * grp, acc[jb]);
      }, wave, lane);
  __syncthreads();
  // ---- o = qd S_in + Mqk U, stored as row pieces
  block_gemm2<T, RT, VT, BN, NW, K, C>(
      Qd, LDK, SinT, LDK, FullRange(), Mqk, LDC, UT, LDC,
      [](int mt, int, int& kb, int& ke) { ke = min(C, round_up<T>(16 * (mt + 1))); },
      [&](int, int mt, int nt0, f32x4(&acc)[BN]) {
#pragma unroll
        for (int jb = 0; jb < BN; ++jb) store_rows<T>(oc, vs, 16 * mt, 16 * (nt0 + jb), acc[jb], lane, len);
      }, wave, lane);
  if constexpr (SAVE) {
    // Q' = qd + Mqk (-w) (Qd and Mqk are still in LDS: the products above only read them),
    // stored transposed in the scan's K x C fragment order
    if constexpr (sizeof(T) == 2) {
      T* __restrict__ qps = reinterpret_cast<T*>(saved.qpT) + ch * SF::P2_ELEMS;
      const int kt = wave;
#pragma unroll
      for (int mt = 0; mt < RT; ++mt) {
        f32x4 acc = zero4();
#pragma unroll
        for (int q = 0; q < SF::CQ; ++q) {
          // A: Mqk rows 16mt + n, columns in the fragment order's contraction order (32q + 4grp
          // .. +3, then 32q + 16 + 4grp .. +3); the second half is absent when C = 16
          const bool pair2 = 2 * q + 1 < RT;
          const T* mr = Mqk + (16 * mt + n) * LDC + 32 * q + 4 * grp;
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(mr);
          bf16x4 hi = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
          if (pair2) hi = *reinterpret_cast<const bf16x4*>(mr + 16);
          const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          bf16x8 b = nwf[q];
          if (!pair2) {  // the fragment order pads C = 16 to a 32-wide step: unwritten there
#pragma unroll
            for (int i = 4; i < 8; ++i) b[i] = (bf16)0.0f;
          }
          acc = Mma<T>::mma(a, b, acc);
        }
        f32x4 qp4;
#pragma unroll
        for (int j = 0; j < 4; ++j) qp4[j] = to_f(Qd[(16 * mt + 4 * grp + j) * LDK + 16 * kt + n]) + acc[j];
        st4(qps + SF::p2(16 * kt + n, 16 * mt + 4 * grp), qp4);
      }
    } else {
      const T* __restrict__ nws = reinterpret_cast<const T*>(saved.nwT) + ch * K * C;
      T* __restrict__ qps = reinterpret_cast<T*>(saved.qpT) + ch * K * C;
      for (int e = tid; e < C * K; e += NTH) {
        const int r = e / K, k = e % K;
        float acc = to_f(Qd[r * LDK + k]);
        for (int j = 0; j < C; ++j) acc += to_f(Mqk[r * LDC + j]) * to_f(nws[k * C + j]);
        qps[k * C + r] = from_f<T>(acc);
      }
    }
  }
}

hipError_t launch_chunk_offsets(const int32_t* cu, int N, int C, int32_t* choff, hipStream_t st) {
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(1024), 0, st, cu, N, C, choff);
  return hipGetLastError();
}

template <class T, int K, int V, int C>
static hipError_t fwd_prep_t(const Shape& s, const void* k, const void* v, const float* g, const float* beta,
                             void* inv, const FwdWs& ws, hipStream_t st, const SavedWs* sv) {
  if (s.NT == 0) return hipSuccess;
  const dim3 grid(group_grid(s.NT * s.nhv, s.HV / s.H)), block(512);
  if (sv != nullptr)
    hipLaunchKernelGGL((fwd_prep_kernel<T, K, V, C, true>), grid, block, 0, st, s, static_cast<const T*>(k),
                       static_cast<const T*>(v), g, beta, static_cast<T*>(inv), ws, *sv);
  else
    hipLaunchKernelGGL((fwd_prep_kernel<T, K, V, C, false>), grid, block, 0, st, s, static_cast<const T*>(k),
                       static_cast<const T*>(v), g, beta, static_cast<T*>(inv), ws, SavedWs{});
  return hipGetLastError();
}

hipError_t launch_fwd_prep(int dtype, int C, const Shape& s, const void* k, const void* v, const float* g,
                           const float* beta, void* inv, const FwdWs& ws, hipStream_t st, const SavedWs* sv) {
  if (dtype == 0) return fwd_prep_t<float, 16, 16, 16>(s, k, v, g, beta, inv, ws, st, sv);
  if (C == 64) return fwd_prep_t<bf16, 128, 128, 64>(s, k, v, g, beta, inv, ws, st, sv);
  return fwd_prep_t<bf16, 128, 128, 16>(s, k, v, g, beta, inv, ws, st, sv);
}

template <class T, int K, int V, int C>
static hipError_t fwd_out_t(const Shape& s, const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const void* states, const void* inv, void* o, hipStream_t st,
                            const SavedWs* sv) {
  if (s.NT == 0) return hipSuccess;
  const dim3 grid(group_grid(s.NT * s.nhv, s.HV / s.H)), block(512);
  if (sv != nullptr)
    hipLaunchKernelGGL((fwd_out_kernel<T, K, V, C, true>), grid, block, 0, st, s, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), g, beta, static_cast<const T*>(states),
                       static_cast<const T*>(inv), static_cast<T*>(o), *sv);
  else
    hipLaunchKernelGGL((fwd_out_kernel<T, K, V, C, false>), grid, block, 0, st, s, static_cast<const T*>(q),
                       static_cast<const T*>(k), static_cast<const T*>(v), g, beta, static_cast<const T*>(states),
                       static_cast<const T*>(inv), static_cast<T*>(o), SavedWs{});
  return hipGetLastError();
}

hipError_t launch_fwd_out(int dtype, int C, const Shape& s, const void* q, const void* k, const void* v,
                          const float* g, const float* beta, const void* states, const void* inv, void* o,
                          hipStream_t st, const SavedWs* sv) {
  if (dtype == 0) return fwd_out_t<float, 16, 16, 16>(s, q, k, v, g, beta, states, inv, o, st, sv);
  if (C == 64) return fwd_out_t<bf16, 128, 128, 64>(s, q, k, v, g, beta, states, inv, o, st, sv);
  return fwd_out_t<bf16, 128, 128, 16>(s, q, k, v, g, beta, states, inv, o, st, sv);
}

}  // namespace kda
