// Forward chunk kernels of KDA for gfx950: the packed-sequence chunk table, the per-chunk
// preparation (gate cumsum, WY/UT inverse, w, u, kr) and the chunk output o.
//
// Chunk algebra (FlashKDA backward page, the forward workspace and the forward it
// differentiates; FLA chunk_kda_bwd page, recompute_w_u_fwd and chunk_gated_delta_rule_fwd_h):
// with G the chunk-local inclusive cumsum of g and gam = G at the chunk's last row,
//   kd = k e^G, ki = k e^-G, kr = k e^(gam-G), qd = scale q e^G,
//   INV = (I + strict_tril(diag(beta) kd ki^T))^-1,  w = INV diag(beta) kd,  u = INV diag(beta) v,
//   U = u - w S_in,  S_out = diag(e^gam) S_in + kr^T U,  o = qd S_in + tril(qd ki^T) U.
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

template <class T, int K, int V, int C>
struct FwdPrepLds {
  static constexpr int P = pad_of<T>();
  static constexpr int LDK = K + P, LDC = C + P, LDL = C + 4;
  static constexpr size_t oKd = 0;
  static constexpr size_t oKi = oKd + sizeof(T) * C * LDK;
  static constexpr size_t oBKdT = oKi + sizeof(T) * C * LDK;
  static constexpr size_t oBVT = oBKdT + sizeof(T) * K * LDC;
  static constexpr size_t oL = oBVT + sizeof(T) * V * LDC;
  static constexpr size_t oINV = oL + sizeof(float) * C * LDL;
  static constexpr size_t oBeta = oINV + sizeof(T) * C * LDC;
  static constexpr size_t total = oBeta + sizeof(float) * C;
};

// One workgroup per (chunk, value head).
template <class T, int K, int V, int C>
__global__ __launch_bounds__(256) void fwd_prep_kernel(Shape s, const T* __restrict__ kp, const T* __restrict__ vp,
                                                        const float* __restrict__ gp, const float* __restrict__ bp,
                                                        T* __restrict__ invp, FwdWs ws) {
  typedef FwdPrepLds<T, K, V, C> Lay;
  constexpr int NW = 4, RT = C / 16, KT = K / 16, VT = V / 16;
  constexpr int LDK = Lay::LDK, LDC = Lay::LDC, LDL = Lay::LDL;
  __shared__ __align__(16) unsigned char smem[Lay::total];
  T* Kd = reinterpret_cast<T*>(smem + Lay::oKd);
  T* Ki = reinterpret_cast<T*>(smem + Lay::oKi);
  T* BKdT = reinterpret_cast<T*>(smem + Lay::oBKdT);
  T* BVT = reinterpret_cast<T*>(smem + Lay::oBVT);
  float* Lf = reinterpret_cast<float*>(smem + Lay::oL);
  T* INVt = reinterpret_cast<T*>(smem + Lay::oINV);
  float* betas = reinterpret_cast<float*>(smem + Lay::oBeta);

  const int c = blockIdx.x, h = s.hv0 + blockIdx.y;
  const int hq = h / (s.HV / s.H);
  const Geo geo = chunk_geo(c, s.cu, s.choff, s.N, s.T, C);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, grp = lane >> 4;
  const long ch = (long)c * s.HV + h;
  const int len = geo.len;
  if (len <= 0) return;
  const int qs = s.H * K, gs = s.HV * K, vs = s.HV * V;
  const T* kc = kp + (geo.bos * s.H + hq) * K;
  const float* gc = gp + (geo.bos * s.HV + h) * K;
  const T* vc = vp + (geo.bos * s.HV + h) * V;
  const float* bc = bp + geo.bos * s.HV + h;

  if (tid < C) betas[tid] = tid < len ? bc[tid * s.HV] : 0.f;
  __syncthreads();

  for (int kt = wave; kt < KT; kt += NW) {
    const int col = 16 * kt + n;
    float G[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * rt + 4 * grp + j;
        G[rt][j] = row < len ? gc[row * gs + col] : 0.f;
      }
    const float gam = col_prefix<RT>(G, lane);  // the column total is gam
    T* __restrict__ krT = reinterpret_cast<T*>(ws.krT) + ch * (sizeof(T) == 2 ? ScanFrag<K, V, C>::P2_ELEMS : K * C);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 bk, kr4;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * rt + 4 * grp + j;
        const float kv = row < len ? to_f(kc[row * qs + col]) : 0.f;
        const float kd = kv * __expf(G[rt][j]);
        Kd[row * LDK + col] = from_f<T>(kd);
        Ki[row * LDK + col] = from_f<T>(kv * __expf(-G[rt][j]));
        bk[j] = betas[row] * kd;
        kr4[j] = kv * __expf(gam - G[rt][j]);
      }
      st4(BKdT + col * LDC + 16 * rt + 4 * grp, bk);
      if constexpr (sizeof(T) == 2) {
        st4(krT + ScanFrag<K, V, C>::p2(col, 16 * rt + 4 * grp), kr4);
      } else {
        st4(krT + col * C + 16 * rt + 4 * grp, kr4);
      }
    }
    if (grp == 0) ws.eg[ch * K + col] = __expf(gam);
  }
  for (int vt = wave; vt < VT; vt += NW) {
    const int col = 16 * vt + n;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 bv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * rt + 4 * grp + j;
        bv[j] = row < len ? betas[row] * to_f(vc[row * vs + col]) : 0.f;
      }
      st4(BVT + col * LDC + 16 * rt + 4 * grp, bv);
    }
  }
  __syncthreads();

  // L = strict_tril(diag(beta) kd ki^T), fp32.
  block_gemm<T, RT, RT, 1, NW, K>(
      Kd, LDK, 1 << 30, Ki, LDK, [](int mt, int nt0, int& kb, int& ke) { if (nt0 > mt) ke = 0; },
      [&](int, int mt, int nt0, f32x4(&acc)[1]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 16 * mt + 4 * grp + j, col = 16 * nt0 + n;
          Lf[row * LDL + col] = col < row ? betas[row] * acc[0][j] : 0.f;
        }
      }, wave, lane);
  __syncthreads();

  // INV = (I + L)^-1 by forward substitution in fp32, one thread per column:
  // X[i][col] = delta(i, col) - sum_{j<i} L[i][j] X[j][col].
  if (tid < C) {
    const int col = tid;
    float x[C];
    T* inv = invp + ch * C * C;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      float acc = i == col ? 1.f : 0.f;
      const float* Lrow = Lf + i * LDL;
#pragma unroll
      for (int j = 0; j < i; ++j) acc -= Lrow[j] * x[j];
      x[i] = acc;
      const T xt = from_f<T>(acc);
      inv[i * C + col] = xt;
      INVt[i * LDC + col] = xt;
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
  static constexpr size_t total = oBeta + sizeof(float) * C;
};

// o = qd S_in + tril(qd ki^T) U with U = INV diag(beta)(v - kd S_in); one workgroup per
// (chunk, value head).
template <class T, int K, int V, int C>
__global__ __launch_bounds__(256) void fwd_out_kernel(Shape s, const T* __restrict__ qp, const T* __restrict__ kp,
                                                       const T* __restrict__ vp, const float* __restrict__ gp,
                                                       const float* __restrict__ bp, const T* __restrict__ states,
                                                       const T* __restrict__ invp, T* __restrict__ op) {
  typedef FwdOutLds<T, K, V, C> Lay;
  constexpr int NW = 4, RT = C / 16, KT = K / 16, VT = V / 16;
  constexpr int LDK = Lay::LDK, LDC = Lay::LDC;
  __shared__ __align__(16) unsigned char smem[Lay::total];
  T* Qd = reinterpret_cast<T*>(smem + Lay::oQd);
  T* Kd = reinterpret_cast<T*>(smem + Lay::oKd);
  T* Ki = reinterpret_cast<T*>(smem + Lay::oKi);
  T* SinT = reinterpret_cast<T*>(smem + Lay::oSinT);
  T* INVt = reinterpret_cast<T*>(smem + Lay::oINV);
  T* VcT = reinterpret_cast<T*>(smem + Lay::oVcT);
  T* Mqk = reinterpret_cast<T*>(smem + Lay::oMqk);
  T* UT = reinterpret_cast<T*>(smem + Lay::oUT);
  float* betas = reinterpret_cast<float*>(smem + Lay::oBeta);

  const int c = blockIdx.x, h = s.hv0 + blockIdx.y;
  const int hq = h / (s.HV / s.H);
  const Geo geo = chunk_geo(c, s.cu, s.choff, s.N, s.T, C);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, grp = lane >> 4;
  const long ch = (long)c * s.HV + h;
  const int len = geo.len;
  if (len <= 0) return;
  const int qs = s.H * K, gs = s.HV * K, vs = s.HV * V;
  const T* qc = qp + (geo.bos * s.H + hq) * K;
  const T* kc = kp + (geo.bos * s.H + hq) * K;
  const float* gc = gp + (geo.bos * s.HV + h) * K;
  const T* vc = vp + (geo.bos * s.HV + h) * V;
  T* oc = op + (geo.bos * s.HV + h) * V;
  const float* bc = bp + geo.bos * s.HV + h;

  if (tid < C) betas[tid] = tid < len ? bc[tid * s.HV] : 0.f;
  for (int kt = wave; kt < KT; kt += NW) {
    const int col = 16 * kt + n;
    float G[RT][4];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * rt + 4 * grp + j;
        G[rt][j] = row < len ? gc[row * gs + col] : 0.f;
      }
    col_prefix<RT>(G, lane);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * rt + 4 * grp + j;
        const int off = row * qs + col;
        const float kv = row < len ? to_f(kc[off]) : 0.f;
        const float qv = row < len ? to_f(qc[off]) : 0.f;
        const float e = __expf(G[rt][j]);
        Qd[row * LDK + col] = from_f<T>(s.scale * qv * e);
        Kd[row * LDK + col] = from_f<T>(kv * e);
        Ki[row * LDK + col] = from_f<T>(kv * __expf(-G[rt][j]));
      }
  }
  const T* Sin = states + ch * K * V;
  for (int vt = wave; vt < VT; vt += NW) {
    const int col = 16 * vt + n;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      f32x4 s4;
#pragma unroll
      for (int j = 0; j < 4; ++j) s4[j] = to_f(Sin[(16 * kt + 4 * grp + j) * V + col]);
      st4(SinT + col * LDK + 16 * kt + 4 * grp, s4);
    }
  }
  for (int idx = tid; idx < C * C; idx += 256) {
    const int i = idx / C, j = idx % C;
    const float val = (i < len && j < len) ? to_f(invp[ch * C * C + idx]) : (i == j ? 1.f : 0.f);
    INVt[i * LDC + j] = from_f<T>(val);
  }
  __syncthreads();

  constexpr int BN = VT % 2 == 0 ? 2 : 1;
  // vcorr = diag(beta)(v - kd S_in), stored transposed.
  block_gemm<T, RT, VT, BN, NW, K>(Kd, LDK, 1 << 30, SinT, LDK, FullRange(),
                                   [&](int, int mt, int nt0, f32x4(&acc)[BN]) {
#pragma unroll
                                     for (int jb = 0; jb < BN; ++jb) {
                                       const int col = 16 * (nt0 + jb) + n;
                                       f32x4 vc4;
#pragma unroll
                                       for (int j = 0; j < 4; ++j) {
                                         const int row = 16 * mt + 4 * grp + j;
                                         const float vv =
                                             row < len ? to_f(vc[row * vs + col]) : 0.f;
                                         vc4[j] = betas[row] * (vv - acc[jb][j]);
                                       }
                                       st4(VcT + col * LDC + 16 * mt + 4 * grp, vc4);
                                     }
                                   }, wave, lane);
  // Mqk = tril(qd ki^T), row-major.
  block_gemm<T, RT, RT, 1, NW, K>(
      Qd, LDK, 1 << 30, Ki, LDK, [](int mt, int nt0, int& kb, int& ke) { if (nt0 > mt) ke = 0; },
      [&](int, int mt, int nt0, f32x4(&acc)[1]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = 16 * mt + 4 * grp + j, col = 16 * nt0 + n;
          Mqk[row * LDC + col] = from_f<T>(col <= row ? acc[0][j] : 0.f);
        }
      }, wave, lane);
  __syncthreads();
  // U = INV vcorr, stored transposed.
  block_gemm<T, RT, VT, BN, NW, C>(
      INVt, LDC, 1 << 30, VcT, LDC, [](int mt, int, int& kb, int& ke) { ke = min(C, round_up<T>(16 * (mt + 1))); },
      [&](int, int mt, int nt0, f32x4(&acc)[BN]) {
#pragma unroll
        for (int jb = 0; jb < BN; ++jb) st4(UT + (16 * (nt0 + jb) + n) * LDC + 16 * mt + 4 * grp, acc[jb]);
      }, wave, lane);
  __syncthreads();
  // o = qd S_in + Mqk U.
  block_gemm2<T, RT, VT, BN, NW, K, C>(
      Qd, LDK, SinT, LDK, FullRange(), Mqk, LDC, UT, LDC,
      [](int mt, int, int& kb, int& ke) { ke = min(C, round_up<T>(16 * (mt + 1))); },
      [&](int, int mt, int nt0, f32x4(&acc)[BN]) {
#pragma unroll
        for (int jb = 0; jb < BN; ++jb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = 16 * mt + 4 * grp + j, col = 16 * (nt0 + jb) + n;
            if (row < len) oc[row * vs + col] = from_f<T>(acc[jb][j]);
          }
      }, wave, lane);
}

hipError_t launch_chunk_offsets(const int32_t* cu, int N, int C, int32_t* choff, hipStream_t st) {
  hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(1024), 0, st, cu, N, C, choff);
  return hipGetLastError();
}

template <class T, int K, int V, int C>
static hipError_t fwd_prep_t(const Shape& s, const void* k, const void* v, const float* g, const float* beta,
                             void* inv, const FwdWs& ws, hipStream_t st) {
  if (s.NT == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_prep_kernel<T, K, V, C>), dim3(s.NT, s.nhv), dim3(256), 0, st, s,
                     static_cast<const T*>(k), static_cast<const T*>(v), g, beta, static_cast<T*>(inv), ws);
  return hipGetLastError();
}

hipError_t launch_fwd_prep(int dtype, int C, const Shape& s, const void* k, const void* v, const float* g,
                           const float* beta, void* inv, const FwdWs& ws, hipStream_t st) {
  if (dtype == 0) return fwd_prep_t<float, 16, 16, 16>(s, k, v, g, beta, inv, ws, st);
  if (C == 64) return fwd_prep_t<bf16, 128, 128, 64>(s, k, v, g, beta, inv, ws, st);
  return fwd_prep_t<bf16, 128, 128, 16>(s, k, v, g, beta, inv, ws, st);
}

template <class T, int K, int V, int C>
static hipError_t fwd_out_t(const Shape& s, const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const void* states, const void* inv, void* o, hipStream_t st) {
  if (s.NT == 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_out_kernel<T, K, V, C>), dim3(s.NT, s.nhv), dim3(256), 0, st, s,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), g, beta,
                     static_cast<const T*>(states), static_cast<const T*>(inv), static_cast<T*>(o));
  return hipGetLastError();
}

hipError_t launch_fwd_out(int dtype, int C, const Shape& s, const void* q, const void* k, const void* v,
                          const float* g, const float* beta, const void* states, const void* inv, void* o,
                          hipStream_t st) {
  if (dtype == 0) return fwd_out_t<float, 16, 16, 16>(s, q, k, v, g, beta, states, inv, o, st);
  if (C == 64) return fwd_out_t<bf16, 128, 128, 64>(s, q, k, v, g, beta, states, inv, o, st);
  return fwd_out_t<bf16, 128, 128, 16>(s, q, k, v, g, beta, states, inv, o, st);
}

}  // namespace kda
