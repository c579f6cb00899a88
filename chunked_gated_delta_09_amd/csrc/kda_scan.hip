// Sequential chunk scans of KDA for gfx950. The fp32 path (small K, V, C) reads its
// operands in plain row-major order; the bf16 path reads them in fragment order.
//
// Both directions are one affine step per chunk on a K x V fp32 matrix X:
//   Y    = Z + P1 X                 (C x V, contraction over K)
//   X'   = diag(e^gam) X + W + P2 Y (K x V, contraction over C)
// Forward (FLA chunk_gated_delta_rule_fwd_h; FlashKDA page, the state update
// S_out = diag(e^gam) S_in + kr^T U): X = S, P1 = -w, Z = u, P2 = kr^T, W = 0, so Y = U and
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


// bf16 path. The per-chunk operands P1, P2 (shared by every column slice of a (sequence,
// head)) and e^gam are stored in fragment order (ScanFrag): each is a run of 1 KB wave
// blocks. A workgroup holds NC column slices of one (sequence, head), one compute wave per
// slice, plus a copy wave that streams the shared operands of chunk i+2 into a three-slot
// LDS ring (global_load_lds, 16 bytes per lane, no registers) while chunk i is computed, and
// waits for chunk i+1's copies to land before the barrier that opens step i+1 (a further
// wave that touched the lines of later chunks into L2 ahead of the copies cost more than it
// gave: with ~32 workgroups per XCD its lines were evicted before use, doubling the fetches
// of the grouped-head workloads). All waves meet at one barrier per chunk step. The compute waves read the fragments from
// LDS (contiguous 16-byte reads per lane, issued well ahead of their MFMAs); their own
// slice's seed tiles (W or Z) come through the ring too when a workgroup holds at most 4
// slices, and otherwise from global memory one step ahead into a register double buffer.
// The shared operands are pulled once per workgroup instead of once per slice (a CU moves
// only ~50 GB/s from L2); with one slice per workgroup the compute wave's own dependency
// chain (two MFMA products and the state update) then sets the step time.
//
// Backward direction: a column slice covers the columns ScanCols::col(vt, n) (not 16
// consecutive ones), and the per-chunk dS leaves exactly as this wave holds it, 4 values
// per lane and row tile in seed order (one 8-byte store per row tile); the gradient kernel
// transposes it, and the column choice makes the transposed values of two slices one
// contiguous B fragment.

// Ring slot layout, in 1 KB blocks: P1 fragments, P2 fragments, e^gam, then either (WQ) the
// Q'^T fragments (P2's layout) and the dO rows of the slices' 32-column groups (C rows x 64
// bytes per group: the columns of slices 2m and 2m + 1 are the value columns 32m .. 32m + 31),
// or (SEED_DMA) the seed tiles of the NC slices.
template <int K, int V, int C, bool FWD, int NC>
struct ScanRing {
  typedef ScanFrag<K, V, C> F;
  // backward with 4 or more slices per workgroup (scan_wq): each slice forms its W = Q'^T dO
  static constexpr bool WQ = !FWD && NC >= 4;
  static constexpr int NB1 = F::CT * F::KP, NB2 = F::KT * F::CQ;  // 1 KB blocks of P1, P2
  static constexpr int OE = NB1 + NB2, O3 = OE + 1;                 // e^gam block, first Q'^T block
  static constexpr int NB3 = WQ ? NB2 : 0;
  static constexpr int NPAIR = (NC + 1) / 2, DKB = C / 16;          // dO: groups, 1 KB blocks per group
  static constexpr int OS = O3 + NB3;                               // first seed / dO block
  static constexpr int SROWS = FWD ? F::CT : F::KT;                 // 16-row seed tiles per slice
  static constexpr bool SEED_DMA = !WQ && NC <= 4 && SROWS % 2 == 0;  // seeds through the ring
  static constexpr int SKB = SROWS / 2;                             // 1 KB blocks per slice's seeds
  static constexpr int NL = OS + (SEED_DMA ? NC * SKB : 0) + (WQ ? NPAIR * DKB : 0);  // copies per chunk
  static constexpr int SLOT = NL * 1024;
  static constexpr int R = 3 * SLOT <= 160 * 1024 ? 3 : 2;  // ring slots (the LDS of one CU)
  static constexpr int LEAD = R - 1;                         // chunks copied ahead of the step
  static_assert(LEAD == 1 || NL <= 63, "the copy wave's wait count must fit vmcnt");
  static_assert(K % 4 == 0 && K * 4 <= 1024, "e^gam fits one block");
};

template <int K, int V, int C, bool FWD, int NC>
__global__ __launch_bounds__(64 * (NC + 1)) void scan_bf16_kernel(Shape s, const bf16* __restrict__ P1,
                                                                  const bf16* __restrict__ P2, const bf16* __restrict__ Zs,
                                                                  const bf16* __restrict__ Ws, const float* __restrict__ eg,
                                                                  const bf16* __restrict__ X0, bf16* __restrict__ Xout,
                                                                  bf16* __restrict__ Yout, float* __restrict__ Xfin,
                                                                  const bf16* __restrict__ dO) {
  typedef ScanFrag<K, V, C> F;
  typedef ScanRing<K, V, C, FWD, NC> RG;
  typedef Mma<bf16> M;
  typedef short s4 __attribute__((ext_vector_type(4)));
  constexpr int KT = F::KT, CT = F::CT, KP = F::KP, CQ = F::CQ, VT = V / 16;
  static_assert(KT % 2 == 0, "the bf16 scan pairs row tiles of X");
  static_assert(VT % NC == 0, "a workgroup holds whole slices");
  constexpr int NG = VT / NC;  // workgroups per (sequence, head)
  // explicit read-ahead schedule of the ring (needs the registers of at most two waves per
  // SIMD)
  constexpr bool PIPE = NC <= 4;
  __shared__ __align__(16) unsigned char ring[RG::R * RG::SLOT];
  // Workgroups are dealt round-robin to the 8 XCDs by linear id, so ids i, i+8, i+16, ...
  // share an XCD (and its L2). The NG workgroups of one (sequence, head) get ids of one
  // residue class mod 8: their shared per-chunk operands are fetched from HBM once per XCD.
  const int wid = blockIdx.x;
  const int xcd = wid % 8, r = wid / 8;
  const int pair = (r / NG) * 8 + xcd;  // (sequence, head) index
  const int vt0 = (r % NG) * NC;
  if (pair >= s.N * s.nhv) return;
  const int h = s.hv0 + pair % s.nhv, nseq = pair / s.nhv;
  const int lane = threadIdx.x & 63, n = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int c0, nc;
  seq_range(nseq, s.cu, s.choff, s.T, C, c0, nc);
  if (c0 + nc > s.NT) nc = max(0, s.NT - c0);
  auto chunk_of = [&](int ii) { return FWD ? c0 + ii : c0 + nc - 1 - ii; };

  if (wave == NC) {
    // copy wave: chunk index clamped to the last one, so every step issues exactly NL
    // copies and the wait count below is exact
    long sbos = (long)nseq * s.T;  // first token of the sequence, and its length
    int slen = s.T;
    if (s.cu != nullptr) {
      sbos = s.cu[nseq];
      slen = s.cu[nseq + 1] - s.cu[nseq];
    }
    auto copy = [&](int ii) {
      const long ch = (long)chunk_of(min(ii, nc - 1)) * s.HV + h;
      unsigned char* slot = ring + (ii % RG::R) * RG::SLOT;
      const bf16* p1 = P1 + ch * F::P1_ELEMS + 8 * lane;
#pragma unroll
      for (int b = 0; b < RG::NB1; ++b) copy16_to_lds(p1 + 512 * b, slot + 1024 * b);
      const bf16* p2 = P2 + ch * F::P2_ELEMS + 8 * lane;
#pragma unroll
      for (int b = 0; b < RG::NB2; ++b)
        copy16_to_lds(p2 + 512 * b, slot + 1024 * (RG::NB1 + b));
      copy16_to_lds(eg + ch * K + 4 * (lane % (K / 4)), slot + 1024 * RG::OE);
      if constexpr (RG::WQ) {
        const bf16* p3 = Ws + ch * F::P2_ELEMS + 8 * lane;  // Q'^T in the W buffer
#pragma unroll
        for (int b = 0; b < RG::NB3; ++b) copy16_to_lds(p3 + 512 * b, slot + 1024 * (RG::O3 + b));
        // dO rows of the chunk (rows past its end repeat its last row: Q' is zero there),
        // lane: row 16 b + lane / 4, columns 8 (lane % 4) .. +7 of the group
        const int lc = nc - 1 - min(ii, nc - 1);
        const long bos = sbos + (long)lc * C;
        const int len = min(C, slen - lc * C);
        const bf16* d0 = dO + (bos * s.HV + h) * V + 32 * (vt0 >> 1) + 8 * (lane & 3);
#pragma unroll
        for (int pp = 0; pp < RG::NPAIR; ++pp)
#pragma unroll
          for (int b = 0; b < RG::DKB; ++b)
            copy16_to_lds(d0 + (long)min(16 * b + (lane >> 2), len - 1) * s.HV * V + 32 * pp,
                          slot + 1024 * (RG::OS + pp * RG::DKB + b));
      }
      if constexpr (RG::SEED_DMA) {
        const bf16* sd = (FWD ? Zs + ch * C * V : Ws + ch * K * V) + 8 * lane;
#pragma unroll
        for (int w = 0; w < NC; ++w)
#pragma unroll
          for (int b = 0; b < RG::SKB; ++b)
            copy16_to_lds(sd + F::seed(vt0 + w, 0, RG::SROWS, 0) + 512 * b, slot + 1024 * (RG::OS + w * RG::SKB + b));
      }
    };
    // Chunk j is copied into slot j % R during step j - LEAD, lands before the barrier that
    // opens step j, and is read during that step.
    if (nc > 0) {
#pragma unroll
      for (int j = 0; j < RG::LEAD; ++j) copy(j);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(RG::NL * (RG::LEAD - 1)) : "memory");  // chunk 0 landed
    }
    for (int ii = 0; ii < nc; ++ii) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      // slot (ii + LEAD) % R was last read during step ii - 1
      copy(ii + RG::LEAD);
      // chunk ii + 1 has landed (only the copies of later chunks may still be in flight)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(RG::NL * (RG::LEAD - 1)) : "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }
  // ---- compute wave: slice vt of this (sequence, head)
  const int vt = vt0 + wave;
  const int vcol = FWD ? 16 * vt + n : ScanCols::col(vt, n);
  struct Seed {  // this slice's seed tiles of one chunk: W (backward) or Z (forward)
    bf16x4 t[FWD ? CT : KT];
  };
  auto load_seed = [&](int ii, Seed& o) {
    if constexpr (RG::SEED_DMA || RG::WQ) return;  // read from the ring at its step instead
    const long ch = (long)chunk_of(min(ii, nc - 1)) * s.HV + h;
    if constexpr (FWD) {
#pragma unroll
      for (int m = 0; m < CT; ++m) o.t[m] = *reinterpret_cast<const bf16x4*>(Zs + ch * C * V + F::seed(vt, m, CT, lane));
    } else {
#pragma unroll
      for (int t = 0; t < KT; ++t) o.t[t] = *reinterpret_cast<const bf16x4*>(Ws + ch * K * V + F::seed(vt, t, KT, lane));
    }
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

  // One chunk step with this slice's seed tiles `cur`; the next step's go into `nxt`.
  auto step = [&](int ii, const Seed& cur, Seed& nxt) {
    // This wave's reads of the ring are complete before the barrier, after which the copy
    // wave may refill a slot. The barrier is a plain one: the ring is written only by the
    // copy wave, which waits for its own copies, and this wave's stores and seed loads may
    // stay in flight across it.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if constexpr (!RG::SEED_DMA) {
      load_seed(ii + 1, nxt);
      // keep the seed loads here, a whole step ahead of their use (the scheduler would
      // otherwise sink them towards the end of the step)
      __builtin_amdgcn_sched_barrier(0);
    }
    const long ch = (long)chunk_of(ii) * s.HV + h;
    const unsigned char* slot = ring + (ii % RG::R) * RG::SLOT;
    const bf16x8* a1 = reinterpret_cast<const bf16x8*>(slot) + lane;
    const bf16x8* a2 = reinterpret_cast<const bf16x8*>(slot + 1024 * RG::NB1) + lane;
    const bf16x8* a3 = reinterpret_cast<const bf16x8*>(slot + 1024 * RG::O3) + lane;
    // WQ: this lane's row piece of dO tile m (row 16m + n, slice columns 4grp .. +3: bytes
    // 16grp + 8(vt % 2) of the group's 64-byte row) at dslot + 1024 m
    const unsigned char* dslot = slot + 1024 * (RG::OS + ((vt >> 1) - (vt0 >> 1)) * RG::DKB) + 64 * n + 16 * grp + 8 * (vt & 1);
    const float* eslot = reinterpret_cast<const float*>(slot + 1024 * RG::OE);
    const bf16x4* sslot = reinterpret_cast<const bf16x4*>(slot + 1024 * (RG::OS + wave * RG::SKB)) + lane;

    // With PIPE the ring is read in this program order -- forward: seed, P1 fragments,
    // e^gam, P2 fragments; backward: P1 fragments, e^gam, seed or (WQ) dO pieces and Q'^T
    // fragments, P2 fragments -- and the schedule at the end of the step issues each read well
    // ahead of its use. Without PIPE the reads stay at their uses and the compiler schedules
    // them.
    bf16x8 f1[PIPE ? CT : 1][KP], f2[PIPE ? KT : 1][CQ], f3[PIPE && RG::WQ ? KT : 1][CQ];
    s4 dr[PIPE && RG::WQ ? CT : 1];
    f32x4 ev[PIPE ? KT : 1];
    bf16x4 sd[RG::SEED_DMA ? RG::SROWS : 1];
    auto read_seed = [&]() {
      if constexpr (RG::SEED_DMA) {
#pragma unroll
        for (int i = 0; i < RG::SROWS; ++i) sd[i] = sslot[64 * i];
      }
    };
    if constexpr (PIPE) {
      if constexpr (FWD) read_seed();
#pragma unroll
      for (int m = 0; m < CT; ++m)
#pragma unroll
        for (int p = 0; p < KP; ++p) f1[m][p] = a1[(m * KP + p) * 64];
#pragma unroll
      for (int t = 0; t < KT; ++t) ev[t] = *reinterpret_cast<const f32x4*>(eslot + 16 * t + 4 * grp);
      if constexpr (!FWD) read_seed();
      if constexpr (RG::WQ) {
#pragma unroll
        for (int m = 0; m < CT; ++m) dr[m] = *reinterpret_cast<const s4*>(dslot + 1024 * m);
#pragma unroll
        for (int q = 0; q < CQ; ++q)
#pragma unroll
          for (int t = 0; t < KT; ++t) f3[t][q] = a3[(t * CQ + q) * 64];
      }
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int q = 0; q < CQ; ++q) f2[t][q] = a2[(t * CQ + q) * 64];
    } else {
      read_seed();
    }
    auto F1 = [&](int m, int p) { if constexpr (PIPE) return f1[m][p]; else return a1[(m * KP + p) * 64]; };
    auto F2 = [&](int t, int q) { if constexpr (PIPE) return f2[t][q]; else return a2[(t * CQ + q) * 64]; };
    auto F3 = [&](int t, int q) {
      if constexpr (PIPE && RG::WQ) return f3[t][q]; else return a3[(t * CQ + q) * 64];
    };
    auto DR = [&](int m) {
      if constexpr (PIPE && RG::WQ) return dr[m]; else return *reinterpret_cast<const s4*>(dslot + 1024 * m);
    };
    auto EV = [&](int t) {
      if constexpr (PIPE) return ev[t]; else return *reinterpret_cast<const f32x4*>(eslot + 16 * t + 4 * grp);
    };
    auto SD = [&](int i) { if constexpr (RG::SEED_DMA) return sd[i]; else return cur.t[i]; };

    bf16x8 bx[KP];
#pragma unroll
    for (int p = 0; p < KP; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bx[p][i] = (bf16)X[2 * p][i];
        bx[p][4 + i] = (bf16)X[2 * p + 1][i];
      }
    if constexpr (FWD && NC <= 2) {
      // S_in row-major: each 16 x 16 tile moved to the row layout by an MFMA against the
      // identity (lane: row 16t + n, columns 16vt + 4grp ..), one 8-byte store per tile. With
      // 4 or more slices per workgroup 2-byte column stores measured faster (workload B=4,
      // T=4096, HV=32: forward 795 vs 803 us) and with 8 the registers are not there.
      bf16* xo = Xout + ch * K * V;
#pragma unroll
      for (int t = 0; t < KT; ++t)
        st4(xo + (16 * t + n) * V + 16 * vt + 4 * grp, to_rows_bf16(X[t][0], X[t][1], X[t][2], X[t][3], lane));
    } else if constexpr (FWD) {
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
        const bf16x4 z = SD(m);
        Y[m] = f32x4{(float)z[0], (float)z[1], (float)z[2], (float)z[3]};
      } else {
        Y[m] = zero4();
      }
    }
#pragma unroll
    for (int p = 0; p < KP; ++p)
#pragma unroll
      for (int m = 0; m < CT; ++m) Y[m] = M::mma(F1(m, p), bx[p], Y[m]);
    if constexpr (!FWD) {
      // (kr dS)^T in the slices' lane-major order (64 lanes x 8 bytes per tile m, contiguous),
      // as the gradient kernel reads it
#pragma unroll
      for (int m = 0; m < CT; ++m) st4(Yout + ch * V * C + F::seed(vt, m, CT, lane), Y[m]);
    }

    // X = diag(e^gam) X + W + P2 Y, accumulated in place (X itself is no longer needed: Y
    // used its bf16 copy)
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      X[t] = EV(t) * X[t];
      if constexpr (!FWD && !RG::WQ) {
        const bf16x4 w = SD(t);
        X[t] += f32x4{(float)w[0], (float)w[1], (float)w[2], (float)w[3]};
      }
    }
    if constexpr (RG::WQ) {
      // W = Q'^T dO: the dO tiles, moved to the column-owner layout by MFMAs against the
      // identity, are B fragments (rows 32q + 4grp + i in slots 0-3, 32q + 16 + 4grp + i in
      // slots 4-7: the order of P2's fragments)
#pragma unroll
      for (int q = 0; q < CQ; ++q) {
        const bool pair2 = 2 * q + 1 < CT;
        const f32x4 lo = rows_to_cols_bf16(DR(2 * q), lane);
        f32x4 hi = zero4();
        if (pair2) hi = rows_to_cols_bf16(DR(pair2 ? 2 * q + 1 : 0), lane);
        bf16x8 b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          b[i] = (bf16)lo[i];
          b[4 + i] = (bf16)hi[i];
        }
#pragma unroll
        for (int t = 0; t < KT; ++t) {
          bf16x8 a = F3(t, q);
          if (!pair2) {
#pragma unroll
            for (int i = 4; i < 8; ++i) a[i] = (bf16)0.0f;
          }
          X[t] = M::mma(a, b, X[t]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < CQ; ++q) {
      const bool pair2 = 2 * q + 1 < CT;
      bf16x8 b;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[i] = (bf16)Y[2 * q][i];
        b[4 + i] = pair2 ? (bf16)Y[pair2 ? 2 * q + 1 : 2 * q][i] : (bf16)0.0f;
      }
#pragma unroll
      for (int t = 0; t < KT; ++t) {
        bf16x8 a = F2(t, q);
        if (!pair2) {
#pragma unroll
          for (int i = 4; i < 8; ++i) a[i] = (bf16)0.0f;
        }
        X[t] = M::mma(a, b, X[t]);
      }
    }
    if constexpr (PIPE) {
      // the first UP ring reads (at least everything the first product needs), then one
      // further read after each MFMA: every read is issued at least 8 MFMAs before its use
      constexpr int NR = CT * KP + KT + KT * CQ + (RG::SEED_DMA ? RG::SROWS : 0) + (RG::WQ ? CT + RG::NB3 : 0);
      constexpr int NMMA = CT * KP + KT * CQ + (RG::WQ ? CT + KT * CQ : 0);
      constexpr int PRE = CT * KP + (FWD && RG::SEED_DMA ? RG::SROWS : 0);
      constexpr int UP = PRE > NR - NMMA + 8 ? PRE : NR - NMMA + 8;
      static_assert(UP <= NR && NR - UP <= NMMA, "the interleave covers every ring read");
      __builtin_amdgcn_sched_group_barrier(0x100, UP, 0);
#pragma unroll
      for (int i = 0; i < NR - UP; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NMMA - (NR - UP), 0);
    }
  };

  if (nc > 0) {
    Seed sa, sb;
    load_seed(0, sa);
    for (int ii = 0; ii < nc; ii += 2) {
      step(ii, sa, sb);
      if (ii + 1 < nc) step(ii + 1, sb, sa);
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
                         const float* eg, const void* X0, void* Xout, void* Yout, float* Xfin, const void* dO,
                         hipStream_t st) {
  if (s.N == 0) return hipSuccess;
  if constexpr (sizeof(T) == 2) {
    // Slices per workgroup (scan_slices): the fewest that keep the grid within about one
    // workgroup per CU (the ring takes ~100-150 KB of LDS); more slices share one pull of the
    // operands.
    const int pairs = s.N * s.nhv, nc = scan_slices(s, V);
    const int grid = ((pairs + 7) / 8) * 8 * (V / 16 / nc);
    auto go = [&](auto kern, int ncw) {
      hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * (ncw + 1)), 0, st, s, static_cast<const bf16*>(P1),
                         static_cast<const bf16*>(P2), static_cast<const bf16*>(Zi), static_cast<const bf16*>(Wi), eg,
                         static_cast<const bf16*>(X0), static_cast<bf16*>(Xout), static_cast<bf16*>(Yout), Xfin,
                         static_cast<const bf16*>(dO));
    };
    if (nc == 1) go(scan_bf16_kernel<K, V, C, FWD, 1>, 1);
    else if (nc == 2) go(scan_bf16_kernel<K, V, C, FWD, 2>, 2);
    else if (nc == 4) go(scan_bf16_kernel<K, V, C, FWD, 4>, 4);
    else go(scan_bf16_kernel<K, V, C, FWD, 8>, 8);
  } else {
    hipLaunchKernelGGL((scan_kernel<T, K, V, C, FWD>), dim3(V / 16, s.nhv, s.N), dim3(64), 0, st, s,
                       static_cast<const T*>(P1), static_cast<const T*>(P2), static_cast<const T*>(Zi),
                       static_cast<const T*>(Wi), eg, static_cast<const T*>(X0), static_cast<T*>(Xout),
                       static_cast<T*>(Yout), Xfin);
  }
  return hipGetLastError();
}

// The per-chunk state gradients the reverse scan leaves in the backward workspace, written
// out as plain [NT, HV, K, V] fp32 (an inspection aid for stage checks; the backward itself
// never calls it). bf16 path: each chunk-head's gradient is in the scan's seed order, slice
// ScanCols::slice(v) holding column v at lane column ScanCols::lane_col(v).
template <class T, int K, int V, int C>
__global__ __launch_bounds__(256) void dstates_out_kernel(const T* __restrict__ dS, float* __restrict__ out) {
  const long base = (long)blockIdx.x * K * V;
  for (int e = threadIdx.x; e < K * V; e += 256) {
    const int k = e / V, v = e % V;
    float x;
    if constexpr (sizeof(T) == 2) {
      const int lane = ScanCols::lane_col(v) + 16 * ((k & 15) >> 2);
      x = (float)dS[base + ScanFrag<K, V, C>::seed(ScanCols::slice(v), k >> 4, K / 16, lane) + (k & 3)];
    } else {
      x = dS[base + e];
    }
    out[base + e] = x;
  }
}

hipError_t launch_dstates_out(int dtype, int C, const Shape& s, const BwdWs& ws, float* out, hipStream_t st) {
  const long nch = (long)s.NT * s.HV;
  if (nch == 0) return hipSuccess;
  if (dtype == 0)
    hipLaunchKernelGGL((dstates_out_kernel<float, 16, 16, 16>), dim3(nch), dim3(256), 0, st,
                       static_cast<const float*>(ws.dS), out);
  else if (C == 64)
    hipLaunchKernelGGL((dstates_out_kernel<bf16, 128, 128, 64>), dim3(nch), dim3(256), 0, st,
                       static_cast<const bf16*>(ws.dS), out);
  else
    hipLaunchKernelGGL((dstates_out_kernel<bf16, 128, 128, 16>), dim3(nch), dim3(256), 0, st,
                       static_cast<const bf16*>(ws.dS), out);
  return hipGetLastError();
}

hipError_t launch_scan_fwd(int dtype, int C, const Shape& s, const FwdWs& ws, const void* h0, void* states,
                           float* final_state, hipStream_t st) {
  if (dtype == 0)
    return scan_t<float, 16, 16, 16, true>(s, ws.negw, ws.krT, ws.uT, nullptr, ws.eg, h0, states, nullptr,
                                           final_state, nullptr, st);
  if (C == 64)
    return scan_t<bf16, 128, 128, 64, true>(s, ws.negw, ws.krT, ws.uT, nullptr, ws.eg, h0, states, nullptr,
                                            final_state, nullptr, st);
  return scan_t<bf16, 128, 128, 16, true>(s, ws.negw, ws.krT, ws.uT, nullptr, ws.eg, h0, states, nullptr,
                                          final_state, nullptr, st);
}

hipError_t launch_scan_bwd(int dtype, int C, const Shape& s, const BwdWs& ws, const void* dO, const void* dSf,
                           float* dh0, hipStream_t st) {
  if (dtype == 0)
    return scan_t<float, 16, 16, 16, false>(s, ws.kr, ws.nwT, nullptr, ws.bcT, ws.eg, dSf, ws.dS, ws.yT, dh0, dO,
                                            st);
  if (C == 64)
    return scan_t<bf16, 128, 128, 64, false>(s, ws.kr, ws.nwT, nullptr, ws.bcT, ws.eg, dSf, ws.dS, ws.yT, dh0, dO,
                                             st);
  return scan_t<bf16, 128, 128, 16, false>(s, ws.kr, ws.nwT, nullptr, ws.bcT, ws.eg, dSf, ws.dS, ws.yT, dh0, dO,
                                           st);
}

}  // namespace kda
