// Device-side building blocks shared by the KDA kernels (gfx950 / CDNA4).
//
// Matrix products use the 16x16 MFMA tiles: bf16 operands with fp32 accumulation
// (v_mfma_f32_16x16x32_bf16) for the bf16 path and fp32 operands (v_mfma_f32_16x16x4_f32)
// for the fp32 path. Both take, per lane l, row (l % 16) of A and column (l % 16) of B,
// with the lane group l / 16 selecting a slice of the contraction index, and return a
// 16x16 fp32 tile in which lane l holds rows 4*(l/16) + j (j = 0..3) of column l % 16.
// Because A and B are indexed by the same (lane group, slot) pairs, any fixed assignment
// of contraction indices to (lane group, slot) computes the same sum; the scan kernel
// uses this to feed accumulator tiles straight back in as B operands.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace kda {

// Phase timestamps for performance work: compiled in only with -DKDA_PHASE_TIMING (never
// in the shipped library). Slot [kernel][block][mark] holds wall_clock64() at a mark.
#ifdef KDA_PHASE_TIMING
extern __device__ unsigned long long kda_phase_ts[3][8][64];
#define KDA_TS(K, I)                                                                        \
  do {                                                                                      \
    if (threadIdx.x == 0 && blockIdx.x < 8 && blockIdx.y == 0 && blockIdx.z == 0)           \
      kda::kda_phase_ts[K][blockIdx.x][I] = wall_clock64();                                 \
  } while (0)
#else
#define KDA_TS(K, I) \
  do {               \
  } while (0)
#endif

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

template <class T>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int KS = 32;   // contraction length of one instruction
  static constexpr int PER = 8;   // contraction values per lane per operand
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag zero() {
    frag z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
    return z;
  }
};

template <>
struct Mma<float> {
  static constexpr int KS = 4;
  static constexpr int PER = 1;
  typedef float frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag zero() { return 0.0f; }
};

__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }
template <class T>
__device__ __forceinline__ T from_f(float x) { return (T)x; }
// x rounded to T and back (the value an operand of type T holds)
template <class T>
__device__ __forceinline__ float rnd(float x) { return to_f(from_f<T>(x)); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// The write strength from the loaded beta value: itself, or the sigmoid of a logit.
__device__ __forceinline__ float beta_of(float raw, int logits) { return logits ? 1.f / (1.f + __expf(-raw)) : raw; }

// Padding (elements) added to the contiguous dimension of LDS matrices: 8 bytes, so a row
// stride is an odd multiple of 8 bytes modulo 128. Measured on gfx950 (bank-conflict
// counter): the 16 lanes of a lane group then hit distinct banks for 8-byte writes at 16
// consecutive rows and for fragment reads done as two 8-byte halves; 16-byte padding cost 4
// conflict cycles on each. bf16 fragments are therefore read as two 8-byte halves.
template <class T>
constexpr int pad_of() { return 8 / (int)sizeof(T); }

// 16 bytes of bf16 as two 8-byte halves (8-byte alignment suffices; whole-vector casts only).
__device__ __forceinline__ bf16x8 ld_2x8(const bf16* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef short s8 __attribute__((ext_vector_type(8)));
  const s4 lo = *reinterpret_cast<const s4*>(p), hi = *reinterpret_cast<const s4*>(p + 4);
  return __builtin_bit_cast(bf16x8, s8(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)));
}
__device__ __forceinline__ void st_2x8(bf16* p, bf16x8 v) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef short s8 __attribute__((ext_vector_type(8)));
  const s8 w = __builtin_bit_cast(s8, v);
  *reinterpret_cast<s4*>(p) = __builtin_shufflevector(w, w, 0, 1, 2, 3);
  *reinterpret_cast<s4*>(p + 4) = __builtin_shufflevector(w, w, 4, 5, 6, 7);
}
__device__ __forceinline__ void st_2x8(float* p, f32x4 v) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  *reinterpret_cast<f2*>(p) = __builtin_shufflevector(v, v, 0, 1);
  *reinterpret_cast<f2*>(p + 2) = __builtin_shufflevector(v, v, 2, 3);
}

// Fragment of a row-major matrix whose contraction index is contiguous: lane l reads
// row r0 + l%16 and contraction indices k0 + PER*(l/16) .. + PER-1. Contraction indices
// >= kmax and rows >= rmax read as zero (kmax must be a multiple of PER).
// Offsets are 32-bit: bases are per-chunk (wave-uniform) pointers and a chunk spans far
// fewer than 2^31 elements.
// The load itself is unconditional (from a clamped, valid row and column) and the zero is
// selected afterwards, so masked loads do not turn into branches that serialise them.
template <class T>
__device__ __forceinline__ typename Mma<T>::frag frag_ld(const T* base, int ld, int r0, int k0, int lane,
                                                           int kmax, int rmax) {
  const int r = r0 + (lane & 15);
  const int kk = k0 + Mma<T>::PER * (lane >> 4);
  const bool ok = kk < kmax && r < rmax;
  const T* p = base + ((ok ? r : 0) * ld + (ok ? kk : 0));
  typename Mma<T>::frag v;
  if constexpr (sizeof(T) == 2) {
    v = ld_2x8(p);
  } else {
    v = *p;
  }
  return ok ? v : Mma<T>::zero();
}

// Same without bounds (all indices known to be valid).
template <class T>
__device__ __forceinline__ typename Mma<T>::frag frag_ld(const T* base, int ld, int r0, int k0, int lane) {
  const int r = r0 + (lane & 15);
  const int kk = k0 + Mma<T>::PER * (lane >> 4);
  if constexpr (sizeof(T) == 2) {
    return ld_2x8(base + (r * ld + kk));
  } else {
    return base[r * ld + kk];
  }
}

// The same as one 16-byte load (global memory, 16-byte aligned rows).
template <class T>
__device__ __forceinline__ typename Mma<T>::frag frag_ld16(const T* base, int ld, int r0, int k0, int lane) {
  const int r = r0 + (lane & 15);
  const int kk = k0 + Mma<T>::PER * (lane >> 4);
  return *reinterpret_cast<const typename Mma<T>::frag*>(base + (r * ld + kk));
}

// Loads 4 consecutive elements as fp32 (8 bytes for bf16, 16 for fp32).
__device__ __forceinline__ f32x4 ld4f(const bf16* p) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ f32x4 ld4f(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Stores 4 fp32 values as 4 consecutive elements.
__device__ __forceinline__ void st4(bf16* p, f32x4 v) {
  bf16x4 o;
  o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
  *reinterpret_cast<bf16x4*>(p) = o;
}
__device__ __forceinline__ void st4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// Geometry of one chunk: sequence index, local chunk index, first token (flat), valid rows.
struct Geo {
  int n;
  int lc;
  int len;
  long bos;
};

// Chunks are numbered sequence by sequence. Dense batches (cu == nullptr): every sequence
// has T tokens and ceil(T/C) chunks. Packed batches: choff[n] is the first chunk of
// sequence n (choff[N] = total chunks); empty sequences own no chunk.
__device__ __forceinline__ Geo chunk_geo(int c, const int32_t* cu, const int32_t* choff, int N, int T, int C) {
  Geo g;
  if (cu == nullptr) {
    const int ntper = (T + C - 1) / C;
    g.n = c / ntper;
    g.lc = c - g.n * ntper;
    g.bos = (long)g.n * T + (long)g.lc * C;
    g.len = min(C, T - g.lc * C);
  } else {
    int lo = 0, hi = N;  // largest n with choff[n] <= c
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (choff[mid] <= c) lo = mid; else hi = mid - 1;
    }
    g.n = lo;
    if (lo >= N) {  // chunk index past the table (host and device copies disagree): empty
      g.lc = 0;
      g.bos = 0;
      g.len = 0;
      return g;
    }
    g.lc = c - choff[lo];
    g.bos = (long)cu[lo] + (long)g.lc * C;
    g.len = min(C, (int)((long)cu[lo + 1] - g.bos));
  }
  return g;
}

// First chunk, chunk count and first token of sequence n.
__device__ __forceinline__ void seq_range(int n, const int32_t* cu, const int32_t* choff, int T, int C,
                                          int& c0, int& nc) {
  if (cu == nullptr) {
    const int ntper = (T + C - 1) / C;
    c0 = n * ntper;
    nc = ntper;
  } else {
    c0 = choff[n];
    nc = choff[n + 1] - choff[n];
  }
}

// ---------------------------------------------------------------------------------
// Column-owner layout. A C x K chunk tensor is split into 16x16 tiles; wave w owns the
// column tiles kt = w, w + NW, ...; inside a column tile lane l owns column
// 16*kt + l%16 and rows 16*rt + 4*(l/16) + j for every row tile rt and j = 0..3, the
// same places an MFMA accumulator tile holds. Per-column scans over the rows run as a
// 4-element in-lane scan plus an exchange of block totals among the 4 lanes
// (l%16, l%16 + 16, +32, +48) that share a column.
// ---------------------------------------------------------------------------------

// Loads rows 16*rt + 4*grp + j (rt < RT, j < 4) of column `col` of a row-major chunk tile
// (row stride ld elements; rows >= len read as zero; needs len >= 1). Every load is issued
// unconditionally before any value is used, so a wave has all of them in flight at once.
template <class T, int RT>
__device__ __forceinline__ void col_load(float (&x)[RT][4], const T* __restrict__ base, int ld, int col, int grp,
                                         int len) {
  T raw[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * rt + 4 * grp + j;
      raw[rt][j] = base[min(row, len - 1) * ld + col];  // len >= 1: always a valid row
    }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) x[rt][j] = 16 * rt + 4 * grp + j < len ? to_f(raw[rt][j]) : 0.f;
}

// Same result as col_load for the 16 columns col0 .. col0+15 (this lane: col0 + lane%16),
// from one row-vector load per 16 x 16 tile: lane (n, grp) reads row row0 + 16rt + n, columns
// col0 + 4grp .. +3 (8 bytes of bf16 or 16 of fp32, so ld and col0 must keep those
// aligned), and MFMAs turn the tile into the column-owner layout: a bf16 16x16x16 against
// the identity, or four fp32 16x16x4 against 0/1 selectors that each place the columns
// c with c % 4 == j. Both are exact (one nonzero product per output). Rows are clamped to
// len - 1 (len >= 1) and read as zero from len on. load() only issues the loads, so that a
// caller can issue all of its loads before the first get() waits. Whole-wave only.
template <class T, int RT>
struct ColTile {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef typename std::conditional<sizeof(T) == 2, s4, f32x4>::type raw_t;
  raw_t raw[RT];
  __device__ __forceinline__ void load(const T* __restrict__ base, int ld, int col0, int lane, int len, int row0 = 0) {
    const int n = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      raw[rt] = *reinterpret_cast<const raw_t*>(base + min(row0 + 16 * rt + n, len - 1) * ld + col0 + 4 * grp);
  }
  __device__ __forceinline__ void get(float (&x)[RT][4], int lane, int len, int row0 = 0) const {
    const int n = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 d;
      if constexpr (sizeof(T) == 2) {
        s4 id;
#pragma unroll
        for (int j = 0; j < 4; ++j) id[j] = (4 * grp + j == n) ? (short)0x3f80 : (short)0;
        d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(raw[rt], id, zero4(), 0, 0, 0);
      } else {
        d = zero4();
#pragma unroll
        for (int j = 0; j < 4; ++j)
          d = __builtin_amdgcn_mfma_f32_16x16x4f32(raw[rt][j], n == 4 * grp + j ? 1.f : 0.f, d, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) x[rt][j] = row0 + 16 * rt + 4 * grp + j < len ? d[j] : 0.f;
    }
  }
};

// The inverse move for bf16 tiles: the values this lane holds in the column-owner layout
// (column lane%16, rows 4(lane/16) .. +3), rounded to bf16, fed as the A operand of an MFMA
// against the identity come out in the row layout: this lane then holds row lane%16,
// columns 4(lane/16) .. +3 (exact, as bf16 values). Whole-wave only.
__device__ __forceinline__ f32x4 to_rows_bf16(float x0, float x1, float x2, float x3, int lane) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const int n = lane & 15, grp = lane >> 4;
  const s4 a = __builtin_bit_cast(s4, bf16x4{(bf16)x0, (bf16)x1, (bf16)x2, (bf16)x3});
  s4 id;
#pragma unroll
  for (int j = 0; j < 4; ++j) id[j] = (4 * grp + j == n) ? (short)0x3f80 : (short)0;
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, id, zero4(), 0, 0, 0);
}

// The forward move for one bf16 tile held in the row layout (this lane: row lane%16, columns
// 4(lane/16) .. +3, as raw bf16 bits): an MFMA against the identity returns it in the
// column-owner layout (column lane%16, rows 4(lane/16) .. +3), exactly. Whole-wave only.
__device__ __forceinline__ f32x4 rows_to_cols_bf16(const short __attribute__((ext_vector_type(4))) raw, int lane) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const int n = lane & 15, grp = lane >> 4;
  s4 id;
#pragma unroll
  for (int j = 0; j < 4; ++j) id[j] = (4 * grp + j == n) ? (short)0x3f80 : (short)0;
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(raw, id, zero4(), 0, 0, 0);
}

// Writes the 16 x 16 tile this wave holds in the column-owner layout (x[j]: row
// r0 + 4(lane/16) + j, column c0 + lane%16) into a row-major array with row stride ld,
// skipping rows >= rmax. bf16: transposed by to_rows_bf16, one 8-byte piece per lane
// (row r0 + lane%16, columns c0 + 4(lane/16) ..); fp32: element by element. Whole-wave.
template <class T>
__device__ __forceinline__ void store_rows(T* __restrict__ base, int ld, int r0, int c0, f32x4 x, int lane, int rmax) {
  const int n = lane & 15, grp = lane >> 4;
  if constexpr (sizeof(T) == 2) {
    const f32x4 r = to_rows_bf16(x[0], x[1], x[2], x[3], lane);
    if (r0 + n < rmax) st4(base + (r0 + n) * ld + c0 + 4 * grp, r);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (r0 + 4 * grp + j < rmax) base[(r0 + 4 * grp + j) * ld + c0 + n] = x[j];
  }
}

// Sums across the 4 lane groups of a column (lanes n, n+16, n+32, n+48) are one fp32
// 16x16x4 MFMA: this lane's value is B[grp][n], and the constant A (lane n_a, grp_a
// supplies A[n_a][grp_a]) picks which groups each output row adds, so output element j
// of this lane is sum over kappa of A[4grp + j][kappa] * value(n, kappa). Exact in fp32.
// Whole-wave only.
__device__ __forceinline__ f32x4 col_mix(float a, float v) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, v, zero4(), 0, 0, 0);
}

// A 16 x 32 block of a row-major bf16 matrix M held as one 16-byte piece per lane (row
// r0 + lane%16, columns c0 + 8(lane/16) .. +7) is written transposed into dst:
// M[r][c] goes to dst[c * ldd + r]. Each half of the pieces is turned around by an MFMA
// against the identity, so every lane writes two 8-byte pieces (4 consecutive rows of one
// column). Whole-wave only.
__device__ __forceinline__ void store_T_block(bf16* __restrict__ dst, int ldd, int r0, int c0, bf16x8 piece, int lane) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef short s8 __attribute__((ext_vector_type(8)));
  const int n = lane & 15, grp = lane >> 4;
  s4 id;
#pragma unroll
  for (int j = 0; j < 4; ++j) id[j] = (4 * grp + j == n) ? (short)0x3f80 : (short)0;
  // whole-vector bit cast (element-wise casts of __bf16 vector elements are not relied on)
  const s8 ps = __builtin_bit_cast(s8, piece);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const s4 a = {ps[4 * h], ps[4 * h + 1], ps[4 * h + 2], ps[4 * h + 3]};
    const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, id, zero4(), 0, 0, 0);
    // this lane: rows r0 + 4grp .. +3 of column c0 + 8(n/4) + 4h + n%4
    st4(dst + (c0 + 8 * (n >> 2) + 4 * h + (n & 3)) * ldd + r0 + 4 * grp, d);
  }
}

// Inclusive prefix sum over rows of one column: x[rt][j] holds row 16*rt + 4*grp + j.
// Returns the column total.
template <int RT>
__device__ __forceinline__ float col_prefix(float (&x)[RT][4], int lane) {
  const int n = lane & 15, grp = lane >> 4;
  // rows 4g+j, j < 3: groups before g; rows 4g+3: every group
  const float a = (n & 3) == 3 ? 1.f : (grp < (n >> 2) ? 1.f : 0.f);
  float carry = 0.f;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    x[rt][1] += x[rt][0];
    x[rt][2] += x[rt][1];
    x[rt][3] += x[rt][2];
    const f32x4 d = col_mix(a, x[rt][3]);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[rt][j] += carry + d[0];
    carry += d[3];
  }
  return carry;
}

// Inclusive suffix (reverse) sum over rows of one column.
template <int RT>
__device__ __forceinline__ void col_suffix(float (&x)[RT][4], int lane) {
  const int n = lane & 15, grp = lane >> 4;
  const float a = (n & 3) == 3 ? 1.f : (grp > (n >> 2) ? 1.f : 0.f);
  float carry = 0.f;
#pragma unroll
  for (int rt = RT - 1; rt >= 0; --rt) {
    x[rt][2] += x[rt][3];
    x[rt][1] += x[rt][2];
    x[rt][0] += x[rt][1];
    const f32x4 d = col_mix(a, x[rt][0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[rt][j] += carry + d[0];
    carry += d[3];
  }
}

// Sum over the 4 lanes that share a column (same l % 16).
__device__ __forceinline__ float col_allsum(float v) { return col_mix(1.f, v)[0]; }

// Sum over the 16 lanes of one lane group (same rows, the 16 columns of a tile): DPP
// rotations within the 16-lane row by 8, 4, 2 and 1.
__device__ __forceinline__ float row_allsum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xF, 0xF, false));
  return v;
}

// ---------------------------------------------------------------------------------
// Block-cooperative product D = A * B over LDS / global operands: A row-major with the
// contraction index contiguous (lda), B given as its transpose Bt (ldb) with the
// contraction contiguous. Output tiles are grouped in blocks of 1 x BN tiles that share
// their A fragments; blocks are dealt to the NW waves round-robin. For each block,
// krange(mt, nt0, kb, ke) narrows the contraction range (triangular operands), and
// epi(it, mt, nt0, acc) consumes the BN accumulator tiles (it = the wave's block
// counter, usable to index per-wave register arrays).
// ---------------------------------------------------------------------------------
template <class T, int MT, int NT, int BN, int NW, int KMAX, class KR, class EPI>
__device__ __forceinline__ void block_gemm(const T* A, int lda, int arows, const T* Bt, int ldb, KR krange,
                                           EPI epi, int wave, int lane) {
  typedef Mma<T> M;
  constexpr int NBN = NT / BN;
  constexpr int NB = MT * NBN;
  constexpr int NIT = (NB + NW - 1) / NW;
  static_assert(NT % BN == 0, "BN must divide the tile columns");
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int blk = wave + it * NW;
    if (blk < NB) {
      const int mt = blk / NBN, nt0 = (blk % NBN) * BN;
      f32x4 acc[BN];
#pragma unroll
      for (int j = 0; j < BN; ++j) acc[j] = zero4();
      int kb = 0, ke = KMAX;
      krange(mt, nt0, kb, ke);
      // every fragment of the block is requested before the first product, so the LDS
      // round trips overlap; the (wave-uniform) range only selects the products
      constexpr int NK = (KMAX + M::KS - 1) / M::KS;
      typename M::frag a[NK], b[NK][BN];
#pragma unroll
      for (int k = 0; k < NK; ++k) {
        a[k] = frag_ld<T>(A, lda, 16 * mt, k * M::KS, lane, KMAX, arows);
#pragma unroll
        for (int j = 0; j < BN; ++j) b[k][j] = frag_ld<T>(Bt, ldb, 16 * (nt0 + j), k * M::KS, lane, KMAX, 1 << 30);
      }
#pragma unroll
      for (int k = 0; k < NK; ++k)
        if (k * M::KS >= kb && k * M::KS < ke) {
#pragma unroll
          for (int j = 0; j < BN; ++j) acc[j] = M::mma(a[k], b[k][j], acc[j]);
        }
      epi(it, mt, nt0, acc);
    }
  }
}

// D = A1 * B1 + A2 * B2 with one accumulator per tile (two contractions of different
// lengths feeding the same output).
template <class T, int MT, int NT, int BN, int NW, int KMAX1, int KMAX2, class KR1, class KR2, class EPI>
__device__ __forceinline__ void block_gemm2(const T* A1, int lda1, const T* Bt1, int ldb1, KR1 kr1, const T* A2,
                                            int lda2, const T* Bt2, int ldb2, KR2 kr2, EPI epi, int wave, int lane) {
  typedef Mma<T> M;
  constexpr int NBN = NT / BN;
  constexpr int NB = MT * NBN;
  constexpr int NIT = (NB + NW - 1) / NW;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int blk = wave + it * NW;
    if (blk < NB) {
      const int mt = blk / NBN, nt0 = (blk % NBN) * BN;
      f32x4 acc[BN];
#pragma unroll
      for (int j = 0; j < BN; ++j) acc[j] = zero4();
      int kb = 0, ke = KMAX1;
      kr1(mt, nt0, kb, ke);
      for (int kk = kb; kk < ke; kk += M::KS) {
        const typename M::frag a = frag_ld<T>(A1, lda1, 16 * mt, kk, lane, KMAX1, 1 << 30);
#pragma unroll
        for (int j = 0; j < BN; ++j)
          acc[j] = M::mma(a, frag_ld<T>(Bt1, ldb1, 16 * (nt0 + j), kk, lane, KMAX1, 1 << 30), acc[j]);
      }
      kb = 0;
      ke = KMAX2;
      kr2(mt, nt0, kb, ke);
      for (int kk = kb; kk < ke; kk += M::KS) {
        const typename M::frag a = frag_ld<T>(A2, lda2, 16 * mt, kk, lane, KMAX2, 1 << 30);
#pragma unroll
        for (int j = 0; j < BN; ++j)
          acc[j] = M::mma(a, frag_ld<T>(Bt2, ldb2, 16 * (nt0 + j), kk, lane, KMAX2, 1 << 30), acc[j]);
      }
      epi(it, mt, nt0, acc);
    }
  }
}

// ---------------------------------------------------------------------------------
// Fragment order of the chunk-scan operands (bf16 path). Per chunk and head:
//   P1 (C x K, the A operand of Y = Z + P1 X):   [C/16][K/32][64 lanes][8]
//   P2 (K x C, the A operand of X' = W + P2 Y):  [K/16][ceil(C/32)][64 lanes][8]
//   Z  (C x V) and W (K x V) accumulator seeds:  [V/16][rows/16][64 lanes][4]
// Lane l = n + 16*g of A fragment (row tile m, contraction pair p) holds row 16m + n at
// contraction indices 32p + 4g + i (slots 0-3) and 32p + 16 + 4g + i (slots 4-7): the
// order in which the scan feeds two accumulator tiles of X (or Y) as one B operand. A
// wave loads one fragment as one contiguous 1 KB block, and the accumulator seeds are
// stored exactly as an accumulator tile is laid out across the lanes.
// ---------------------------------------------------------------------------------
template <int K, int V, int C>
struct ScanFrag {
  static constexpr int KT = K / 16, CT = C / 16, VT = V / 16, KP = K / 32, CQ = (CT + 1) / 2;
  static constexpr int P1_ELEMS = CT * KP * 64 * 8;
  static constexpr int P2_ELEMS = KT * CQ * 64 * 8;
  // element offset of P1[r][k]
  __device__ __forceinline__ static int p1(int r, int k) {
    const int kk = k & 31;
    return (((r >> 4) * KP + (k >> 5)) * 64 + (r & 15) + 16 * ((kk & 15) >> 2)) * 8 + 4 * (kk >> 4) + (kk & 3);
  }
  // element offset of P2[r][c]
  __device__ __forceinline__ static int p2(int r, int c) {
    const int cc = c & 31;
    return (((r >> 4) * CQ + (c >> 5)) * 64 + (r & 15) + 16 * ((cc & 15) >> 2)) * 8 + 4 * (cc >> 4) + (cc & 3);
  }
  // element offset of the 4 values lane `lane` holds of seed tile (column tile vt, row tile m)
  __device__ __forceinline__ static int seed(int vt, int m, int rows16, int lane) {
    return ((vt * rows16 + m) * 64 + lane) * 4;
  }
};

// Global -> LDS copies (lane i's bytes land at lds + i * bytes). Issued as inline assembly:
// the compiler's wait insertion would otherwise treat every LDS read of a buffer they fill
// as depending on these copies and make the reading wave wait for all of its own outstanding
// global stores. The copying wave waits for its copies explicitly (vmcnt) before a barrier
// hands them over, and before the workgroup ends.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}
__device__ __forceinline__ void copy16_to_lds(const void* g, const void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr(lds)), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void copy4_to_lds(const void* g, const void* lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_addr(lds)), "v"(g) : "memory", "m0");
}

// Columns of the backward scan's column slices. Slice vt, lane column n, holds value
// column col(vt, n): slices 2m and 2m+1 share the 32 columns 32m.., each taking 4 of every
// 8. After a 16 x 16 transpose the 4 values a lane holds of slice 2m and those of slice
// 2m+1 are the 8 consecutive columns 32m + 8(lane/16) .. + 7 of a B operand fragment.
struct ScanCols {
  __device__ __forceinline__ static int col(int vt, int n) {
    return 32 * (vt >> 1) + 8 * (n >> 2) + 4 * (vt & 1) + (n & 3);
  }
  // inverse: the slice and lane column of value column v
  __device__ __forceinline__ static int slice(int v) { return 2 * (v >> 5) + ((v & 7) >> 2); }
  __device__ __forceinline__ static int lane_col(int v) { return 4 * ((v & 31) >> 3) + (v & 3); }
};

// ---------------------------------------------------------------------------------
// Sub-block reference points of the intra-chunk gate factors. A chunk's rows are taken in
// blocks of 16, with R_b the chunk-local cumsum G at block b's first row (G is
// non-increasing while g <= 0). For i in block a and j in block b <= a,
//   e^(G_i - G_j) = e^(G_i - R_a) * e^(R_a - R_b) * e^(R_b - G_j),
// with e^(G_i - R_a) <= 1, e^(R_a - R_b) <= 1 and 1 <= e^(R_b - G_j) <= e^(15 max|g|): no
// factor leaves the fp32 / bf16 range however strong the decay across the whole chunk,
// whereas e^(G_i) and e^(-G_j) taken apart overflow once a chunk's G drops below about -87
// (the FLA chunk_kda_bwd page passes this as its safe_gate mode: sub-chunk reference
// points). The kernels keep block-referenced rows (a e^(G - R), k e^(R - G)) and apply the
// middle factor to one operand of each tile below the diagonal block.
// ---------------------------------------------------------------------------------

// R of every row tile for this lane's column, from its column-owner cumsum x[rt][j] (rows
// 16rt + 4grp + j): row 16rt is held by lane group 0, slot 0; broadcast over the lane groups.
template <int RT>
__device__ __forceinline__ void block_refs(const float (&x)[RT][4], float (&R)[RT], int lane) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
    R[rt] = __int_as_float(__builtin_amdgcn_ds_bpermute((lane & 15) << 2, __float_as_int(x[rt][0])));
}

// The kernels choose the references per wave (per 16-column tile of a chunk-head): where
// every |G| of the wave's columns is at most kMildG, R = 0 for every block (the chunk-start
// reference: e^(+-G) themselves are in range and no operand needs the middle factor, which
// is then exactly 1); otherwise R = the block references above. Any R gives the same
// products. Returns whether block references were taken (wave-uniform).
constexpr float kMildG = 80.f;
template <int RT>
__device__ __forceinline__ bool choose_refs(const float (&x)[RT][4], float (&R)[RT], int lane) {
  bool big = false;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) big = big || !(fabsf(x[rt][j]) <= kMildG);
  const bool strong = __builtin_amdgcn_ballot_w64(big) != 0;
  if (strong) {
    block_refs<RT>(x, R, lane);
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) R[rt] = 0.f;
  }
  return strong;
}

// OR of the NW per-wave flags in LDS, as a wave-uniform value.
template <int NW>
__device__ __forceinline__ bool any_flag(const int* f) {
  int a = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) a |= f[i];
  return __builtin_amdgcn_readfirstlane(a) != 0;
}

// Scales the PER contraction values of a fragment by e^(R_a - R_b) of their channels
// k0 .. k0 + PER - 1, b < a, as the product of the consecutive block ratios
// D[c][k] = e^(R_(c+1)[k] - R_c[k]) for c = b .. a-1 (fp32 [RT-1][ldd]; each ratio <= 1).
template <class T>
__device__ __forceinline__ typename Mma<T>::frag scale_channels(typename Mma<T>::frag f, const float* D, int ldd,
                                                                 int a, int b, int k0) {
  if constexpr (sizeof(T) == 2) {
    f32x4 x0 = *reinterpret_cast<const f32x4*>(D + b * ldd + k0);
    f32x4 x1 = *reinterpret_cast<const f32x4*>(D + b * ldd + k0 + 4);
    for (int c = b + 1; c < a; ++c) {
      const f32x4 y0 = *reinterpret_cast<const f32x4*>(D + c * ldd + k0);
      const f32x4 y1 = *reinterpret_cast<const f32x4*>(D + c * ldd + k0 + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x0[i] *= y0[i];
        x1[i] *= y1[i];
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = (bf16)((float)f[i] * x0[i]);
      f[4 + i] = (bf16)((float)f[4 + i] * x1[i]);
    }
    return f;
  } else {
    float x = D[b * ldd + k0];
    for (int c = b + 1; c < a; ++c) x *= D[c * ldd + k0];
    return f * x;
  }
}

// A fragment times one fp32 factor (bf16: rounded back to bf16).
template <class T>
__device__ __forceinline__ typename Mma<T>::frag scale_frag(typename Mma<T>::frag f, float x) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (bf16)((float)f[i] * x);
    return f;
  } else {
    return f * x;
  }
}

// Lower-triangular C x C products over the channels with block-referenced operands:
// tile (mt, nt), nt <= mt, of A Bt^T, where A holds rows a_i e^(G_i - R) and Bt rows
// b_j e^(R - G_j) (row-major, contraction contiguous) and the Bt fragments of tiles below the
// diagonal are scaled by e^(R_mt - R_nt) per channel (from the block ratios D, as in
// scale_channels). Every RT x RT tile is dealt to the NW waves round-robin (as block_gemm
// with BN = 1) and passed to epi(mt, nt, acc); tiles above the diagonal pass zero. scale:
// whether any channel takes block references (else the middle factors are all 1). BATCH:
// request every fragment of a tile before its first product (overlapping the LDS round
// trips, at 8 more VGPRs per contraction step).
template <class T, int RT, int NW, int KC, bool BATCH = true, class EPI>
__device__ __forceinline__ void tri_tiles(const T* A, int lda, const T* Bt, int ldb, const float* D, int ldd, bool scale,
                                          EPI epi, int wave, int lane) {
  typedef Mma<T> M;
  constexpr int NB = RT * RT, NIT = (NB + NW - 1) / NW, NK = KC / M::KS;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int blk = wave + it * NW;
    if (blk < NB) {
      const int mt = blk / RT, nt = blk % RT;
      f32x4 acc = zero4();
      if (nt <= mt && !BATCH) {
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          typename M::frag b = frag_ld<T>(Bt, ldb, 16 * nt, k * M::KS, lane);
          if (scale && nt < mt) b = scale_channels<T>(b, D, ldd, mt, nt, k * M::KS + M::PER * (lane >> 4));
          acc = M::mma(frag_ld<T>(A, lda, 16 * mt, k * M::KS, lane), b, acc);
        }
      } else if (nt <= mt) {
        typename M::frag a[NK], b[NK];
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          a[k] = frag_ld<T>(A, lda, 16 * mt, k * M::KS, lane);
          b[k] = frag_ld<T>(Bt, ldb, 16 * nt, k * M::KS, lane);
        }
        if (scale && nt < mt) {
#pragma unroll
          for (int k = 0; k < NK; ++k) b[k] = scale_channels<T>(b[k], D, ldd, mt, nt, k * M::KS + M::PER * (lane >> 4));
        }
#pragma unroll
        for (int k = 0; k < NK; ++k) acc = M::mma(a[k], b[k], acc);
      }
      epi(mt, nt, acc);
    }
  }
}

// Task of a per-(chunk, value head) workgroup, t = chunk-major index c * nhv + local head,
// dealt so that the G value heads of one q/k group share an XCD (and its L2, which then
// serves their common q and k rows once): workgroups go to the 8 XCDs round-robin by
// linear id, so within each run of 8 G ids, id base + 8 e + gi holds member e of the run's
// group gi. Launch group_grid(total, G) workgroups; ids past the last task get -1.
__host__ __device__ inline int group_grid(int total, int G) {
  return G == 1 ? total : (total + 8 * G - 1) / (8 * G) * (8 * G);
}
__device__ __forceinline__ int group_task(int b, int G, int total) {
  const int run = 8 * G, base = (b / run) * run, rem = b % run;
  const int t = base + (rem % 8) * G + rem / 8;
  return t < total ? t : -1;
}

// Contraction-range helpers for triangular operands (K step = KS, tiles of 16 rows).
template <class T>
__device__ __forceinline__ int round_dn(int x) { return (x / Mma<T>::KS) * Mma<T>::KS; }
template <class T>
__device__ __forceinline__ int round_up(int x) { return ((x + Mma<T>::KS - 1) / Mma<T>::KS) * Mma<T>::KS; }

// Returns x unchanged but opaque to the optimiser, so values derived from it are
// recomputed where they are used instead of being hoisted out of an enclosing loop and
// kept live across it.
__device__ __forceinline__ int opaque_v(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ int opaque_s(int x) {
  asm volatile("" : "+s"(x));
  return x;
}

struct FullRange {
  __device__ void operator()(int, int, int&, int&) const {}
};

}  // namespace kda
