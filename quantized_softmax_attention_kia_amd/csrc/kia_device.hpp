// Device-side building blocks of the K-interval attention kernels for gfx950.
//
// Scores are computed once, in the forward, as bf16 slice products on the matrix
// pipe with a rigorous error bound, and recomputed exactly (double products and
// sums, one rounding to fp32) wherever that bound could change an extremum or a
// decision; the forward stores them as 32 x 32 tiles that every later pass reads
// back.  Calibration, grid tables and decisions go through the functions below
// in every kernel, so all kernels take the same decisions on the same stored
// scores.
//
// Operator: "Pretraining Transformers with Quantized Softmax in Attention",
// §3 (Objects and calibration; Reconstruction) and App. A (edge cases).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kia_launch.hpp"

namespace kia {

typedef float f16v __attribute__((ext_vector_type(16)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int KMAX = 64;
constexpr float DEGENERATE_EPS = 1e-12f;

// ---------------------------------------------------------------------------------------------
// 32x32 MFMA accumulator layout: lane l, register v holds C[crow(v, l/32)][l%32].
__device__ __forceinline__ int crow(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }

__device__ __forceinline__ f16v zero16() {
  f16v z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ---------------------------------------------------------------------------------------------
// Stored score tiles.  A tile holds the 32 x 32 scores of (query tile qt, key tile kt) in the
// accumulator order of the fp32 32x32x2 MFMA computing S^T: element (query a, key b) sits at
// float offset v * 64 + a + 32 g where b = crow(v, g).  So a lane whose query is l%32 reads
// its 16 scores at offsets v * 64 + l, one coalesced 256-byte load per register.
// Causal heads store the tiles kt <= qt only.
__device__ __forceinline__ size_t tile_index(int qt, int kt, int nt, int causal) {
  return causal ? (size_t)qt * (qt + 1) / 2 + kt : (size_t)qt * nt + kt;
}

// ---------------------------------------------------------------------------------------------
// Input element types: float32, or bfloat16 stored as raw uint16 bits.
template <typename T> struct Ld;
template <> struct Ld<float> {
  __device__ static f4v four(const float* p) { return *reinterpret_cast<const f4v*>(p); }
  __device__ static float one(const float* p) { return *p; }
};
template <> struct Ld<uint16_t> {
  __device__ static float one(const uint16_t* p) { return __uint_as_float(((uint32_t)*p) << 16); }
  __device__ static f4v four(const uint16_t* p) {
    uint2 raw = *reinterpret_cast<const uint2*>(p);
    f4v r;
    r[0] = __uint_as_float(raw.x << 16);
    r[1] = __uint_as_float(raw.x & 0xffff0000u);
    r[2] = __uint_as_float(raw.y << 16);
    r[3] = __uint_as_float(raw.y & 0xffff0000u);
    return r;
  }
};

// ---------------------------------------------------------------------------------------------
// bf16 MFMA (32x32x16): lane l supplies A[l%32][8(l/32) + e] and B[8(l/32) + e][l%32] for e < 8;
// the accumulator has the layout of the fp32 32x32 MFMA.  These run on the matrix pipe, beside
// the VALU, while the fp32 / fp64 MFMAs share the VALU's issue.  An fp32 product is carried out
// on three bf16 slices per operand, x = h + m + l (each the round-to-nearest-even bf16 of what
// the previous slices leave; |x - (h + m + l)| <= 2^-24 |x|), keeping the six slice products
// whose weight is at least 2^-16 of h h'.
typedef __bf16 bf8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f16v mfma_bf16(bf8v a, bf8v b, f16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp64 MFMA (16x16x4): lane l supplies A[l%16][l/16] and B[l/16][l%16]; element i of lane l of
// the accumulator is C[l/16 + 4 i][l%16].  Products and sums in double: operands that are floats
// (fp32 or bf16 inputs, bfloat16 weights) multiply exactly.
typedef double d4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ d4v mfma_f64(double a, double b, d4v c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ d4v zero4d() { return d4v{0.0, 0.0, 0.0, 0.0}; }

// Number of bf16 slices that represent an input element exactly enough: bf16 inputs are exact.
template <typename TIn> constexpr int nslices() { return sizeof(TIn) == 2 ? 1 : 3; }

struct Split8 {
  bf8v h, m, l;
};

// Two floats rounded to bf16 (round to nearest even) in one packed conversion: a in the low
// half, b in the high half.
typedef float f2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2v{a, b}, bf2v));
}
__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// Three-slice split of two floats, each slice packed as a bf16 pair (a low, b high).  Each
// residual is exact: a slice is within a factor 2 of what it rounds.
struct SplitPair {
  uint32_t h, m, l;
};
template <int NS = 3>
__device__ __forceinline__ SplitPair split_pair(float a, float b) {
  SplitPair s;
  s.h = cvt_pk_bf16(a, b);
  if (NS == 3) {
    const float ra = a - bf16_lo(s.h), rb = b - bf16_hi(s.h);
    s.m = cvt_pk_bf16(ra, rb);
    s.l = cvt_pk_bf16(ra - bf16_lo(s.m), rb - bf16_hi(s.m));
  }
  return s;
}

__device__ __forceinline__ Split8 split8(const float* x) {
  uint32_t h[4], m[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const SplitPair sp = split_pair(x[2 * e], x[2 * e + 1]);
    h[e] = sp.h;
    m[e] = sp.m;
    l[e] = sp.l;
  }
  Split8 s;
  __builtin_memcpy(&s.h, h, 16);
  __builtin_memcpy(&s.m, m, 16);
  __builtin_memcpy(&s.l, l, 16);
  return s;
}

// c += A B for one 16-deep block, smallest products first.  NSA / NSB = 1 when that operand is
// exact in bf16 (its m, l slices are zero and are not read).
template <int NSB, int NSA = 3>
__device__ __forceinline__ f16v mfma_split(const Split8& a, const Split8& b, f16v c) {
  if (NSA == 3) c = mfma_bf16(a.l, b.h, c);
  if (NSA == 3 && NSB == 3) c = mfma_bf16(a.m, b.m, c);
  if (NSB == 3) c = mfma_bf16(a.h, b.l, c);
  if (NSA == 3) c = mfma_bf16(a.m, b.h, c);
  if (NSB == 3) c = mfma_bf16(a.h, b.m, c);
  return mfma_bf16(a.h, b.h, c);
}

// A 32-row tile of a [T, D] head tensor staged transposed into LDS as NS bf16 slices,
// XT[s][d * TP + r] (r = row within the tile), the B operand of a bf16 product that contracts
// over the rows.  Thread t of the NTH staging threads holds rows 2 (t % 16) and 2 (t % 16) + 1
// at the columns (t / 16) * CW ... + CW - 1 and writes each pair of rows as one 32-bit word.
// TP = 36 keeps the 8-byte operand reads free of bank conflicts.
constexpr int TP = 36;

template <int D, typename T, int NTH = 128>
struct PairRegs {
  static constexpr int CW = D * 16 / NTH;
  float x0[CW], x1[CW];
  __device__ __forceinline__ void load(const T* src, int row0, int nrows) {
    const int t = threadIdx.x % NTH, rp = t & 15, cg = t >> 4;
    const int r0 = row0 + 2 * rp;
#pragma unroll
    for (int j = 0; j < CW / 4; ++j) {
      const f4v a = r0 < nrows ? Ld<T>::four(src + (size_t)r0 * D + cg * CW + 4 * j) : f4v{0.f, 0.f, 0.f, 0.f};
      const f4v b = r0 + 1 < nrows ? Ld<T>::four(src + (size_t)(r0 + 1) * D + cg * CW + 4 * j)
                                   : f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) { x0[4 * j + e] = a[e]; x1[4 * j + e] = b[e]; }
    }
  }
  template <int NS>
  __device__ __forceinline__ void store_t(__bf16* xt) const {
    const int t = threadIdx.x % NTH, rp = t & 15, cg = t >> 4;
    uint32_t* w = reinterpret_cast<uint32_t*>(xt);
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int at = ((cg * CW + j) * TP + 2 * rp) >> 1;
      const SplitPair sp = split_pair<NS>(x0[j], x1[j]);
      w[at] = sp.h;
      if (NS == 3) {
        w[at + (D * TP >> 1)] = sp.m;
        w[at + (D * TP)] = sp.l;
      }
    }
  }
  // the two rows in their natural layout as floats, X[r * stride + d] (stride a multiple of 4)
  __device__ __forceinline__ void store_f32(float* x, int stride) const {
    const int t = threadIdx.x % NTH, rp = t & 15, cg = t >> 4;
#pragma unroll
    for (int j = 0; j < CW / 4; ++j) {
      float* p = x + (2 * rp) * stride + cg * CW + 4 * j;
      *reinterpret_cast<f4v*>(p) = f4v{x0[4 * j], x0[4 * j + 1], x0[4 * j + 2], x0[4 * j + 3]};
      *reinterpret_cast<f4v*>(p + stride) = f4v{x1[4 * j], x1[4 * j + 1], x1[4 * j + 2], x1[4 * j + 3]};
    }
  }
};

// bf16 inputs: the rows stay packed as loaded (two bf16 to a word), half the registers of the
// float form; they are exact bf16 values, so the transposed store only moves their halves
template <int D, int NTH>
struct PairRegs<D, uint16_t, NTH> {
  static constexpr int CW = D * 16 / NTH;
  uint32_t x0[CW / 2], x1[CW / 2];  // columns 2 i (low half) and 2 i + 1 (high half)
  __device__ __forceinline__ void load(const uint16_t* src, int row0, int nrows) {
    const int t = threadIdx.x % NTH, rp = t & 15, cg = t >> 4;
    const int r0 = row0 + 2 * rp;
#pragma unroll
    for (int j = 0; j < CW / 4; ++j) {
      const uint2 a = r0 < nrows ? *reinterpret_cast<const uint2*>(src + (size_t)r0 * D + cg * CW + 4 * j) : uint2{0u, 0u};
      const uint2 b = r0 + 1 < nrows ? *reinterpret_cast<const uint2*>(src + (size_t)(r0 + 1) * D + cg * CW + 4 * j)
                                     : uint2{0u, 0u};
      x0[2 * j] = a.x; x0[2 * j + 1] = a.y;
      x1[2 * j] = b.x; x1[2 * j + 1] = b.y;
    }
  }
  template <int NS>
  __device__ __forceinline__ void store_t(__bf16* xt) const {
    static_assert(NS == 1, "bf16 inputs are one slice");
    const int t = threadIdx.x % NTH, rp = t & 15, cg = t >> 4;
    uint32_t* w = reinterpret_cast<uint32_t*>(xt);
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      const int at = ((cg * CW + j) * TP + 2 * rp) >> 1;
      const uint32_t a = (j & 1) ? x0[j >> 1] >> 16 : x0[j >> 1] & 0xffffu;
      const uint32_t b = (j & 1) ? x1[j >> 1] & 0xffff0000u : x1[j >> 1] << 16;
      w[at] = a | b;
    }
  }
  __device__ __forceinline__ void store_f32(float* x, int stride) const {
    const int t = threadIdx.x % NTH, rp = t & 15, cg = t >> 4;
#pragma unroll
    for (int j = 0; j < CW / 4; ++j) {
      float* p = x + (2 * rp) * stride + cg * CW + 4 * j;
      *reinterpret_cast<f4v*>(p) = f4v{bf16_lo(x0[2 * j]), bf16_hi(x0[2 * j]), bf16_lo(x0[2 * j + 1]), bf16_hi(x0[2 * j + 1])};
      *reinterpret_cast<f4v*>(p + stride) =
          f4v{bf16_lo(x1[2 * j]), bf16_hi(x1[2 * j]), bf16_lo(x1[2 * j + 1]), bf16_hi(x1[2 * j + 1])};
    }
  }
};

// A 32-row tile staged in its natural layout as NS bf16 slices, XN[s][r * NP + d], for A / B
// operands that contract over the columns (8 consecutive columns per lane).  Thread t of the
// NTH holds PER consecutive values of one row.  NP = D + 8 keeps the 16-byte reads and writes
// free of bank conflicts.
template <int D>
constexpr int np() { return D + 8; }

template <int D, typename T, int NTH = 128>
struct RowRegs {
  static constexpr int PER = 32 * D / NTH;
  float x[PER];
  __device__ __forceinline__ void load(const T* src, int row0, int nrows) {
    const int t = threadIdx.x % NTH, r = t / (D / PER), c0 = (t % (D / PER)) * PER;
    const int gr = row0 + r;
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) {
      const f4v a = gr < nrows ? Ld<T>::four(src + (size_t)gr * D + c0 + 4 * j) : f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * j + e] = a[e];
    }
  }
  template <int NS>
  __device__ __forceinline__ void store(__bf16* xn) const {
    const int t = threadIdx.x % NTH, r = t / (D / PER), c0 = (t % (D / PER)) * PER;
#pragma unroll
    for (int j = 0; j < PER / 8; ++j) {
      const Split8 sp = split8(x + 8 * j);
      __bf16* o = xn + r * np<D>() + c0 + 8 * j;
      *reinterpret_cast<bf8v*>(o) = sp.h;
      if (NS == 3) {
        *reinterpret_cast<bf8v*>(o + 32 * np<D>()) = sp.m;
        *reinterpret_cast<bf8v*>(o + 64 * np<D>()) = sp.l;
      }
    }
  }
  // the row in its natural layout as floats, X[r * stride + d] (stride a multiple of 4)
  __device__ __forceinline__ void store_f32(float* xs, int stride) const {
    const int t = threadIdx.x % NTH, r = t / (D / PER), c0 = (t % (D / PER)) * PER;
#pragma unroll
    for (int j = 0; j < PER / 4; ++j)
      *reinterpret_cast<f4v*>(xs + r * stride + c0 + 4 * j) = f4v{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
  }
};

// bf16 inputs: the row stays packed as loaded (two bf16 to a word)
template <int D, int NTH>
struct RowRegs<D, uint16_t, NTH> {
  static constexpr int PER = 32 * D / NTH;
  uint32_t x[PER / 2];
  __device__ __forceinline__ void load(const uint16_t* src, int row0, int nrows) {
    const int t = threadIdx.x % NTH, r = t / (D / PER), c0 = (t % (D / PER)) * PER;
    const int gr = row0 + r;
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) {
      const uint2 a = gr < nrows ? *reinterpret_cast<const uint2*>(src + (size_t)gr * D + c0 + 4 * j) : uint2{0u, 0u};
      x[2 * j] = a.x;
      x[2 * j + 1] = a.y;
    }
  }
  template <int NS>
  __device__ __forceinline__ void store(__bf16* xn) const {
    static_assert(NS == 1, "bf16 inputs are one slice");
    const int t = threadIdx.x % NTH, r = t / (D / PER), c0 = (t % (D / PER)) * PER;
#pragma unroll
    for (int j = 0; j < PER / 8; ++j)
      *reinterpret_cast<uint4*>(xn + r * np<D>() + c0 + 8 * j) = uint4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
  }
  __device__ __forceinline__ void store_f32(float* xs, int stride) const {
    const int t = threadIdx.x % NTH, r = t / (D / PER), c0 = (t % (D / PER)) * PER;
#pragma unroll
    for (int j = 0; j < PER / 4; ++j)
      *reinterpret_cast<f4v*>(xs + r * stride + c0 + 4 * j) =
          f4v{bf16_lo(x[2 * j]), bf16_hi(x[2 * j]), bf16_lo(x[2 * j + 1]), bf16_hi(x[2 * j + 1])};
  }
};

// Slices of 8 consecutive columns 16 kb + 8 (l/32) .. of row `row` of a natural-layout tile.
template <int D, int NS>
__device__ __forceinline__ Split8 load_an(const __bf16* xn, int row, int kb) {
  const int g = (threadIdx.x & 63) >> 5;
  const __bf16* p = xn + row * np<D>() + 16 * kb + 8 * g;
  Split8 r;
  r.h = *reinterpret_cast<const bf8v*>(p);
  if (NS == 3) {
    r.m = *reinterpret_cast<const bf8v*>(p + 32 * np<D>());
    r.l = *reinterpret_cast<const bf8v*>(p + 64 * np<D>());
  }
  return r;
}

// One lane's operand of a row of a [T, D] tensor for a product that contracts over the columns:
// columns 16 kb + 8 (l/32) .. + 7, split into bf16 slices on demand (bf16 inputs are their own
// single slice).
template <int D, typename TIn> struct RowOp;
template <int D> struct RowOp<D, float> {
  float x[D / 2];
  __device__ __forceinline__ void load(const float* base, int row, int nrows) {
    const int g = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f4v a = row < nrows ? *reinterpret_cast<const f4v*>(base + (size_t)row * D + 16 * kb + 8 * g + 4 * h)
                                  : f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) x[8 * kb + 4 * h + e] = a[e];
      }
  }
  __device__ __forceinline__ Split8 split(int kb) const { return split8(x + 8 * kb); }
};
template <int D> struct RowOp<D, uint16_t> {
  uint4 x[D / 16];
  __device__ __forceinline__ void load(const uint16_t* base, int row, int nrows) {
    const int g = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb)
      x[kb] = row < nrows ? *reinterpret_cast<const uint4*>(base + (size_t)row * D + 16 * kb + 8 * g)
                          : uint4{0u, 0u, 0u, 0u};
  }
  __device__ __forceinline__ Split8 split(int kb) const {
    Split8 s;
    s.h = __builtin_bit_cast(bf8v, x[kb]);
    return s;
  }
};

// The exact score of one (query, key) pair: products and sum in double, scale in double,
// rounded once to fp32 -- the value the bound is measured against.
template <int D, typename TIn, int UNROLL = 8>
__device__ __forceinline__ float exact_score(const TIn* qrow, const TIn* krow, double scale) {
  double acc = 0.0;
#pragma unroll UNROLL
  for (int d = 0; d < D; d += 4) {
    const f4v x = Ld<TIn>::four(qrow + d), y = Ld<TIn>::four(krow + d);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fma((double)x[e], (double)y[e], acc);
  }
  return (float)(scale * acc);
}

// B operand slices for k-block b (rows 16b .. 16b+15) and output column n of the transposed tile.
// Lane (n, g) supplies rows 16b + 4g + (0..3) and 16b + 8 + 4g + (0..3): the rows that the
// accumulator-layout coefficients v = 8b .. 8b+7 of lane (., g) stand for (crow(v, g)).
template <int D, int NS>
__device__ __forceinline__ Split8 load_bt(const __bf16* xt, int b, int n) {
  const int g = (threadIdx.x & 63) >> 5;
  Split8 r;
  const __bf16* p = xt + n * TP + 16 * b + 4 * g;
  auto rd = [&](const __bf16* q) {
    const uint2 lo = *reinterpret_cast<const uint2*>(q);
    const uint2 hi = *reinterpret_cast<const uint2*>(q + 8);
    bf8v v;
    const uint4 u = uint4{lo.x, lo.y, hi.x, hi.y};
    __builtin_memcpy(&v, &u, 16);
    return v;
  };
  r.h = rd(p);
  if (NS == 3) {
    r.m = rd(p + D * TP);
    r.l = rd(p + 2 * D * TP);
  }
  return r;
}

// The wave's index in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// LDS written by some lanes of the wave and read by others: the wave's LDS operations run in
// program order, so only the compiler has to be kept from moving them across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------------------------
// Per-row calibration (§3 "Objects and calibration"; App. A degenerate branch).  The position
// u of a key is formed in double from its stored fp32 score: with K up to 64, u reaches K and
// an fp32 u would lose the low bits of the local position t.
struct RowCal {
  // u is measured down from the row maximum, u = K - (M - s)/h (the maximum's own weight is then
  // exactly the top grid value); the degenerate MinMax branch measures it up from m (h = 1)
  double origin;  // m (MinMax) or M
  float top_f;    // M
  double inv_h;   // 1/h
  float inv_hf;   // 1/h rounded to float
  float kappa;    // 1 on the regular MinMax branch (h depends on M, m), 0 on the degenerate one
  float origin_f; // the origin as a float (m or M: exact)
  // Secant slope over the grid value: Delta_r = (e^{b_{r+1}} - e^{b_r}) / h = e^{b_r} expm1(b_{r+1} -
  // b_r) / h, and the grid step b_{r+1} - b_r is the same for every r ((M - m)/K, or tau/K).  The
  // difference of two fp32 grid values would lose about (e^step - 1)^-1 ulps when the step is
  // small (K/tau = 64: 64 ulps); the factor formed in double keeps Delta within 2 ulps.
  float slope;
};

template <int CAL>
__device__ __forceinline__ RowCal row_calibration(float M, float m, int K, float tau) {
  RowCal rc;
  if (CAL == MINMAX) {
    const double span = (double)M - (double)m;
    const bool deg = !(span > (double)DEGENERATE_EPS);
    const double h = deg ? 1.0 : span / (double)K;
    rc.origin = (double)m;
    rc.inv_h = 1.0 / h;
    rc.kappa = deg ? 0.0f : 1.0f;
    rc.slope = (float)(expm1(span / (double)K) / h);
  } else {
    const double h = (double)tau / (double)K;
    rc.origin = (double)M;
    rc.inv_h = (double)K / (double)tau;
    rc.kappa = 1.0f;
    rc.slope = (float)(expm1(h) / h);
  }
  rc.inv_hf = (float)rc.inv_h;
  rc.origin_f = CAL == MINMAX ? m : M;
  rc.top_f = M;
  return rc;
}

// Grid value e^{b_r} (exponent and exponential in double, rounded to float):
// MinMax b_r = (1 - r/K)(m - M); FWM b_r = -tau + r tau/K (any integer r on the resolved grid).
template <int CAL>
__device__ __forceinline__ float grid_value(float M, float m, int K, float tau, int r) {
  double b;
  if (CAL == MINMAX) b = (1.0 - (double)r / (double)K) * ((double)m - (double)M);
  else b = -(double)tau + (double)r * ((double)tau / (double)K);
  return (float)exp(b);
}

// Bin decision for one score: interval index r in [0, K-1] (any r <= K-1 on the resolved FWM
// grid), local position t in [0, 1], and the FWM tail flag (z = s - M < -tau; never set on the
// resolved grid).
struct Decision {
  int r;
  float t;
  bool tail;
};

// lowest interval index formed on the resolved grid: keeps the conversion to int defined (the
// grid values there are far below the smallest float)
constexpr int RES_RMIN = -(1 << 24);

template <int CAL>
__device__ __forceinline__ Decision decide(float s, const RowCal& rc, int K, float tau) {
  Decision d;
  double u;
  if (CAL == FWM_RES) {  // App. D.4: the grid continues below -tau, nothing is clipped below
    const double z = (double)s - (double)rc.top_f;
    d.tail = false;
    u = (double)K + fmin(z, 0.0) * rc.inv_h;
    const int r = min((int)fmax(floor(u), (double)RES_RMIN), K - 1);
    d.r = r;
    d.t = (float)fmin(fmax(u - (double)r, 0.0), 1.0);
    return d;
  }
  if (CAL == MINMAX) {
    u = rc.kappa != 0.f ? (double)K - ((double)rc.top_f - (double)s) * rc.inv_h : (double)s - rc.origin;
    d.tail = false;
  } else {
    const double z = (double)s - (double)rc.top_f;
    d.tail = z < -(double)tau;
    u = (double)K + fmax(z, -(double)tau) * rc.inv_h;
  }
  int r = (int)floor(u);
  r = min(max(r, 0), K - 1);
  d.r = r;
  d.t = (float)fmin(fmax(u - (double)r, 0.0), 1.0);
  return d;
}

// The same decision with u formed in float, for a caller that checks it against a margin.  Each
// of the (at most four) roundings on the way to u errs by at most 2^-24 of a quantity below
// (K + 1) interval widths, so this u is within (K + 1) 2^-22 of decide()'s: a decision whose t
// is farther than that from 0, 1 (interior boundaries) and 1/2 (Nearest) is decide()'s, and so
// is the FWM tail flag when |(s - M) + tau| (in float) exceeds tau 2^-21.  Measured from the
// maximum, the error shrinks toward the top of the grid (K - u widths times a few 2^-24), where
// the weights are largest, and vanishes at the maximum itself.
// On the resolved grid |u| is not bounded by K + 1: the caller widens the margin by |r| 2^-22.
template <int CAL>
__device__ __forceinline__ Decision decide_fast(float s, const RowCal& rc, int K, float tau) {
  Decision d;
  float u;
  if (CAL == FWM_RES) {
    const float z = s - rc.top_f;
    d.tail = false;
    u = fmaf(fminf(z, 0.f), rc.inv_hf, (float)K);
    const int r = min((int)floorf(fmaxf(u, (float)RES_RMIN)), K - 1);
    d.r = r;
    d.t = __builtin_amdgcn_fmed3f(u - (float)r, 0.f, 1.f);
    return d;
  }
  if (CAL == MINMAX) {
    u = rc.kappa != 0.f ? fmaf(s - rc.top_f, rc.inv_hf, (float)K) : s - rc.origin_f;
    d.tail = false;
  } else {
    const float z = s - rc.top_f;
    d.tail = z < -tau;
    u = fmaf(fmaxf(z, -tau), rc.inv_hf, (float)K);
  }
  // the interval index clamped in float (one med3), then converted once
  const float rf = __builtin_amdgcn_fmed3f(floorf(u), 0.f, (float)(K - 1));
  d.r = (int)rf;
  d.t = __builtin_amdgcn_fmed3f(u - rf, 0.f, 1.f);
  return d;
}
// Reconstructed weights of one key (§3 "Reconstruction"), from the row's grid table.
struct Weights {
  float E0, E1;  // e^{b_r}, e^{b_{r+1}}
  float wL;      // LERP: (1-t) E0 + t E1
  float wN;      // Nearest: E0 or E1 at index r + 1[t >= 1/2]
};

// Grid value r of the row sits at trow[r * ST]: ST = 1 for a table of its own (FWM: one for all
// rows), ST = rows per workgroup for the per-row MinMax tables, kept interval-major so that the
// rows of a wave read distinct LDS banks whatever their intervals.
template <int ST = 1>
__device__ __forceinline__ Weights weights(const Decision& d, const float* trow) {
  Weights w;
  w.E0 = trow[d.r * ST];
  w.E1 = trow[(d.r + 1) * ST];
  w.wL = fmaf(d.t, w.E1 - w.E0, w.E0);
  w.wN = (d.t >= 0.5f) ? w.E1 : w.E0;
  return w;
}

// The same for any calibration.  The FWM tables are shared by the rows (the FWM grid does not
// depend on the row) and, on the resolved grid, start lres levels below the window: trow[r] for
// r >= -lres.  When the table reaches b <= -104, where e^b rounds to 0 in float, a key further
// below reads that zero entry; otherwise (far: the level cap was hit, K/tau large) such a key has
// its grid values computed here.
template <int CAL, int ST = 1>
__device__ __forceinline__ Weights weights_cal(const Decision& d, const float* trow, int lres, bool far, int K,
                                               float tau) {
  if (CAL != FWM_RES) return weights<ST>(d, trow);
  Weights w;
  w.E0 = trow[max(d.r, -lres)];
  w.E1 = trow[max(d.r + 1, -lres)];
  if (far && d.r < -lres) {
    w.E0 = grid_value<FWM_RES>(0.f, 0.f, K, tau, d.r);
    w.E1 = grid_value<FWM_RES>(0.f, 0.f, K, tau, d.r + 1);
  }
  w.wL = fmaf(d.t, w.E1 - w.E0, w.E0);
  w.wN = (d.t >= 0.5f) ? w.E1 : w.E0;
  return w;
}

// ---------------------------------------------------------------------------------------------
// Exponential baselines ("Pretraining Transformers with Quantized Softmax in Attention", App. B
// "Softmax", App. D.5 "Definitions"): w = e^z (softmax), the bfloat16 exponential of z rounded
// to bfloat16 (BF16-exp), e^z rounded to E4M3 (FP8-rounded exp), z = s - M.  Roundings are to
// nearest, ties to even, of the exact value.  The fast forms work in float and report when the
// result may differ from the exact one (a rounding within the error of its float inputs of a
// midpoint); the exact forms take the score difference and the exponential in double.

// nearest bfloat16 value of a float (ties to even), as a float
__device__ __forceinline__ float bf16_round(float x) {
  const uint32_t b = __float_as_uint(x);
  return __uint_as_float((b + 0x7fffu + ((b >> 16) & 1u)) & 0xffff0000u);
}
// distance of a float from the nearest bfloat16 rounding midpoint, in bfloat16 spacings
__device__ __forceinline__ float bf16_mid_dist(float x) {
  return fabsf((float)(__float_as_uint(x) & 0xffffu) - 32768.f) * 0x1p-16f;
}
// nearest bfloat16 value of a double (normal range) or of a value in the bfloat16 subnormal range
__device__ __forceinline__ double bf16_round_d(double x) {
  if (fabs(x) < 0x1p-126) return rint(x * 0x1p133) * 0x1p-133;
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t r = (b + 0xfffffffffffull + ((b >> 45) & 1ull)) & ~0x1fffffffffffull;
  return __longlong_as_double((long long)r);
}
// nearest E4M3 value (3 significand bits, subnormal multiples of 2^-9) of x in [0, 1]
__device__ __forceinline__ float e4m3_round(float x) {
  if (x < 0x1p-6f) return __builtin_rintf(x * 0x1p9f) * 0x1p-9f;
  const uint32_t b = __float_as_uint(x);
  return __uint_as_float((b + 0x7ffffu + ((b >> 20) & 1u)) & 0xfff00000u);
}
__device__ __forceinline__ float e4m3_mid_dist(float x) {
  if (x < 0x1p-6f) {
    const float q = x * 0x1p9f;
    return fabsf(q - floorf(q) - 0.5f);
  }
  return fabsf((float)(__float_as_uint(x) & 0xfffffu) - 524288.f) * 0x1p-20f;
}
__device__ __forceinline__ double e4m3_round_d(double x) {
  if (x < 0x1p-6) return rint(x * 0x1p9) * 0x1p-9;
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t r = (b + 0xffffffffffffull + ((b >> 49) & 1ull)) & ~0x1ffffffffffffull;
  return __longlong_as_double((long long)r);
}
// E4M3 byte of a value the format represents, in [0, 1]
__device__ __forceinline__ int e4m3_code(float w) {
  if (w < 0x1p-6f) return (int)(w * 0x1p9f);
  const uint32_t b = __float_as_uint(w);
  return (int)((((b >> 23) & 0xffu) - 120u) << 3 | ((b >> 20) & 7u));
}

struct ExpW {
  float w;  // the weight
  float d;  // dw/dz: e^z (softmax: w; FP8: the unrounded exponential; BF16: the bfloat16 weight)
};
// fast form: float z, expf.  ez bounds the error of the score behind s (the scores are
// approximations within ez of the exact ones).  *risky_s is set when the exact form on the exact
// score may differ, *risky_e when only the exponential's own rounding may (BF16-exp: z's rounding
// is settled, so the exact form on this score gives the exact value).
template <int MODE>
__device__ __forceinline__ ExpW exp_weight_fast(float s, float M, float ez, bool* risky_s, bool* risky_e) {
  const float z = s - M;
  ExpW r;
  *risky_e = false;
  if (MODE == EXP32) {
    r.w = __expf(z);
    r.d = r.w;
    *risky_s = false;
  } else if (MODE == EXPF8) {
    const float e = __expf(z);
    r.w = e4m3_round(e);
    r.d = e;
    // relative error of e: the score's, z's rounding, the exponential's; times at most 16 spacings
    *risky_s = e4m3_mid_dist(e) < 16.f * (ez + fabsf(z) * 0x1p-23f + 0x1p-20f);
  } else {
    const float zb = bf16_round(z);
    const float e = __expf(zb);
    r.w = bf16_round(e);
    r.d = r.w;
    // z within the score error (plus its own rounding) of a midpoint, in units of z's spacing
    // (at least |z| 2^-8): dist < 256 ez / |z| + 2^-14, multiplied out; the exponential within its
    // error (|zb| 2^-23 + 2^-20 of its value) of a midpoint, in units of its spacing (at least
    // 2^-8 of its value)
    const float az = fabsf(z);
    *risky_s = z != 0.f && bf16_mid_dist(z) * az < fmaf(256.f, ez, az * 0x1p-14f);
    *risky_e = bf16_mid_dist(e) < fmaf(fabsf(zb), 0x1p-15f, 0x1p-12f);
  }
  return r;
}
// exact form: z = s - M in double (exact for floats), the exponential in double, one rounding
template <int MODE>
__device__ __forceinline__ ExpW exp_weight_exact(float s, float M) {
  const double z = (double)s - (double)M;
  ExpW r;
  if (MODE == EXP32) {
    r.w = __expf((float)z);
    r.d = r.w;
  } else if (MODE == EXPF8) {
    const double e = exp(z);
    r.w = (float)e4m3_round_d(e);
    r.d = (float)e;
  } else {
    const double e = exp(bf16_round_d(z));
    r.w = (float)bf16_round_d(e);
    r.d = r.w;
  }
  return r;
}

// Work order.  The dispatcher hands workgroup b to XCD b % 8.  Each XCD gets a contiguous range
// of heads (their K, V and score tiles then stay in that XCD's L2) and walks its tiles heaviest
// first over all of its heads (rank 0 = most work), so the hardware's greedy dispatch balances
// the causal triangle across CUs.  Falls back to rank-major order when the head count is not a
// multiple of 8.
__device__ __forceinline__ void block_work(int nheads, int& head, int& rank) {
  const int b = blockIdx.x;
  if ((nheads & 7) == 0) {
    const int x = b & 7, i = b >> 3, hpx = nheads >> 3;
    rank = i / hpx;
    head = x * hpx + i % hpx;
  } else {
    rank = b / nheads;
    head = b % nheads;
  }
}

}  // namespace kia
