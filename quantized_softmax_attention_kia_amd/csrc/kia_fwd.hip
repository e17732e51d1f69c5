// Forward kernel of K-interval attention for gfx950 (CDNA4).
//
// "Pretraining Transformers with Quantized Softmax in Attention", §3: the grid
// of a row depends on the row's final extrema, so the online-softmax rescale
// does not apply.  A workgroup owns 32 query rows of one head (heaviest first); its
// FWD_NW waves split the visible key tiles between them (wave w takes every
// FWD_NW-th), so the longest rows do not hold the whole kernel back, and sweep them
// twice, loading the next tile while they compute the current one (pass 2 under Nearest
// with Prob-STE loads each tile's V while it weighs that tile); partial results meet in
// LDS, in a fixed order:
//   pass 1  scores of each 32 x 32 tile as bf16 slice products on the matrix pipe
//           (K operands loaded straight from memory into registers) with a
//           rigorous error bound per row, stored for every later pass; the row
//           max (and for MinMax min), first index attaining it and tie count are then
//           settled on exact scores (double products and sums, rounded once to fp32)
//           of every candidate within twice the bound, each patched into the stored
//           tile by the lane that stored it;
//   then    per-row calibration and the grid table e^{b_r} in LDS (the only
//           exponentials of the operator): K+1 entries per row under MinMax, one
//           table for every row under FWM (from lres levels below the window on the
//           resolved grid of App. D.4);
//   pass 2  stored scores -> bin decision (one closer to a boundary than the
//           bound is taken again on the exact score, patched in likewise, so every
//           pass decides as on exact scores) -> LERP / Nearest weight from the table
//           (no exp) -> row sums W^L, W^N -> O += w V as bf16 slice products on the
//           matrix pipe, V^T staged in LDS by the wave (and O^L += w^L V for Nearest
//           with Prob-STE; BF16-exp multiplies in double on the fp64 MFMA and stores O
//           with its residual) -> O = num / W (the strict hard forward for Nearest).  Row sums are kept in double and each tile's P V is summed
//           into a fresh accumulator before joining the running O, so the
//           precision of O (which the backward's D_i = dO . O amplifies) does not
//           decay with T.
// Built once per calibration: KIA_CAL (a kia::Calib value) selects the one this build supplies.
#include "kia_device.hpp"
#include "kia_launch.hpp"

#ifndef KIA_CAL
#error "build with -DKIA_CAL=<calibration>"
#endif

#include <climits>
#include <type_traits>

namespace kia {

constexpr int FWD_NW = 2;            // waves per workgroup, splitting the key tiles of a query tile
constexpr int FWD_NT = 64 * FWD_NW;
constexpr int BN = 32;               // keys per tile, query rows per workgroup
constexpr int FWD_EARLY = 4;         // causal: query tiles dispatched before the heaviest-first order
// A key that carries P >= 1/HEAVY_INV of its row is heavy: its score is recomputed exactly after
// pass 2 and its weight corrected, up to HMAX keys per lane
constexpr double HEAVY_INV = 16.0;
constexpr int HMAX = 4;


// Approximate extrema of the keys one lane stored: the two largest values and the key of the
// largest, likewise for the smallest.  Keys reach a lane in increasing order.
struct Lane2 {
  float mx, mx2, mn, mn2;
  int ax, an;
};
// Exact extrema of a row over the stored scores: value, first key, count of ties.
struct XExt {
  float v;
  int k, n;
};

// BF16-exp multiplies its weights by V in double (fp64 MFMA): V as floats, row stride VFS, and
// the tile's weights, row stride PTS (strides that keep the operand reads free of bank conflicts)
template <int D> constexpr int vfs() { return D + 16; }
constexpr int PTS = 36;

template <int D, int NS, bool F64>
constexpr int fwd_wave_bytes() {  // per wave: V of its key tile (as staged), later its partial O
  // (the partial O in double at D = 128 and under BF16-exp)
  return F64 ? (32 * vfs<D>() * 4 + 32 * PTS * 4 > 32 * D * 8 ? 32 * vfs<D>() * 4 + 32 * PTS * 4 : 32 * D * 8)
             : (NS * D * TP * 2 > D / 32 * (D == 128 ? 8192 : 4096) ? NS * D * TP * 2 : D / 32 * (D == 128 ? 8192 : 4096));
}

template <int D, int NS, bool F64>
struct FwdSmem {
  __align__(16) unsigned char wave[FWD_NW][fwd_wave_bytes<D, NS, F64>()];
  float rmx[FWD_NW][BN], rmn[FWD_NW][BN], amx[FWD_NW][BN];
  XExt xM[FWD_NW][BN], xm[FWD_NW][BN];
  double sL[FWD_NW][BN], sN[FWD_NW][BN];
  float rowW[BN], rowWL[BN];
  double rowWd[BN], rowWLd[BN];  // the row sums in double: O's normalizer, and W^L
  // heavy keys retaken after pass 2: per lane up to HMAX keys with their stored scores (batched)
  // or their weight changes (one at a time); per row the sum of the weight changes (batched) or
  // per lane the number of keys (one at a time)
  int hk[FWD_NW][64][HMAX];
  float hd[FWD_NW][64][HMAX];
  union {
    double hs[FWD_NW][BN];
    int hn[FWD_NW][64];
  };
  // long rows: per wave, the key tiles pass 2 flagged for the heavy-key stage (tile iteration i:
  // bit i % 32 of word i / 32), and per row the lowest score that can be heavy for any row sum
  uint32_t tflag[FWD_NW][4];
  float sflag[BN];
  // followed in dynamic LDS by the grid table: BN rows x (K + 1) floats
};

// Error bound of a score taken from bf16 slice products (u = 2^-24).  With fp32 inputs each
// operand is split into three slices (x = h + m + l + e, |m| <= 2^-8 |x|, |l| <= 2^-16 |x|,
// |e| <= 2^-24 |x|); h h' is accumulated apart from the five smaller products kept (their
// magnitudes add up to at most 0.008 |q_d k_d|), every product exact in fp32.  Any order of
// n fp32 additions errs by at most (n - 1) u sum|terms|, so the two sums err by at most
// 1.008 (D - 1) u S and 5D u 0.008 S (S = sum_d |q_d k_d|), the dropped products by 4.1 u S,
// and the final add, the fp32 scale product and the rounding of the exact score to fp32 by
// 4 u |s| <= 4 u S (scale folded in).  S <= 1.01 A, where A is the fp32 sum of |q_h| |k_h|
// (|x| <= |h| / (1 - 2^-8)), one more bf16 product.  With bf16 inputs only h h' exists, exact
// in bf16.  So |s~ - s| <= scale * ACC_C * A, and a decision this bound cannot settle is taken
// again on the score recomputed exactly (double products and sums, rounded once).
template <int D, int NS>
constexpr double acc_c() {
  return NS == 3 ? 1.01 * (1.008 * (D - 1) + 0.04 * D + 8.1) * 0x1p-24 : 1.01 * (D + 4) * 0x1p-24;
}

// Exact scores of one query against two keys in one sweep (the loads of both in flight together).
template <int D, typename TIn>
__device__ __forceinline__ void exact_score2(const TIn* qrow, const TIn* k1, const TIn* k2, double scale,
                                             float& s1, float& s2) {
  double a1 = 0.0, a2 = 0.0;
#pragma unroll 8
  for (int d = 0; d < D; d += 4) {
    const f4v x = Ld<TIn>::four(qrow + d), y1 = Ld<TIn>::four(k1 + d), y2 = Ld<TIn>::four(k2 + d);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a1 = fma((double)x[e], (double)y1[e], a1);
      a2 = fma((double)x[e], (double)y2[e], a2);
    }
  }
  s1 = (float)(scale * a1);
  s2 = (float)(scale * a2);
}

__device__ __forceinline__ bf8v bf_abs(bf8v v) {
  uint4 u;
  __builtin_memcpy(&u, &v, 16);
  u.x &= 0x7fff7fffu; u.y &= 0x7fff7fffu; u.z &= 0x7fff7fffu; u.w &= 0x7fff7fffu;
  bf8v r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// With mx >= mx2 the new second value is the median of (x, mx, mx2); likewise for the minimum.
// A value equal to the extremum keeps the earlier key and becomes the second (a tie).  The minimum
// is tracked for MinMax only (FWM calibrates on the maximum alone).  One key per side is enough:
// a lane whose second value is also a candidate rescans its tiles (near ties, rare).
template <int CAL>
__device__ __forceinline__ void track(Lane2& e, float x, int key) {
  const bool g1 = x > e.mx;
  e.ax = g1 ? key : e.ax;
  e.mx2 = __builtin_amdgcn_fmed3f(x, e.mx, e.mx2);
  e.mx = fmaxf(x, e.mx);
  if (CAL == MINMAX) {
    const bool l1 = x < e.mn;
    e.an = l1 ? key : e.an;
    e.mn2 = __builtin_amdgcn_fmed3f(x, e.mn, e.mn2);
    e.mn = fminf(x, e.mn);
  }
}

// One more exact value of a side: a larger (smaller) one replaces the extremum, an equal one
// is a tie (the lower key is the first index).
__device__ __forceinline__ void xext_add(XExt& a, float v, int key, bool is_max) {
  const bool better = is_max ? v > a.v : v < a.v;
  if (better) { a.v = v; a.k = key; a.n = 1; }
  else if (v == a.v) { a.k = min(a.k, key); ++a.n; }
}

__device__ __forceinline__ void xext_combine(XExt& a, const XExt& b, bool is_max) {
  const float v = is_max ? (a.v > b.v ? a.v : b.v) : (a.v < b.v ? a.v : b.v);
  a.k = min(a.v == v ? a.k : INT_MAX, b.v == v ? b.k : INT_MAX);
  a.n = (a.v == v ? a.n : 0) + (b.v == v ? b.n : 0);
  a.v = v;
}
__device__ __forceinline__ void xext_merge(XExt& a, int lanemask, bool is_max) {
  XExt b;
  b.v = __shfl_xor(a.v, lanemask);
  b.k = __shfl_xor(a.k, lanemask);
  b.n = __shfl_xor(a.n, lanemask);
  xext_combine(a, b, is_max);
}

// At D = 64 the register budget is held to two waves per SIMD.  NB: bins held under bin mean.
// PHASE: 0 the whole forward; 1 pass 1 and the exact extrema only (the stored scores and the row
// record's extrema and score bounds); 2 the rest, from what phase 1 stored.
template <int D, int CAL, int MODE, typename TIn, int NB = BINM_MAXB, int PHASE = 0>
__global__ __launch_bounds__(FWD_NT) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void fwd_kernel(FwdArgs a) {
  constexpr int NS = nslices<TIn>();
  // BF16-exp: the weights are bfloat16 values, taken exactly, and their products with V are summed
  // in double (fp64 MFMA) with the row sums, so that the output carries double precision (O and its
  // residual): the backward's D_i = dO_i . O_i is then exact enough to round dL/dw to bfloat16 as
  // the exact values do
  constexpr bool F64 = MODE == EXPBF;
  // At D = 128 (long rows; one wave per SIMD, registers to spare) the running sum of O (of O^L
  // under Nearest with Prob-STE, whose D_i = dO_i . O^L_i the backward amplifies; O itself stays
  // in float) is kept in double: a row of 8192 keys adds 128 fresh tile products into it, and
  // float roundings of the running sum would reach D_i at about 1e-6 relative
  constexpr bool DRUN = D == 128 && !F64;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  FwdSmem<D, NS, F64>& sm = *reinterpret_cast<FwdSmem<D, NS, F64>*>(smem_raw);
  float* tbl = reinterpret_cast<float*>(smem_raw + sizeof(FwdSmem<D, NS, F64>));
  const int w = wave_id(), l = threadIdx.x & 63, g = l >> 5, c = l & 31;
  const int T = a.T, K = a.K, nt = a.rec.nt;
  int head, rank;
  block_work(a.nheads, head, rank);
  // causal order: the FWD_EARLY earliest query tiles first (short rows, where the heavy-key stage
  // has the most keys to retake: at the end of the launch their latency was its tail), then the
  // rest heaviest first (rank FWD_EARLY: the latest query tile, the most keys)
  const int early = nt < FWD_EARLY ? nt : FWD_EARLY;
  const int qt = a.causal ? (rank < early ? rank : nt - 1 - (rank - early)) : rank;
  const size_t hb = (size_t)head * T * D;
  const TIn* Kp = reinterpret_cast<const TIn*>(a.k) + hb;
  const TIn* Vp = reinterpret_cast<const TIn*>(a.v) + hb;
  const int q0 = qt * BN, qi = q0 + c;
  const bool qvalid = qi < T;
  const int ntiles = a.causal ? qt + 1 : nt;  // wave w takes key tiles w, w + FWD_NW, ...
  float* Sh = a.rec.S + (size_t)head * a.rec.tiles_per_head * 1024;
  __bf16* VT = reinterpret_cast<__bf16*>(sm.wave[w]);
  float* VF = reinterpret_cast<float*>(sm.wave[w]);  // F64: V as floats, then the weights
  float* PT = VF + 32 * vfs<D>();
  // a tile whose every (query, key) pair is visible needs no masks
  auto full_tile = [&](int kt) { return kt * BN + BN <= T && q0 + BN <= T && (!a.causal || kt < qt); };
  auto stored_at = [&](int key) {  // where the lane that stored (qi, key) keeps it
    return tile_index(qt, key / BN, nt, a.causal) * 1024 + (4 * ((key & 31) >> 3) + (key & 3)) * 64 + l;
  };

  const TIn* qrow = reinterpret_cast<const TIn*>(a.q) + hb + (size_t)(qvalid ? qi : 0) * D;
  PairRegs<D, TIn, 64> vr;  // V rows of pass 2's tiles
  // the row's exact extrema (FWM: m = M) and the error bound of its stored scores
  float M, m, Erow;
  if constexpr (PHASE == 2) {
    const size_t row = (size_t)head * T + (qvalid ? qi : 0);
    M = qvalid ? a.rec.M[row] : -INFINITY;
    m = qvalid ? a.rec.m[row] : (CAL == MINMAX ? INFINITY : -INFINITY);
    Erow = qvalid ? a.rec.E[row] : 1e-30f;
    if (MODE != NEAREST_P && w < ntiles) vr.load(Vp, w * BN, T);
  } else {
  // ---- pass 1: scores (bf16 slice products) stored once; approximate row extrema
  // lane (c, g) holds query q0 + c and, in register v of a tile, key k0 + crow(v, g): the order of
  // the stored tiles, so pass 2 reads back exactly what this lane wrote.
  const float scale_f = (float)a.scale;
  // two K operand buffers in turn: the next tile's K is in flight while this one computes (the
  // first is requested before the Q row, so both loads overlap)
  RowOp<D, TIn> kr0, kr1;
  if (w < ntiles) kr0.load(Kp, w * BN + c, T);
  Split8 qs[D / 16];
  bf8v qa[D / 16];
  {
    RowOp<D, TIn> qr;
    qr.load(reinterpret_cast<const TIn*>(a.q) + hb, qi, T);
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      qs[kb] = qr.split(kb);
      qa[kb] = bf_abs(qs[kb].h);
    }
  }
  // keys are tracked without the lane's 4 g (crow(v, g) = crow(v, 0) + 4 g), a wave-uniform value
  Lane2 ex{-INFINITY, -INFINITY, INFINITY, INFINITY, INT_MAX - 4, INT_MAX - 4};
  float amx = 0.f;  // largest sum of |q_h| |k_h| over the row's visible keys
  // one key tile: its scores from the K operand kr (slice products), stored, and tracked
  auto score_tile = [&](int kt, const RowOp<D, TIn>& kr) {
    const int k0 = kt * BN;
    f16v acc = zero16(), asm_ = zero16(), aacc = zero16();  // h h', the smaller products, |h| |h'|
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      const Split8 ks = kr.split(kb);
      if (NS == 3) {
        asm_ = mfma_bf16(ks.l, qs[kb].h, asm_);
        asm_ = mfma_bf16(ks.m, qs[kb].m, asm_);
        asm_ = mfma_bf16(ks.h, qs[kb].l, asm_);
        asm_ = mfma_bf16(ks.m, qs[kb].h, asm_);
        asm_ = mfma_bf16(ks.h, qs[kb].m, asm_);
      }
      acc = mfma_bf16(ks.h, qs[kb].h, acc);
      aacc = mfma_bf16(bf_abs(ks.h), qa[kb], aacc);
    }
    if (NS == 3) acc += asm_;
    float* St = Sh + tile_index(qt, kt, nt, a.causal) * 1024 + l;
    auto epilogue = [&](auto masked) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float x = acc[v] * scale_f;
        const int key = k0 + crow(v, g);
        St[v * 64] = x;
        const bool ok = !decltype(masked)::value || (qvalid & (key < T) & (!a.causal | (key <= qi)));
        if (ok) {
          track<CAL>(ex, x, k0 + crow(v, 0));
          amx = fmaxf(amx, aacc[v]);
        }
      }
    };
    if (full_tile(kt)) epilogue(std::false_type{});
    else epilogue(std::true_type{});
  };
  for (int kt = w; kt < ntiles; kt += 2 * FWD_NW) {
    if (kt + FWD_NW < ntiles) kr1.load(Kp, (kt + FWD_NW) * BN + c, T);
    score_tile(kt, kr0);
    if (kt + FWD_NW >= ntiles) break;
    if (kt + 2 * FWD_NW < ntiles) kr0.load(Kp, (kt + 2 * FWD_NW) * BN + c, T);
    score_tile(kt + FWD_NW, kr1);
  }
  // pass 2's first V tile, loaded while the extrema are settled (not under Nearest with Prob-STE,
  // which loads each tile's V in its own step)
  if (PHASE == 0 && MODE != NEAREST_P && w < ntiles) vr.load(Vp, w * BN, T);
  ex.ax += 4 * g;
  ex.an += 4 * g;
  const Lane2& loc = ex;  // this lane's own extrema: keys whose scores it stored
  // the row's approximate extrema and error bound: lanes of a row, then the waves, in LDS
  {
    const float rmx = fmaxf(loc.mx, __shfl_xor(loc.mx, 32)), rmn = fminf(loc.mn, __shfl_xor(loc.mn, 32));
    amx = fmaxf(amx, __shfl_xor(amx, 32));
    if (g == 0) {
      sm.rmx[w][c] = rmx;
      sm.rmn[w][c] = rmn;
      sm.amx[w][c] = amx;
    }
  }
  __syncthreads();
  float rowmx = sm.rmx[0][c], rowmn = sm.rmn[0][c];
  amx = sm.amx[0][c];
#pragma unroll
  for (int v = 1; v < FWD_NW; ++v) {
    rowmx = fmaxf(rowmx, sm.rmx[v][c]);
    rowmn = fminf(rowmn, sm.rmn[v][c]);
    amx = fmaxf(amx, sm.amx[v][c]);
  }
  // error bound of the row's scores, and of u in interval widths (below)
  const float Er = (float)(a.scale * acc_c<D, NS>()) * amx + 1e-30f;
  Erow = Er;

  // ---- exact extrema.  Every key whose exact score can attain the row maximum (minimum) has a
  // stored score within 2 Erow of the approximate one: a candidate.  Each lane recomputes its own
  // candidate exactly (one per side, whose key it kept) and patches the element it stored; a lane
  // holding more (near ties, rare) rescans its tiles for them.  First index and tie count are then
  // taken over exact values.
  const float thrM = rowmx - 2.f * Er, thrm = rowmn + 2.f * Er;
  XExt yM{-INFINITY, INT_MAX, 0}, ym{INFINITY, INT_MAX, 0};
  // whether this lane's kept key covers its candidates of each side, or it has to rescan
  const bool scanM = qvalid && loc.mx2 >= thrM;
  const bool scanm = CAL == MINMAX && qvalid && loc.mn2 <= thrm;
  const bool oneM = qvalid && loc.mx >= thrM && !scanM, onem = CAL == MINMAX && qvalid && loc.mn <= thrm && !scanm;
  auto exact_pair = [&](bool dM, int kM, bool dm, int km) {
    // exact scores of a max and a min candidate (either may be absent), patched in
    float xM_ = 0.f, xm_ = 0.f;  // (under FWM there is no min candidate: xm_ stays unused)
    const int kM_ = dM ? kM : km, km_ = dm ? km : kM;
    if (CAL == MINMAX) exact_score2<D, TIn>(qrow, Kp + (size_t)kM_ * D, Kp + (size_t)km_ * D, a.scale, xM_, xm_);
    else xM_ = exact_score<D, TIn>(qrow, Kp + (size_t)kM_ * D, a.scale);
    if (dM) {
      Sh[stored_at(kM_)] = xM_;
      xext_add(yM, xM_, kM_, true);
    }
    if (dm) {
      Sh[stored_at(km_)] = xm_;
      xext_add(ym, xm_, km_, false);
    }
  };
  if (oneM || onem) exact_pair(oneM, loc.ax, onem, loc.an);
  if (__any(scanM || scanm)) {
    constexpr int TB = 4;  // tiles per batch of loads
    for (int kt0 = w; kt0 < ntiles; kt0 += TB * FWD_NW) {
      uint32_t cand[TB];  // per tile: bit v for a max candidate, bit 16 + v for a min candidate
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        const int kt = kt0 + i * FWD_NW;
        cand[i] = 0u;
        if ((scanM || scanm) && kt < ntiles) {
          const float* St = Sh + tile_index(qt, kt, nt, a.causal) * 1024 + l;
          float x[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) x[v] = St[v * 64];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kt * BN + crow(v, g);
            const bool ok = key < T && (!a.causal || key <= qi);
            cand[i] |= (scanM && ok && x[v] >= thrM) ? 1u << v : 0u;
            cand[i] |= (scanm && ok && x[v] <= thrm) ? 1u << (16 + v) : 0u;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < TB; ++i) {
        const int kt = kt0 + i * FWD_NW;
        uint32_t bits = (cand[i] | (cand[i] >> 16)) & 0xffffu;  // elements v = 0..15 of the tile
        while (bits) {
          const int v = __builtin_ctz(bits);
          bits &= bits - 1u;
          const int key = kt * BN + crow(v, g);
          const float xe = exact_score<D, TIn>(qrow, Kp + (size_t)key * D, a.scale);
          Sh[tile_index(qt, kt, nt, a.causal) * 1024 + v * 64 + l] = xe;
          if ((cand[i] >> v) & 1u) xext_add(yM, xe, key, true);
          if ((cand[i] >> (16 + v)) & 1u) xext_add(ym, xe, key, false);
        }
      }
    }
  }
  xext_merge(yM, 32, true);
  if (CAL == MINMAX) xext_merge(ym, 32, false);
  if (g == 0) {
    sm.xM[w][c] = yM;
    sm.xm[w][c] = ym;
  }
  __syncthreads();
  XExt xM = sm.xM[0][c], xm = sm.xm[0][c];
#pragma unroll
  for (int v = 1; v < FWD_NW; ++v) {
    xext_combine(xM, sm.xM[v][c], true);
    if (CAL == MINMAX) xext_combine(xm, sm.xm[v][c], false);
  }
  if (CAL != MINMAX) xm = xM;  // FWM: no minimum (recorded as M)
  M = xM.v;
  m = xm.v;
  if (w == 0 && g == 0 && qvalid) {
    const size_t row = (size_t)head * T + qi;
    a.rec.M[row] = M;
    a.rec.m[row] = m;
    a.rec.amax[row] = xM.k;
    a.rec.amin[row] = CAL == MINMAX ? xm.k : 0;
    a.rec.nA[row] = xM.n;
    a.rec.nC[row] = CAL == MINMAX ? xm.n : 0;
    a.rec.E[row] = Er;
  }
  }  // pass 1
  if constexpr (PHASE == 1) return;

  // ---- calibration and grid table (K+1 exponentials per row), shared by the waves
  const RowCal rc = row_calibration<CAL>(M, m, K, a.tau);
  // the error bound in interval widths, with room for the float arithmetic of decide_fast and the
  // rounding of t itself
  const float du = 1.01f * Erow * rc.inv_hf + 0x1p-20f + (float)(K + 1) * 0x1p-22f;

  const float edge = Erow + a.tau * 0x1p-21f;  // FWM window edge: margin of |(s - M) + tau|
  // MinMax: one table row per query row; FWM: one table for all rows, from lres levels below
  // the window (resolved grid) to K; bin mean: one row per query row holding the bin means
  float* trow = tbl;
  if constexpr (MODE == BINM) {
    // ---- bin mean (§5, App. I): a pass over the row's stored scores settles every Nearest
    // decision as pass 2 will (float decisions checked against the bound, exact scores patched in
    // where it cannot settle them, then the half tile decided in double), and sums e^{s - M} and
    // the member count of each bin, per lane in registers; the sums meet per row in a fixed order
    // and the table then holds each bin's mean, so pass 2 runs as Nearest on it.  Keys below an
    // FWM window belong to no bin.
    trow = tbl + c;
    float bs[NB], bn[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) { bs[q] = 0.f; bn[q] = 0.f; }
    for (int kt = w; kt < ntiles; kt += FWD_NW) {
      const int k0 = kt * BN;
      float* Sw = Sh + tile_index(qt, kt, nt, a.causal) * 1024 + l;
      float s[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = Sw[v * 64];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        uint32_t risky = 0, okm = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int v = 8 * b + j, key = k0 + crow(v, g);
          const bool ok = qvalid & (key < T) & (!a.causal | (key <= qi));
          const Decision d = decide_fast<CAL>(s[v], rc, K, a.tau);
          bool r = ((d.t < du) & (d.r > 0)) | ((d.t > 1.f - du) & (d.r < K - 1)) | (fabsf(d.t - 0.5f) < du);
          if (CAL == FWM) r |= fabsf((s[v] - M) + a.tau) <= edge;
          risky |= (ok & r) ? (1u << j) : 0u;
          okm |= ok ? (1u << j) : 0u;
        }
        const bool redo = __any(risky != 0u);
        uint32_t bits = risky;
        while (__any(bits != 0u)) {
          const int j = bits ? __builtin_ctz(bits) : 0;
          if (bits) {
            const float xe = exact_score<D, TIn>(qrow, Kp + (size_t)(k0 + crow(8 * b + j, g)) * D, a.scale);
            Sw[(8 * b + j) * 64] = xe;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) s[8 * b + jj] = jj == j ? xe : s[8 * b + jj];
            bits &= bits - 1u;
          }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int v = 8 * b + j;
          const Decision d = redo ? decide<CAL>(s[v], rc, K, a.tau) : decide_fast<CAL>(s[v], rc, K, a.tau);
          const int ell = d.r + (d.t >= 0.5f ? 1 : 0);
          const bool in = ((okm >> j) & 1u) & !d.tail;
          const float x = __expf(s[v] - M);
#pragma unroll
          for (int q = 0; q < NB; ++q) {
            bs[q] += (in && ell == q) ? x : 0.f;
            bn[q] += (in && ell == q) ? 1.f : 0.f;
          }
        }
      }
    }
    // the row's two lanes of each wave, then the two waves in order
    float* part = reinterpret_cast<float*>(sm.wave[0]);  // [wave][row][bin][sum, count]
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      bs[q] += __shfl_xor(bs[q], 32);
      bn[q] += __shfl_xor(bn[q], 32);
      if (g == 0) {
        part[((w * BN + c) * BINM_MAXB + q) * 2] = bs[q];
        part[((w * BN + c) * BINM_MAXB + q) * 2 + 1] = bn[q];
      }
    }
    __syncthreads();
    for (int q = g + 2 * w; q <= K; q += 2 * FWD_NW) {
      float S = 0.f, n = 0.f;
#pragma unroll
      for (int u = 0; u < FWD_NW; ++u) {
        S += part[((u * BN + c) * BINM_MAXB + q) * 2];
        n += part[((u * BN + c) * BINM_MAXB + q) * 2 + 1];
      }
      trow[q * BN] = n > 0.f ? S / n : 0.f;
    }
  } else if (CAL == MINMAX) {
    trow = tbl + c;  // interval-major: entry r of row c at r * BN + c
    for (int r = g + 2 * w; r <= K; r += 2 * FWD_NW) trow[r * BN] = grid_value<CAL>(M, m, K, a.tau, r);
  } else if (CAL != EXPB) {  // the exponential baselines have no grid
    trow = tbl + a.lres;
    for (int i = threadIdx.x; i <= a.lres + K; i += FWD_NT) tbl[i] = grid_value<CAL>(M, m, K, a.tau, i - a.lres);
  }
  __syncthreads();

  // The lowest stored score whose weight can reach thrL (w^L) or thrN (w^N, Nearest), or `loose`
  // where the grid cannot tell (a bound that holds on every grid).  The weights rise with u, so
  // the grid inverted at the threshold gives it; a margin of 1e-3 interval widths, or 1e-3 of a
  // score unit for softmax, covers the roundings of the inversion and of the float decisions.
  const double hgrid = CAL == EXPB ? 0.0 : 1.0 / rc.inv_h;
  auto lowest_score = [&](double thrL, double thrN, float loose) -> float {
    if constexpr (CAL == EXPB) {
      return fmaxf(loose, (float)((double)M + log(thrL) - 1e-3));
    } else if constexpr (CAL == MINMAX || CAL == FWM || CAL == FWM_FLOOR) {
      constexpr int ST = CAL == MINMAX ? BN : 1;
      // interval r with E_r < thr <= E_{r+1} (E rises with r), or -1 (thr <= E_0), or K (thr > E_K)
      auto interval = [&](double thr) {
        if (thr <= (double)trow[0]) return -1;
        if (thr > (double)trow[K * ST]) return K;
        int lo = 0, hi = K;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if ((double)trow[mid * ST] < thr) lo = mid;
          else hi = mid;
        }
        return lo;
      };
      // LERP: the u at which the interpolated weight reaches the threshold
      const int rL = interval(thrL);
      double ustar = rL < 0 ? -1.0
                     : rL >= K ? (double)K + 1.0
                               : rL + (thrL - (double)trow[rL * ST]) /
                                          ((double)trow[(rL + 1) * ST] - (double)trow[rL * ST]);
      if (is_nearest(MODE)) {  // Nearest: a weight E_rho with E_rho >= thr from u >= rho - 1/2
        const int rN = interval(thrN);
        ustar = fmin(ustar, rN < 0 ? -1.0 : rN + 0.5);
      }
      const bool regular = CAL != MINMAX || rc.kappa != 0.f;
      return regular && ustar >= 0.0 ? fmaxf(loose, (float)((double)M - ((double)K - ustar + 1e-3) * hgrid)) : loose;
    } else {
      return loose;
    }
  };
  // Long rows (fp32 inputs): pass 2 flags, per wave, the key tiles holding a key that can be heavy
  // for any row sum (W >= 1: the maximum weighs 1), so that the heavy-key stage reads only those
  constexpr bool HFLAG = MODE != BINM && MODE != EXPBF && MODE != EXPF8 && std::is_same_v<TIn, float>;
  const bool track = HFLAG && ntiles > 2 * 32;
  if (track) {
    if (w == 0 && g == 0)
      sm.sflag[c] = qvalid ? lowest_score(1.0 / (HEAVY_INV * (1.0 + 1e-3)), 1.0 / (HEAVY_INV * (1.0 + 1e-3)),
                                          (float)((double)M - log(HEAVY_INV * (1.0 + 1e-3)) - hgrid) - Erow)
                           : INFINITY;
    if (l < 4) sm.tflag[w][l] = 0u;
    __syncthreads();
  }

  // ---- pass 2: reconstruct, normalize, multiply by V
  double sumL = 0.0, sumN = 0.0;  // row sums of positive weights: double, no absorption of small terms
  f16v o[D / 32], ol[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) { o[nb] = zero16(); ol[nb] = zero16(); }
  // DRUN: the running sum in double, in the layout of o
  double od[DRUN ? D / 32 : 1][DRUN ? 16 : 1];
  if constexpr (DRUN) {
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) od[nb][v] = 0.0;
  }
  // F64: the double accumulator, element i of block (qh, nb): row 16 qh + l/16 + 4 i, column 16 nb + l%16
  d4v o64[F64 ? 2 : 1][F64 ? D / 16 : 1];
  if constexpr (F64) {
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) { o64[0][nb] = zero4d(); o64[1][nb] = zero4d(); }
  }
  // the next V tile is loaded while this one computes, except under Nearest with Prob-STE,
  // whose second output accumulator takes those registers: there the tile's own V is loaded
  // first, arrives while both half tiles are weighed, and is staged before their products
  constexpr bool VPRE = MODE != NEAREST_P;
  float s[16];  // this lane's scores of the tile, as it stored them in pass 1
  auto load_scores = [&](int kt) {
    const float* St = Sh + tile_index(qt, kt, nt, a.causal) * 1024 + l;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = St[v * 64];
  };
  // without the V prefetch, the next tile's scores are requested once this tile is weighed
  if (!VPRE && w < ntiles) load_scores(w);
  for (int kt = w; kt < ntiles; kt += FWD_NW) {
    const int k0 = kt * BN;
    if (!VPRE) vr.load(Vp, k0, T);
    float* Sw = Sh + tile_index(qt, kt, nt, a.causal) * 1024 + l;
    if (VPRE) load_scores(kt);
    if (VPRE) {
      if constexpr (F64) vr.store_f32(VF, vfs<D>());
      else vr.template store_t<NS>(VT);
      wave_lds_sync();
      if (kt + FWD_NW < ntiles) vr.load(Vp, k0 + FWD_NW * BN, T);  // next V tile in flight
    }
    const bool full = full_tile(kt);
    // each tile's P V (bf16 slice products on the matrix pipe) goes into a fresh accumulator,
    // then into the running sum: the long accumulation chain then holds one add per tile
    // (DRUN under Nearest with Prob-STE: O^L's tile product reuses ot once O's has joined o)
    constexpr int NOTL = MODE == NEAREST_P && !DRUN ? D / 32 : 1;
    f16v ot[D / 32], otl[NOTL];
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) ot[nb] = zero16();
#pragma unroll
    for (int nb = 0; nb < NOTL; ++nb) otl[nb] = zero16();
    // without the prefetch: the weights of both half tiles, kept until V is staged
    float pa[VPRE ? 1 : 2][8], pla[VPRE ? 1 : 2][8];
#pragma unroll
    for (int b = 0; b < 2; ++b) {  // half tiles: keys crow(v, g) for v = 8b .. 8b+7
      // the half tile's V^T operands are read from LDS first, so that their latency overlaps the
      // weighing (not under Nearest with Prob-STE, whose second accumulator takes the registers)
      Split8 vb[D / 32];
      if (MODE != NEAREST_P && !F64) {
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) vb[nb] = load_bt<D, NS>(VT, b, 32 * nb + c);
        __builtin_amdgcn_sched_barrier(0);
      }
      float p[8], pl[8];
      // the half tile's weight sums: eight positive terms summed in float (error at most 7 u of
      // the half tile's sum, no absorption across the row), joined to the row sums in double once
      // the half tile is settled
      std::conditional_t<F64, double, float> tL, tN;  // F64: the exact weights' sums in double
      uint32_t risky = 0;
      uint32_t riske = 0;  // exponential baselines: keys whose weight alone is taken again
      auto weigh = [&](auto masked, auto check) {
        tL = 0.f;
        tN = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int v = 8 * b + j, key = k0 + crow(v, g);
          const bool ok = !decltype(masked)::value || (qvalid & (key < T) & (!a.causal | (key <= qi)));
          float wl, wn;
          if constexpr (CAL == EXPB) {
            // exponential baselines: first pass in float, checked against the score's error bound;
            // again: the exact rounding
            bool rs = false, re = false;
            const ExpW ew = decltype(check)::value ? exp_weight_fast<MODE>(s[v], M, Erow, &rs, &re)
                                                   : exp_weight_exact<MODE>(s[v], M);
            if (decltype(check)::value) {
              risky |= (ok && rs) ? (1u << j) : 0u;
              riske |= (ok && re && !rs) ? (1u << j) : 0u;
            }
            wl = ok ? ew.w : 0.f;
            wn = wl;
          } else {
            // first pass: float arithmetic, checked against the margin.  Again (a half tile with a key
            // the margin could not settle): that key's decision in double on its exact score, the
            // others' as before (so that a key's weight is always the float form on its stored score
            // unless that score was retaken)
            const bool exact_d = !decltype(check)::value && ((risky >> j) & 1u);
            const Decision d = exact_d ? decide<CAL>(s[v], rc, K, a.tau) : decide_fast<CAL>(s[v], rc, K, a.tau);
            if (decltype(check)::value) {
              // a decision within the score's error bound of a boundary must be taken on the exact
              // score (interior boundaries: 1 .. K-1, every integer below K on the resolved grid).
              // Bitwise operators: every test is cheap, and short-circuit forms become branches.
              const float dur = CAL == FWM_RES ? fmaf((float)max(-d.r, 0), 0x1p-22f, du) : du;
              bool r = ((d.t < dur) & (CAL == FWM_RES || d.r > 0)) | ((d.t > 1.f - dur) & (d.r < K - 1));
              if (is_nearest(MODE)) r |= fabsf(d.t - 0.5f) < dur;
              if (CAL == FWM || CAL == FWM_FLOOR) r |= fabsf((s[v] - M) + a.tau) <= edge;
              risky |= (ok & r) ? (1u << j) : 0u;
            }
            constexpr int ST = (CAL == MINMAX || MODE == BINM) ? BN : 1;
            const Weights wt = weights_cal<CAL, ST>(d, trow, a.lres, a.res_far != 0, K, a.tau);
            // a floored tail key keeps the weight of the window edge (r = 0, t = 0)
            const bool keep = ok && (CAL == FWM_FLOOR || !d.tail);
            wl = keep ? wt.wL : 0.f;
            wn = keep ? wt.wN : 0.f;
          }
          tL += wl;
          if (is_nearest(MODE)) tN += wn;
          p[j] = is_nearest(MODE) ? wn : wl;
          pl[j] = wl;
        }
      };
      if (full) weigh(std::false_type{}, std::true_type{});
      else weigh(std::true_type{}, std::true_type{});
      if (__any((risky | riske) != 0u)) {
        // rare: the exact scores replace the stored ones (this lane stored them) for every later
        // pass, and the half tile is weighed again on them (the exponential baselines weigh only
        // the keys concerned again: their weights do not depend on one another; a key in riske
        // keeps its score and has its weight taken in exact form)
        uint32_t bits = risky | riske;
        while (__any(bits != 0u)) {
          const int j = bits ? __builtin_ctz(bits) : 0;
          if (bits) {
            float xe = s[8 * b];
#pragma unroll
            for (int jj = 1; jj < 8; ++jj) xe = jj == j ? s[8 * b + jj] : xe;
            if ((risky >> j) & 1u) {
              xe = exact_score<D, TIn>(qrow, Kp + (size_t)(k0 + crow(8 * b + j, g)) * D, a.scale);
              Sw[(8 * b + j) * 64] = xe;
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) s[8 * b + jj] = jj == j ? xe : s[8 * b + jj];
            }
            if constexpr (CAL == EXPB) {
              const float we = exp_weight_exact<MODE>(xe, M).w;
              float old = 0.f;
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) {
                old = jj == j ? p[jj] : old;
                p[jj] = jj == j ? we : p[jj];
                pl[jj] = jj == j ? we : pl[jj];
              }
              tL += (decltype(tL))we - (decltype(tL))old;
            }
            bits &= bits - 1u;
          }
        }
        if constexpr (CAL != EXPB) {
          if (full) weigh(std::false_type{}, std::false_type{});
          else weigh(std::true_type{}, std::false_type{});
        }
      }
      sumL += (double)tL;
      sumN += (double)tN;
      if constexpr (!VPRE) {
#pragma unroll
        for (int j = 0; j < 8; ++j) { pa[b][j] = p[j]; pla[b][j] = pl[j]; }
        continue;
      }
      if constexpr (F64) {  // the tile's weights as rows of queries
#pragma unroll
        for (int j = 0; j < 8; ++j) PT[c * PTS + crow(8 * b + j, g)] = p[j];
        continue;
      }
      const Split8 ps = split8(p);
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) ot[nb] = mfma_split<NS>(ps, vb[nb], ot[nb]);
    }
    if (track) {  // (before the next tile's scores replace this one's)
      float mx = s[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[v]);
      const int it = (kt - w) / FWD_NW;
      if (__ballot(mx >= sm.sflag[c]) != 0ull && it < 128 && l == 0) sm.tflag[w][it >> 5] |= 1u << (it & 31);
    }
    if constexpr (F64) {
      // O += P V in double: A = the weights (query l%16 of the block, key 4 s4 + l/16), B = V
      wave_lds_sync();
      const int m16 = l & 15, k4 = l >> 4;
#pragma unroll
      for (int s4 = 0; s4 < 8; ++s4) {
        const int kk = 4 * s4 + k4;
        const double a0 = PT[m16 * PTS + kk], a1 = PT[(16 + m16) * PTS + kk];
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
          const double bv = VF[kk * vfs<D>() + 16 * nb + m16];
          o64[0][nb] = mfma_f64(a0, bv, o64[0][nb]);
          o64[1][nb] = mfma_f64(a1, bv, o64[1][nb]);
        }
      }
    }
    if constexpr (!VPRE) {
      if (kt + FWD_NW < ntiles) load_scores(kt + FWD_NW);
      vr.template store_t<NS>(VT);
      wave_lds_sync();
      if constexpr (DRUN) {
        // O's product, into o; then O^L's in the same registers, into the double running sum
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const Split8 ps = split8(pa[b]);
#pragma unroll
          for (int nb = 0; nb < D / 32; ++nb) ot[nb] = mfma_split<NS>(ps, load_bt<D, NS>(VT, b, 32 * nb + c), ot[nb]);
        }
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) { o[nb] += ot[nb]; ot[nb] = zero16(); }
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const Split8 psl = split8(pla[b]);
#pragma unroll
          for (int nb = 0; nb < D / 32; ++nb) ot[nb] = mfma_split<NS>(psl, load_bt<D, NS>(VT, b, 32 * nb + c), ot[nb]);
        }
      } else {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          Split8 vb[D / 32];
#pragma unroll
          for (int nb = 0; nb < D / 32; ++nb) vb[nb] = load_bt<D, NS>(VT, b, 32 * nb + c);
          const Split8 ps = split8(pa[b]);
#pragma unroll
          for (int nb = 0; nb < D / 32; ++nb) ot[nb] = mfma_split<NS>(ps, vb[nb], ot[nb]);
          const Split8 psl = split8(pla[b]);
#pragma unroll
          for (int nb = 0; nb < NOTL; ++nb) otl[nb] = mfma_split<NS>(psl, vb[nb], otl[nb]);
        }
      }
    }
    if constexpr (DRUN) {
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) od[nb][v] += (double)ot[nb][v];
    } else if constexpr (!F64) {
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) {
        o[nb] += ot[nb];
        if (MODE == NEAREST_P) ol[nb] += otl[nb % NOTL];
      }
    }
    wave_lds_sync();  // this tile's V^T reads come before the next tile's staging
  }

  // ---- the waves' partial row sums and outputs meet in LDS; wave 0 adds them in wave order
  sumL += __shfl_xor(sumL, 32);
  sumN += __shfl_xor(sumN, 32);
  if (g == 0) {
    sm.sL[w][c] = sumL;
    sm.sN[w][c] = sumN;
  }

  // ---- heavy keys.  The faster scores are within Erow of the exact ones, and every decision is
  // the exact scores' one, but a key that carries much of its row's probability passes a few fp32
  // ulps of score error into the output and, through D_i = dO_i . O_i, into every score gradient
  // of the row (the row maximum's calibration term and the outputs with cancelling terms are the
  // most sensitive).  Once the row sums are known, a row whose largest probability can reach
  // 1/HEAVY_INV (every weight is at most 1, so W <= HEAVY_INV) recomputes the exact score of each
  // key that can carry that much (its LERP weight is at most e^{z + h}: z >= ln(W / HEAVY_INV) - h),
  // patches it into the stored tile for the backward, and records the change of its continuous
  // weight (w^L, or softmax's e^z) for the output.  Bin mean sums its bins before pass 2 and keeps
  // its faster scores; the rounded exponentials (BF16-exp, FP8) have taken every weight exactly.
  constexpr bool HEAVY = MODE != BINM && MODE != EXPBF && MODE != EXPF8;
  // whether a heavy key's weight change reaches the output (the continuous weight: w^L, or e^z)
  constexpr bool HCORR = MODE == LERP || MODE == EXP32 || MODE == NEAREST_P;
  // fp32 inputs take the heavy keys in batches: found first, then their exact scores with every
  // load of a batch in flight, then their weight changes summed per output row in LDS and added to
  // the accumulators once.  bfloat16 inputs take them one key at a time (a key's exact score and
  // correction before the next).
  constexpr bool HBATCH = std::is_same_v<TIn, float>;
  double hsum = 0.0;  // batched: the weight changes of this lane's heavy keys (all in its own row)
  int nh_any = 0;     // one at a time: whether this lane retook a heavy key
  if constexpr (HEAVY && HBATCH) {
    __syncthreads();
    double WLr = 0.0, WNr = 0.0;
#pragma unroll
    for (int u = 0; u < FWD_NW; ++u) {
      WLr += sm.sL[u][c];
      WNr += sm.sN[u][c];
    }
    const double Wmin = is_nearest(MODE) ? fmin(WLr, WNr) : WLr;
    const bool maybe = qvalid && Wmin <= HEAVY_INV * (1.0 + 1e-3);
    // (the same margin as the heavy test below)
    const float s_thr =
        maybe ? (float)((double)M + log(Wmin / (HEAVY_INV * (1.0 + 1e-3))) - hgrid) - Erow : INFINITY;
    if (__any(maybe)) {
      // (a) the heavy keys, found on the stored scores (the next tile's scores are in flight while
      // one is tested); up to HMAX per lane, with their stored scores
      int nh = 0;
      // The lowest stored score that the heavy test below can accept.  The bound above holds on
      // every grid; where the weight threshold falls inside the grid, the grid inverted at it gives
      // a tighter one (the weights rise with u; a margin of 1e-3 interval widths, or 1e-3 of a
      // score unit for softmax, covers the roundings of the inversion and of the float decisions).
      const float s_cand =
          maybe ? lowest_score(WLr / (HEAVY_INV * (1.0 + 1e-3)), WNr / (HEAVY_INV * (1.0 + 1e-3)), s_thr) : INFINITY;
      float sc[16], sn[16];
      auto load16 = [&](float(&dst)[16], int kt) {
        const float* St = Sh + tile_index(qt, kt, nt, a.causal) * 1024 + l;
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[v] = St[v * 64];
      };
      // the wave's tiles that pass 2 flagged (every tile where it flagged none)
      auto visit = [&](int kt) {
        const int it = (kt - w) / FWD_NW;
        return !track || it >= 128 || ((sm.tflag[w][it >> 5] >> (it & 31)) & 1u) != 0u;
      };
      auto next_visit = [&](int kt) {
        for (kt += FWD_NW; kt < ntiles && !visit(kt); kt += FWD_NW) {
        }
        return kt;
      };
      int kt = w < ntiles && visit(w) ? w : next_visit(w);
      if (kt < ntiles) load16(sc, kt);
      while (kt < ntiles) {
        const int kn = next_visit(kt);
        const bool more = kn < ntiles;
        if (more) load16(sn, kn);
        const int k0 = kt * BN;
        uint32_t bits = 0u;
        // candidates (a lane without a possible heavy key has s_cand = infinity); the extremum
        // keys' stored scores are exact already
        if (full_tile(kt)) {
#pragma unroll
          for (int v = 0; v < 16; ++v) bits |= (sc[v] >= s_cand && sc[v] != M) ? (1u << v) : 0u;
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = k0 + crow(v, g);
            const bool ok = (key < T) & (!a.causal | (key <= qi));
            bits |= (ok && sc[v] >= s_cand && sc[v] != M) ? (1u << v) : 0u;
          }
        }
        while (__any(bits != 0u)) {
          const int j = bits ? __builtin_ctz(bits) : 0;
          if (bits) {
            bits &= bits - 1u;
            float old = sc[0];
#pragma unroll
            for (int v = 1; v < 16; ++v) old = v == j ? sc[v] : old;
            // the key's probability under either normalizer, from its faster score (a margin of
            // 1e-3 for that score's error)
            bool heavy;
            if constexpr (CAL == EXPB) {
              heavy = (double)__expf(old - M) * (HEAVY_INV * (1.0 + 1e-3)) >= WLr;
            } else {
              constexpr int ST = CAL == MINMAX ? BN : 1;
              const Weights w0 = weights_cal<CAL, ST>(decide<CAL>(old, rc, K, a.tau), trow, a.lres, a.res_far != 0,
                                                       K, a.tau);
              heavy = (double)w0.wL * (HEAVY_INV * (1.0 + 1e-3)) >= WLr ||
                      (is_nearest(MODE) && (double)w0.wN * (HEAVY_INV * (1.0 + 1e-3)) >= WNr);
            }
            if (heavy && nh < HMAX) {
              sm.hk[w][l][nh] = k0 + crow(j, g);
              sm.hd[w][l][nh] = old;
              ++nh;
            }
          }
        }
        if (more) {
#pragma unroll
          for (int v = 0; v < 16; ++v) sc[v] = sn[v];
        }
        kt = kn;
      }
      // the wave's heavy keys as one list in its LDS region (V^T is no longer read): lane order
      int incl = nh;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(incl, d);
        if (l >= d) incl += t;
      }
      const int off = incl - nh;
      const int total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
      int* fk = reinterpret_cast<int*>(sm.wave[w]);  // key
      int* fr = fk + 64 * HMAX;                       // query row in the tile
      float* fx = reinterpret_cast<float*>(fr + 64 * HMAX);  // exact score, then weight change
      for (int x = 0; x < nh; ++x) {
        fk[off + x] = sm.hk[w][l][x];
        fr[off + x] = c;
      }
      wave_lds_sync();
      // (b) their exact scores (double products and sums, double scale, one rounding), LPK lanes
      // to a key: each lane sums 32 products, then the lanes' sums are added across the group;
      // every load of a batch of 64 / LPK keys is in flight at once
      constexpr int LPK = D / 32;
      const TIn* Qh = reinterpret_cast<const TIn*>(a.q) + hb;
      for (int e0 = 0; e0 < total; e0 += 64 / LPK) {
        const int e = e0 + l / LPK, part = l % LPK;
        const int ee = e < total ? e : e0;  // a spare lane repeats a listed key (in bounds)
        const TIn* qp = Qh + (size_t)(q0 + fr[ee]) * D + 32 * part;
        const TIn* kp = Kp + (size_t)fk[ee] * D + 32 * part;
        f4v xq[8], yk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          xq[i] = Ld<TIn>::four(qp + 4 * i);
          yk[i] = Ld<TIn>::four(kp + 4 * i);
        }
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int k = 0; k < 4; ++k) acc = fma((double)xq[i][k], (double)yk[i][k], acc);
#pragma unroll
        for (int s = LPK / 2; s >= 1; s >>= 1) acc += __shfl_xor(acc, s);
        if (e < total && part == 0) fx[e] = (float)(a.scale * acc);
      }
      wave_lds_sync();
      // (c) each lane patches its keys' exact scores into the tiles it stored (for the backward)
      // and takes the change of each continuous weight: pass 2 weighed the key with the float
      // decision on its stored score (the decision itself is the same: pass 2 settled it against
      // the bound)
      for (int x = 0; x < nh; ++x) {
        const float xe = fx[off + x], old = sm.hd[w][l][x];
        float dw = 0.f;
        if (xe != old) {
          const int key = fk[off + x];
          Sh[stored_at(key)] = xe;
          if constexpr (MODE == EXP32) {
            dw = __expf(xe - M) - __expf(old - M);
          } else if constexpr (MODE == LERP || MODE == NEAREST_P) {
            constexpr int ST = CAL == MINMAX ? BN : 1;
            const Decision d0 = decide_fast<CAL>(old, rc, K, a.tau), d1 = decide<CAL>(xe, rc, K, a.tau);
            const bool keep = CAL == FWM_FLOOR || !d0.tail;
            dw = keep ? weights_cal<CAL, ST>(d1, trow, a.lres, a.res_far != 0, K, a.tau).wL -
                            weights_cal<CAL, ST>(d0, trow, a.lres, a.res_far != 0, K, a.tau).wL
                      : 0.f;
          }
        }
        fx[off + x] = dw;
        hsum += (double)dw;
      }
      if constexpr (HCORR) {
        // (d) the weight changes into this wave's output rows (O, or O^L under Nearest with
        // Prob-STE): summed per row in an LDS tile in list order (lane l takes columns l + 64 i;
        // the V rows of eight keys are loaded together), then added to the accumulators once.
        // Lane (c, g) holds row crow(v, g) of the tile at columns 32 nb + c.
        constexpr int DS = D + 4;  // row stride of the correction tile
        float* dO = fx + 64 * HMAX;
#pragma unroll
        for (int i = 4 * l; i < 32 * DS; i += 256) *reinterpret_cast<f4v*>(dO + i) = f4v{0.f, 0.f, 0.f, 0.f};
        wave_lds_sync();
        constexpr int EB = 8;
        for (int e0 = 0; e0 < total; e0 += EB) {
          float vv[EB][D / 64];
#pragma unroll
          for (int j = 0; j < EB; ++j) {
            const TIn* vp = Vp + (size_t)fk[e0 + j < total ? e0 + j : e0] * D + l;
#pragma unroll
            for (int i = 0; i < D / 64; ++i) vv[j][i] = Ld<TIn>::one(vp + 64 * i);
          }
#pragma unroll
          for (int j = 0; j < EB; ++j) {
            if (e0 + j < total) {
              const float dw = fx[e0 + j];
              float* row = dO + fr[e0 + j] * DS + l;
#pragma unroll
              for (int i = 0; i < D / 64; ++i) row[64 * i] = fmaf(dw, vv[j][i], row[64 * i]);
            }
          }
        }
        wave_lds_sync();
        f16v(&acc)[D / 32] = MODE == NEAREST_P ? ol : o;  // DRUN: od
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float* row = dO + crow(v, g) * DS + c;
#pragma unroll
          for (int nb = 0; nb < D / 32; ++nb) {
            if constexpr (DRUN) od[nb][v] += (double)row[32 * nb];
            else acc[nb][v] += row[32 * nb];
          }
        }
      }
    }
    hsum += __shfl_xor(hsum, 32);
    if (g == 0) sm.hs[w][c] = hsum;
  } else if constexpr (HEAVY) {
    __syncthreads();
    double WLr = 0.0, WNr = 0.0;
#pragma unroll
    for (int u = 0; u < FWD_NW; ++u) {
      WLr += sm.sL[u][c];
      WNr += sm.sN[u][c];
    }
    const double Wmin = is_nearest(MODE) ? fmin(WLr, WNr) : WLr;
    const bool maybe = qvalid && Wmin <= HEAVY_INV;
    const double hgrid = CAL == EXPB ? 0.0 : 1.0 / rc.inv_h;
    const float s_thr = maybe ? (float)((double)M + log(Wmin / HEAVY_INV) - hgrid) - Erow : INFINITY;
    int nh = 0;
    if (__any(maybe)) {
      for (int kt = w; kt < ntiles; kt += FWD_NW) {
        const int k0 = kt * BN;
        float* Sw = Sh + tile_index(qt, kt, nt, a.causal) * 1024 + l;
        uint32_t bits = 0u;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = k0 + crow(v, g);
          const bool ok = maybe & (key < T) & (!a.causal | (key <= qi));
          const float x = Sw[v * 64];
          // the extremum keys' stored scores are exact already
          bits |= (ok && x >= s_thr && x != M) ? (1u << v) : 0u;
        }
        while (__any(bits != 0u)) {
          const int j = bits ? __builtin_ctz(bits) : 0;
          if (bits) {
            bits &= bits - 1u;
            const float old = Sw[j * 64];
            const int key = k0 + crow(j, g);
            // the key's probability under either normalizer, from its faster score (a margin of
            // 1e-3 for that score's error)
            bool heavy;
            if constexpr (CAL == EXPB) {
              heavy = (double)__expf(old - M) * (HEAVY_INV * (1.0 + 1e-3)) >= WLr;
            } else {
              constexpr int ST = CAL == MINMAX ? BN : 1;
              const Weights w0 = weights_cal<CAL, ST>(decide<CAL>(old, rc, K, a.tau), trow, a.lres, a.res_far != 0,
                                                       K, a.tau);
              heavy = (double)w0.wL * (HEAVY_INV * (1.0 + 1e-3)) >= WLr ||
                      (is_nearest(MODE) && (double)w0.wN * (HEAVY_INV * (1.0 + 1e-3)) >= WNr);
            }
            // (a lean form: the output accumulators are live here)
            const float xe = heavy && nh < HMAX ? exact_score<D, TIn, 2>(qrow, Kp + (size_t)key * D, a.scale) : old;
            if (xe != old) {
              // the change of the continuous weight, computed as pass 2 computed the old one (the
              // decision itself is the same: pass 2 settled it against the bound)
              float dw = 0.f;
              if constexpr (MODE == EXP32) {
                dw = __expf(xe - M) - __expf(old - M);
              } else if constexpr (MODE == LERP || MODE == NEAREST_P) {
                // pass 2 weighed the key with the float decision on its stored score
                constexpr int ST = CAL == MINMAX ? BN : 1;
                const Decision d0 = decide_fast<CAL>(old, rc, K, a.tau), d1 = decide<CAL>(xe, rc, K, a.tau);
                const bool keep = CAL == FWM_FLOOR || !d0.tail;
                dw = keep ? weights_cal<CAL, ST>(d1, trow, a.lres, a.res_far != 0, K, a.tau).wL -
                                weights_cal<CAL, ST>(d0, trow, a.lres, a.res_far != 0, K, a.tau).wL
                          : 0.f;
              }
              Sw[j * 64] = xe;  // stored by this lane in pass 1
              sm.hk[w][l][nh] = key;
              sm.hd[w][l][nh] = dw;
              ++nh;
            }
          }
        }
      }
    }
    sm.hn[w][l] = nh;
    nh_any = nh;
  }
  float* part = reinterpret_cast<float*>(sm.wave[w]);  // this wave's V^T is no longer read
  auto gather = [&](f16v (&acc)[D / 32]) {
    __syncthreads();
    if (w > 0) {
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) part[(nb * 16 + v) * 64 + l] = acc[nb][v];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int u = 1; u < FWD_NW; ++u) {
        const float* op = reinterpret_cast<const float*>(sm.wave[u]);
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[nb][v] += op[(nb * 16 + v) * 64 + l];
      }
    }
  };
  // one key at a time: whether any lane of the workgroup retook a heavy key (a barrier, which also
  // orders the slots)
  bool anyheavy = false;
  if constexpr (HEAVY && !HBATCH) anyheavy = __syncthreads_or(nh_any);
  if constexpr (F64) {
    double* pd = reinterpret_cast<double*>(sm.wave[w]);
    __syncthreads();
    if (w > 0) {
#pragma unroll
      for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) pd[((qh * (D / 16) + nb) * 4 + i) * 64 + l] = o64[qh][nb][i];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int u = 1; u < FWD_NW; ++u) {
        const double* op = reinterpret_cast<const double*>(sm.wave[u]);
#pragma unroll
        for (int qh = 0; qh < 2; ++qh)
#pragma unroll
          for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) o64[qh][nb][i] += op[((qh * (D / 16) + nb) * 4 + i) * 64 + l];
      }
    }
  } else if constexpr (DRUN) {
    double* pd = reinterpret_cast<double*>(sm.wave[w]);
    __syncthreads();
    if (w > 0) {
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) pd[(nb * 16 + v) * 64 + l] = od[nb][v];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int u = 1; u < FWD_NW; ++u) {
        const double* op = reinterpret_cast<const double*>(sm.wave[u]);
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
          for (int v = 0; v < 16; ++v) od[nb][v] += op[(nb * 16 + v) * 64 + l];
      }
    }
    if (MODE == NEAREST_P) gather(o);
  } else {
    gather(o);
    if (MODE == NEAREST_P) gather(ol);
  }
  if (w != 0) return;
  sumL = sm.sL[0][c];
  sumN = sm.sN[0][c];
#pragma unroll
  for (int u = 1; u < FWD_NW; ++u) {
    sumL += sm.sL[u][c];
    sumN += sm.sN[u][c];
  }
  if constexpr (HEAVY && HBATCH) {
#pragma unroll
    for (int u = 0; u < FWD_NW; ++u) sumL += sm.hs[u][c];  // the heavy keys' weight changes (W^L, softmax's W)
  }
  if (HEAVY && !HBATCH && HCORR && anyheavy) {
    // the heavy keys' weight changes, in a fixed order (waves, lanes, slots): into the continuous
    // row sum (W^L, softmax's W) and into the output rows (O, or O^L under Nearest with Prob-STE).
    // Lane (c, g) holds output row crow(v, g) of the tile at columns 32 nb + c.
    f16v(&acc)[D / 32] = MODE == NEAREST_P ? ol : o;  // DRUN: od
    for (int u = 0; u < FWD_NW; ++u)
      for (int hl = 0; hl < 64; ++hl) {
        const int n = sm.hn[u][hl];
        const int r = hl & 31, gr = (r >> 2) & 1, vr_ = 4 * (r >> 3) + (r & 3);  // crow(vr_, gr) == r
        for (int x = 0; x < n; ++x) {
          const int key = sm.hk[u][hl][x];
          const float dw = sm.hd[u][hl][x];
          if (c == r) sumL += (double)dw;
          float vv[D / 32];
#pragma unroll
          for (int nb = 0; nb < D / 32; ++nb) vv[nb] = Ld<TIn>::one(Vp + (size_t)key * D + 32 * nb + c);
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (v == vr_ && g == gr) {
#pragma unroll
              for (int nb = 0; nb < D / 32; ++nb) {
                if (DRUN) od[nb][v] = fma((double)dw, (double)vv[nb], od[nb][v]);
                else acc[nb][v] = fmaf(dw, vv[nb], acc[nb][v]);
              }
            }
        }
      }
  }
  const float WLf = (float)sumL, WNf = is_nearest(MODE) ? (float)sumN : WLf;
  if (g == 0) {
    sm.rowW[c] = is_nearest(MODE) ? WNf : WLf;
    sm.rowWL[c] = WLf;
    sm.rowWd[c] = is_nearest(MODE) ? sumN : sumL;
    sm.rowWLd[c] = sumL;
    if (qvalid) {
      const size_t row = (size_t)head * T + qi;
      // F64: W^N holds the residual of W, so that W^L + W^N is the double sum
      a.rec.WN[row] = F64 ? (float)(sumL - (double)WLf) : WNf;
      a.rec.WL[row] = WLf;
    }
  }
  wave_lds_sync();
  if constexpr (F64) {
    // O = num / W in double, stored as its float and the residual (in the O^L slot of the record)
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * qh + (l >> 4) + 4 * i, qrow = q0 + r;
        if (qrow < T) {
          const double Wd = sm.rowWd[r];
          const size_t at = hb + (size_t)qrow * D + (l & 15);
#pragma unroll
          for (int nb = 0; nb < D / 16; ++nb) {
            const double ov = o64[qh][nb][i] / Wd;
            const float hi = (float)ov;
            a.o[at + 16 * nb] = hi;
            a.rec.OL[at + 16 * nb] = (float)(ov - (double)hi);
          }
        }
      }
    return;
  }
  // O = num / W; lane l holds rows crow(v, g) of the tile and columns 32 nb + c
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int qrow = q0 + crow(v, g);
    if (qrow < T) {
      const float inv = 1.0f / sm.rowW[crow(v, g)];
      float* orow = a.o + hb + (size_t)qrow * D + c;
      if (DRUN && MODE != NEAREST_P) {
        // the double sum over the double row sum, rounded once
        const double Wd = sm.rowWd[crow(v, g)];
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) orow[32 * nb] = (float)(od[nb][v] / Wd);
      } else {
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) orow[32 * nb] = o[nb][v] * inv;
      }
      if (MODE == NEAREST_P) {
        const float invl = 1.0f / sm.rowWL[crow(v, g)];
        float* olrow = a.rec.OL + hb + (size_t)qrow * D + c;
        if (DRUN) {
          const double Wd = sm.rowWLd[crow(v, g)];
#pragma unroll
          for (int nb = 0; nb < D / 32; ++nb) olrow[32 * nb] = (float)(od[nb][v] / Wd);
        } else {
#pragma unroll
          for (int nb = 0; nb < D / 32; ++nb) olrow[32 * nb] = ol[nb][v] * invl;
        }
      }
    }
  }
}

template <int D, int CAL, int MODE, typename TIn>
size_t fwd_smem_bytes(int K, int lres) {
  return sizeof(FwdSmem<D, nslices<TIn>(), MODE == EXPBF>) +
         sizeof(float) * (CAL == MINMAX || MODE == BINM ? BN * (K + 1) : (CAL == EXPB ? 0 : lres + K + 1));
}
static_assert(sizeof(float) * 2 * BINM_MAXB * BN * FWD_NW <= FWD_NW * fwd_wave_bytes<64, 1, false>(),
              "bin-mean partial sums fit the V^T staging area");
static_assert(3 * 64 * HMAX * 4 + 32 * (64 + 4) * 4 <= fwd_wave_bytes<64, 3, false>() &&
                  3 * 64 * HMAX * 4 + 32 * (128 + 4) * 4 <= fwd_wave_bytes<128, 3, false>(),
              "a wave's heavy-key list and correction tile fit its staging area (fp32 inputs)");

// Test hook: the bin decision of every (query, key) pair, from the stored scores and row record.
template <int CAL, int MODE>
__global__ __launch_bounds__(256) void bins_kernel(BinsArgs a) {
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 5, c = l & 31;
  const int T = a.T, K = a.K, nt = a.rec.nt;
  const int L = blockIdx.x;
  const int head = L / nt, qt = L % nt;
  const int qi = qt * BN + c;
  const bool qvalid = qi < T;
  const size_t row = (size_t)head * T + (qvalid ? qi : 0);
  const RowCal rc = row_calibration<CAL>(a.rec.M[row], a.rec.m[row], K, a.tau);
  const float* Sh = a.rec.S + (size_t)head * a.rec.tiles_per_head * 1024;
  const int kt_end = a.causal ? qt + 1 : nt;
  for (int kt = w; kt < nt; kt += 4) {
    const bool stored = kt < kt_end;
    const float* St = Sh + (stored ? tile_index(qt, kt, nt, a.causal) : 0) * 1024;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = kt * BN + crow(v, g);
      if (!qvalid || key >= T) continue;
      const bool ok = stored && (!a.causal || key <= qi);
      uint8_t val = 255;
      if (ok) {
        if constexpr (CAL == EXPB) {
          // exponential baselines: the E4M3 byte of the weight (FP8), the low byte of the
          // bfloat16 weight (BF16), 0 (softmax)
          const float M = a.rec.M[row];
          if (MODE == EXPF8) val = (uint8_t)e4m3_code(exp_weight_exact<EXPF8>(St[v * 64 + l], M).w);
          else if (MODE == EXPBF) val = (uint8_t)(__float_as_uint(exp_weight_exact<EXPBF>(St[v * 64 + l], M).w) >> 16);
          else val = 0;
        } else {
          const Decision d = decide<CAL>(St[v * 64 + l], rc, K, a.tau);
          const int idx = MODE == LERP ? d.r : d.r + (d.t >= 0.5f ? 1 : 0);
          // resolved grid: the index + 64, indices below -64 sharing the value 0
          val = d.tail ? 254 : (uint8_t)(CAL == FWM_RES ? max(idx + 64, 0) : idx);
        }
      }
      a.bins[(size_t)head * T * T + (size_t)qi * T + key] = val;
    }
  }
}

// ------------------------------------------------------------------------------- launchers
// a.phase: 0 the whole forward in one launch; 1 and 2 its two halves (phase 1 is the same for every
// reconstruction and is built once per calibration)
template <int D, int CAL, int MODE, typename TIn, int PHASE>
static hipError_t fwd_launch(const Problem& p, const FwdArgs& a, hipStream_t s) {
  const int nqt = (p.T + BN - 1) / BN;
  const size_t smem = fwd_smem_bytes<D, CAL, MODE, TIn>(p.K, p.lres);
  if constexpr (MODE == BINM) {
    if (p.K < BINM_SMALLB) {
      hipLaunchKernelGGL((fwd_kernel<D, CAL, MODE, TIn, BINM_SMALLB, PHASE>), dim3(p.nheads * nqt), dim3(FWD_NT), smem,
                         s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fwd_kernel<D, CAL, MODE, TIn, BINM_MAXB, PHASE>), dim3(p.nheads * nqt), dim3(FWD_NT), smem, s, a);
  return hipGetLastError();
}
template <int D, int CAL, int MODE, typename TIn>
static hipError_t fwd_go(const Problem& p, const FwdArgs& a, hipStream_t s) {
  constexpr int MODE1 = CAL == EXPB ? EXP32 : LERP;
  if (a.phase == 1) return fwd_launch<D, CAL, MODE1, TIn, 1>(p, a, s);
  if (a.phase == 2) return fwd_launch<D, CAL, MODE, TIn, 2>(p, a, s);
  return fwd_launch<D, CAL, MODE, TIn, 0>(p, a, s);
}
template <int D, int CAL, int MODE>
static hipError_t fwd_dt(const Problem& p, const FwdArgs& a, hipStream_t s) {
  return p.bf16 ? fwd_go<D, CAL, MODE, uint16_t>(p, a, s) : fwd_go<D, CAL, MODE, float>(p, a, s);
}
template <int D, int CAL>
static hipError_t fwd_md(const Problem& p, const FwdArgs& a, hipStream_t s) {
  if constexpr (CAL == EXPB) {
    if (p.mode == EXPF8) return fwd_dt<D, CAL, EXPF8>(p, a, s);
    return p.mode == EXPBF ? fwd_dt<D, CAL, EXPBF>(p, a, s) : fwd_dt<D, CAL, EXP32>(p, a, s);
  } else {
    switch (p.mode) {
      case LERP: return fwd_dt<D, CAL, LERP>(p, a, s);
      case NEAREST_W: return fwd_dt<D, CAL, NEAREST_W>(p, a, s);
      case NEAREST_P: return fwd_dt<D, CAL, NEAREST_P>(p, a, s);
      case BINM:
        if constexpr (CAL == MINMAX || CAL == FWM) return fwd_dt<D, CAL, BINM>(p, a, s);
        else return hipErrorInvalidValue;
      default: return fwd_dt<D, CAL, NEAREST_W>(p, a, s);  // NEARB: the strict Nearest forward
    }
  }
}
template <>
hipError_t forward_cal<KIA_CAL>(const Problem& p, const FwdArgs& a, hipStream_t s) {
  return p.D == 128 ? fwd_md<128, KIA_CAL>(p, a, s) : fwd_md<64, KIA_CAL>(p, a, s);
}

template <int CAL, int MODE>
static hipError_t bins_go(const Problem& p, const BinsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bins_kernel<CAL, MODE>), dim3(p.nheads * a.rec.nt), dim3(256), 0, s, a);
  return hipGetLastError();
}
template <>
hipError_t bins_cal<KIA_CAL>(const Problem& p, const BinsArgs& a, hipStream_t s) {
  if constexpr (KIA_CAL == EXPB) {
    if (p.mode == EXPF8) return bins_go<KIA_CAL, EXPF8>(p, a, s);
    return p.mode == EXPBF ? bins_go<KIA_CAL, EXPBF>(p, a, s) : bins_go<KIA_CAL, EXP32>(p, a, s);
  } else {
    return p.mode == LERP ? bins_go<KIA_CAL, LERP>(p, a, s) : bins_go<KIA_CAL, NEAREST_W>(p, a, s);
  }
}

}  // namespace kia
