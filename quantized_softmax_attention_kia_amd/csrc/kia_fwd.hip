// Forward kernel of K-interval attention for gfx950 (CDNA4).
//
// "Pretraining Transformers with Quantized Softmax in Attention", §3: the grid
// of a row depends on the row's final extrema, so the online-softmax rescale
// does not apply.  One workgroup owns 128 query rows of one head (4 waves x 32
// rows) and sweeps the visible key tiles twice:
//   pass 1  S^T = K Q^T on the fp32 MFMA -> row max / min, first arg, tie counts;
//   then    per-row calibration and the (K+1)-entry grid table e^{b_r} in LDS
//           (the only exponentials of the pass);
//   pass 2  recompute S^T (same instructions, bit-identical scores) -> bin
//           decision -> LERP / Nearest weight from the table (no exp) -> row
//           sums W^L, W^N -> O += w V on the MFMA (and O^L += w^L V for Nearest
//           with Prob-STE) -> O = num / W (strict hard forward for Nearest).
// K and V tiles are staged through LDS and shared by the four waves.
#include "kia_device.hpp"
#include "kia_launch.hpp"

#include <climits>

namespace kia {

constexpr int FWD_BM = 128;  // query rows per workgroup
constexpr int BN = 32;       // keys per tile

// Stage 32 rows of a [T, D] head tensor (rows row0..row0+31, zero past T) into LDS.
template <int D, typename T>
__device__ __forceinline__ void stage_rows(float* dst, int ld, const T* src, int row0, int nrows, float mul) {
  constexpr int CH = BN * D / 4;
#pragma unroll
  for (int id = threadIdx.x; id < CH; id += 256) {
    const int r = id / (D / 4), c4 = (id % (D / 4)) * 4;
    const int gr = row0 + r;
    f4v x = f4v{0.f, 0.f, 0.f, 0.f};
    if (gr < nrows) x = Ld<T>::four(src + (size_t)gr * D + c4);
    if (mul != 1.0f) x *= mul;
    *reinterpret_cast<f4v*>(dst + r * ld + c4) = x;
  }
}

template <int D>
struct FwdSmem {
  float Ks[BN * (D + 4)];
  float Vs[BN * (D + 8)];
  float tbl[FWD_BM * (KMAX + 1)];
  float rowW[FWD_BM];
  float rowWL[FWD_BM];
};

template <int D, int CAL, int MODE, typename TIn>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs a) {
  __shared__ FwdSmem<D> sm;
  constexpr int LDK = D + 4, LDV = D + 8;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, c = l & 31;
  const int T = a.T, K = a.K, ts = K + 1;
  const int nqt = (T + FWD_BM - 1) / FWD_BM;
  const int L = logical_block();
  const int head = L / nqt;
  const int qt = nqt - 1 - (L % nqt);  // heaviest (latest) query tiles of a head first
  const size_t hb = (size_t)head * T * D;
  const TIn* Qp = reinterpret_cast<const TIn*>(a.q) + hb;
  const TIn* Kp = reinterpret_cast<const TIn*>(a.k) + hb;
  const TIn* Vp = reinterpret_cast<const TIn*>(a.v) + hb;
  const int qb0 = qt * FWD_BM, qw0 = qb0 + 32 * w, qi = qw0 + c;
  const bool qvalid = qi < T;
  const int qlast_w = min(qw0 + 31, T - 1);
  const int kend = a.causal ? min(T, qb0 + FWD_BM) : T;
  const int ntiles = (kend + BN - 1) / BN;
  const int rl = 32 * w + c;

  float qreg[D / 2];
  load_row_operand<D>(qreg, Qp + (size_t)qi * D, qvalid, a.scale);

  // ---- pass 1: row extrema, first index attaining them, tie counts
  float mx = -INFINITY, mn = INFINITY;
  int ax = INT_MAX, an = INT_MAX, cx = 0, cn = 0;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    stage_rows<D>(sm.Ks, LDK, Kp, k0, T, 1.0f);
    __syncthreads();
    if (qw0 >= T || (a.causal && k0 > qlast_w)) continue;
    const f16v s = tile_dot<D>(sm.Ks, LDK, qreg);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = k0 + crow(v, g);
      const bool ok = qvalid && key < T && (!a.causal || key <= qi);
      const float x = s[v];
      if (ok) {
        if (x > mx) { mx = x; ax = key; cx = 1; } else if (x == mx) { ++cx; }
        if (x < mn) { mn = x; an = key; cn = 1; } else if (x == mn) { ++cn; }
      }
    }
  }
  // merge the two half-waves that share a query row
  float M, m;
  int amax, amin, nA, nC;
  {
    const float mx2 = __shfl_xor(mx, 32), mn2 = __shfl_xor(mn, 32);
    const int ax2 = __shfl_xor(ax, 32), an2 = __shfl_xor(an, 32);
    const int cx2 = __shfl_xor(cx, 32), cn2 = __shfl_xor(cn, 32);
    M = fmaxf(mx, mx2);
    m = fminf(mn, mn2);
    amax = min(mx == M ? ax : INT_MAX, mx2 == M ? ax2 : INT_MAX);
    amin = min(mn == m ? an : INT_MAX, mn2 == m ? an2 : INT_MAX);
    nA = (mx == M ? cx : 0) + (mx2 == M ? cx2 : 0);
    nC = (mn == m ? cn : 0) + (mn2 == m ? cn2 : 0);
  }

  // ---- calibration and grid table (K+1 exponentials per row)
  const RowCal rc = row_calibration<CAL>(M, m, K, a.tau);
  float* trow = sm.tbl + rl * ts;
  for (int r = g; r <= K; r += 2) trow[r] = grid_value<CAL>(M, m, K, a.tau, r);

  // ---- pass 2: reconstruct, normalize, multiply by V
  float sumL = 0.f, sumN = 0.f;
  f16v o[D / 32], ol[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) { o[nb] = zero16(); ol[nb] = zero16(); }
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    stage_rows<D>(sm.Ks, LDK, Kp, k0, T, 1.0f);
    stage_rows<D>(sm.Vs, LDV, Vp, k0, T, 1.0f);
    __syncthreads();
    if (qw0 >= T || (a.causal && k0 > qlast_w)) continue;
    const f16v s = tile_dot<D>(sm.Ks, LDK, qreg);
    f16v p, pl;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = k0 + crow(v, g);
      const bool ok = qvalid && key < T && (!a.causal || key <= qi);
      const Decision d = decide<CAL>(s[v], rc, K, a.tau);
      const Weights wt = weights(d, trow);
      const bool keep = ok && !d.tail;
      const float wl = keep ? wt.wL : 0.f;
      const float wn = keep ? wt.wN : 0.f;
      sumL += wl;
      sumN += wn;
      p[v] = (MODE == LERP) ? wl : wn;
      pl[v] = wl;
    }
    tile_accum<D>(o, p, sm.Vs, LDV);
    if (MODE == NEAREST_P) tile_accum<D>(ol, pl, sm.Vs, LDV);
  }
  sumL += __shfl_xor(sumL, 32);
  sumN += __shfl_xor(sumN, 32);
  if (g == 0) {
    sm.rowW[rl] = (MODE == LERP) ? sumL : sumN;
    sm.rowWL[rl] = sumL;
    if (qvalid) {
      const size_t row = (size_t)head * T + qi;
      a.rec.M[row] = M;
      a.rec.m[row] = m;
      a.rec.amax[row] = amax;
      a.rec.amin[row] = amin;
      a.rec.nA[row] = nA;
      a.rec.nC[row] = nC;
      a.rec.WN[row] = sumN;
      a.rec.WL[row] = sumL;
    }
  }
  __syncthreads();
  // O = num / W; lane l holds rows crow(v, g) of the wave's 32 and columns 32 nb + c
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int qrow = qw0 + crow(v, g);
    if (qrow < T) {
      const float inv = 1.0f / sm.rowW[32 * w + crow(v, g)];
      float* orow = a.o + hb + (size_t)qrow * D + c;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) orow[32 * nb] = o[nb][v] * inv;
      if (MODE == NEAREST_P) {
        const float invl = 1.0f / sm.rowWL[32 * w + crow(v, g)];
        float* olrow = a.rec.OL + hb + (size_t)qrow * D + c;
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) olrow[32 * nb] = ol[nb][v] * invl;
      }
    }
  }
}

// Test hook: the bin decision of every (query, key) pair, from the forward's row record.
template <int D, int CAL, bool NEAREST, typename TIn>
__global__ __launch_bounds__(256) void bins_kernel(BinsArgs a) {
  __shared__ float Ks[BN * (D + 4)];
  constexpr int LDK = D + 4;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, c = l & 31;
  const int T = a.T, K = a.K;
  const int nqt = (T + FWD_BM - 1) / FWD_BM;
  const int L = logical_block();
  const int head = L / nqt, qt = L % nqt;
  const size_t hb = (size_t)head * T * D;
  const TIn* Qp = reinterpret_cast<const TIn*>(a.q) + hb;
  const TIn* Kp = reinterpret_cast<const TIn*>(a.k) + hb;
  const int qw0 = qt * FWD_BM + 32 * w, qi = qw0 + c;
  const bool qvalid = qi < T;
  float qreg[D / 2];
  load_row_operand<D>(qreg, Qp + (size_t)qi * D, qvalid, a.scale);
  const size_t row = (size_t)head * T + (qvalid ? qi : 0);
  const RowCal rc = row_calibration<CAL>(a.rec.M[row], a.rec.m[row], K, a.tau);
  const int ntiles = (T + BN - 1) / BN;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    stage_rows<D>(Ks, LDK, Kp, k0, T, 1.0f);
    __syncthreads();
    const f16v s = tile_dot<D>(Ks, LDK, qreg);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = k0 + crow(v, g);
      if (!qvalid || key >= T) continue;
      const bool ok = !a.causal || key <= qi;
      const Decision d = decide<CAL>(s[v], rc, K, a.tau);
      uint8_t val = 255;
      if (ok) val = d.tail ? 254 : (uint8_t)(NEAREST ? d.r + (d.t >= 0.5f ? 1 : 0) : d.r);
      a.bins[(size_t)head * T * T + (size_t)qi * T + key] = val;
    }
  }
}

// ------------------------------------------------------------------------------- launchers
template <int D, int CAL, int MODE, typename TIn>
static hipError_t fwd_go(const Problem& p, const FwdArgs& a, hipStream_t s) {
  const int nqt = (p.T + FWD_BM - 1) / FWD_BM;
  hipLaunchKernelGGL((fwd_kernel<D, CAL, MODE, TIn>), dim3(p.nheads * nqt), dim3(256), 0, s, a);
  return hipGetLastError();
}
template <int D, int CAL, int MODE>
static hipError_t fwd_dt(const Problem& p, const FwdArgs& a, hipStream_t s) {
  return p.bf16 ? fwd_go<D, CAL, MODE, uint16_t>(p, a, s) : fwd_go<D, CAL, MODE, float>(p, a, s);
}
template <int D, int CAL>
static hipError_t fwd_md(const Problem& p, const FwdArgs& a, hipStream_t s) {
  switch (p.mode) {
    case LERP: return fwd_dt<D, CAL, LERP>(p, a, s);
    case NEAREST_W: return fwd_dt<D, CAL, NEAREST_W>(p, a, s);
    default: return fwd_dt<D, CAL, NEAREST_P>(p, a, s);
  }
}
template <int D>
static hipError_t fwd_cl(const Problem& p, const FwdArgs& a, hipStream_t s) {
  return p.calib == FWM ? fwd_md<D, FWM>(p, a, s) : fwd_md<D, MINMAX>(p, a, s);
}
hipError_t launch_forward(const Problem& p, const FwdArgs& a, hipStream_t s) {
  return p.D == 128 ? fwd_cl<128>(p, a, s) : fwd_cl<64>(p, a, s);
}

template <int D, int CAL, bool NEAREST, typename TIn>
static hipError_t bins_go(const Problem& p, const BinsArgs& a, hipStream_t s) {
  const int nqt = (p.T + FWD_BM - 1) / FWD_BM;
  hipLaunchKernelGGL((bins_kernel<D, CAL, NEAREST, TIn>), dim3(p.nheads * nqt), dim3(256), 0, s, a);
  return hipGetLastError();
}
template <int D, int CAL, bool NEAREST>
static hipError_t bins_dt(const Problem& p, const BinsArgs& a, hipStream_t s) {
  return p.bf16 ? bins_go<D, CAL, NEAREST, uint16_t>(p, a, s) : bins_go<D, CAL, NEAREST, float>(p, a, s);
}
template <int D, int CAL>
static hipError_t bins_md(const Problem& p, const BinsArgs& a, hipStream_t s) {
  return p.mode == LERP ? bins_dt<D, CAL, false>(p, a, s) : bins_dt<D, CAL, true>(p, a, s);
}
template <int D>
static hipError_t bins_cl(const Problem& p, const BinsArgs& a, hipStream_t s) {
  return p.calib == FWM ? bins_md<D, FWM>(p, a, s) : bins_md<D, MINMAX>(p, a, s);
}
hipError_t launch_bins(const Problem& p, const BinsArgs& a, hipStream_t s) {
  return p.D == 128 ? bins_cl<128>(p, a, s) : bins_cl<64>(p, a, s);
}

}  // namespace kia
