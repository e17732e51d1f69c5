// Forward kernel of K-interval attention for gfx950 (CDNA4).
//
// "Pretraining Transformers with Quantized Softmax in Attention", §3: the grid
// of a row depends on the row's final extrema, so the online-softmax rescale
// does not apply.  One workgroup owns 64 query rows of one head (2 waves x 32
// rows; small workgroups, heaviest first, so the causal triangle balances over
// the CUs) and sweeps the visible key tiles twice, loading the next tile while
// it computes the current one:
//   pass 1  scores of each 32 x 32 tile on the fp64 MFMA (exact products of the
//           fp32 inputs, double accumulation, scale applied in double), rounded
//           once to fp32 and stored for every later pass; row max / min, first
//           index attaining them and tie counts on the stored values;
//   then    per-row calibration and the (K+1)-entry grid table e^{b_r} in LDS
//           (the only exponentials of the operator);
//   pass 2  stored scores -> bin decision -> LERP / Nearest weight from the
//           table (no exp) -> row sums W^L, W^N -> O += w V on the fp32 MFMA (and
//           O^L += w^L V for Nearest with Prob-STE) -> O = num / W (the strict
//           hard forward for Nearest).  Row sums are kept in double and each
//           tile's P V is summed into a fresh accumulator before joining the
//           running O, so the precision of O (which the backward's D_i = dO . O
//           amplifies) does not decay with T.
// K (pass 1) and V (pass 2) tiles are staged through LDS and shared by the waves.
#include "kia_device.hpp"
#include "kia_launch.hpp"

#include <climits>

namespace kia {

constexpr int NW = 2;              // waves per workgroup
constexpr int NT = 64 * NW;        // threads per workgroup
constexpr int FWD_BM = 32 * NW;    // query rows per workgroup
constexpr int BN = 32;             // keys per tile
constexpr int SCR = 80;            // row stride of the per-wave tile scratch (bank-conflict free writes)

template <int D>
struct FwdSmem {
  union {
    float Ks[BN * (D + 4)];  // pass 1
    float Vs[BN * (D + 8)];  // pass 2
  };
  float scratch[NW][16 * SCR];  // per-wave tile re-layout (pass 1)
  float rowM[FWD_BM], rowm[FWD_BM], rowW[FWD_BM], rowWL[FWD_BM];
  int rowax[FWD_BM], rowan[FWD_BM], rowcx[FWD_BM], rowcn[FWD_BM];
  // followed in dynamic LDS by the grid table: FWD_BM rows x (K + 1) floats
};

struct Ext {  // running max / min with first index and count
  float mx, mn;
  int ax, an, cx, cn;
};

__device__ __forceinline__ void ext_merge(Ext& a, int lanemask) {
  const float mx2 = __shfl_xor(a.mx, lanemask), mn2 = __shfl_xor(a.mn, lanemask);
  const int ax2 = __shfl_xor(a.ax, lanemask), an2 = __shfl_xor(a.an, lanemask);
  const int cx2 = __shfl_xor(a.cx, lanemask), cn2 = __shfl_xor(a.cn, lanemask);
  const float M = fmaxf(a.mx, mx2), m = fminf(a.mn, mn2);
  a.ax = min(a.mx == M ? a.ax : INT_MAX, mx2 == M ? ax2 : INT_MAX);
  a.an = min(a.mn == m ? a.an : INT_MAX, mn2 == m ? an2 : INT_MAX);
  a.cx = (a.mx == M ? a.cx : 0) + (mx2 == M ? cx2 : 0);
  a.cn = (a.mn == m ? a.cn : 0) + (mn2 == m ? cn2 : 0);
  a.mx = M;
  a.mn = m;
}

// At D = 64 the register budget is held to two waves per SIMD.
template <int D, int CAL, int MODE, typename TIn>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void fwd_kernel(FwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  FwdSmem<D>& sm = *reinterpret_cast<FwdSmem<D>*>(smem_raw);
  constexpr int LDK = D + 4, LDV = D + 8;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, c = l & 31;
  const int G = l >> 4, c16 = l & 15;
  const int T = a.T, K = a.K, ts = K + 1;
  const int nqt = (T + FWD_BM - 1) / FWD_BM;
  int head, rank;
  block_work(a.nheads, head, rank);
  const int qt = a.causal ? nqt - 1 - rank : rank;  // rank 0: the latest query tile, the most keys
  const size_t hb = (size_t)head * T * D;
  const TIn* Qp = reinterpret_cast<const TIn*>(a.q) + hb;
  const TIn* Kp = reinterpret_cast<const TIn*>(a.k) + hb;
  const TIn* Vp = reinterpret_cast<const TIn*>(a.v) + hb;
  const int qb0 = qt * FWD_BM, qw0 = qb0 + 32 * w, qi = qw0 + c;
  const int qtw = qw0 / BN;  // the wave's query tile
  const bool qvalid = qi < T;
  const int qlast_w = min(qw0 + 31, T - 1);
  const int kend = a.causal ? min(T, qb0 + FWD_BM) : T;
  const int ntiles = (kend + BN - 1) / BN;
  const int rl = 32 * w + c;
  float* Sh = a.rec.S + (size_t)head * a.rec.tiles_per_head * 1024;

  // ---- pass 1: scores (fp64 MFMA) stored once; row extrema with first index and tie counts
  float qr[D / 2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qw0 + 16 * qb + c16;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      f4v x = f4v{0.f, 0.f, 0.f, 0.f};
      if (row < T) x = Ld<TIn>::four(Qp + (size_t)row * D + 16 * j + 4 * G);
#pragma unroll
      for (int e = 0; e < 4; ++e) qr[qb * (D / 4) + 4 * j + e] = x[e];
    }
  }
  Ext ex[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) ex[qb] = Ext{-INFINITY, INFINITY, INT_MAX, INT_MAX, 0, 0};
  float* scr = sm.scratch[w];
  TileRegs<D, NT, TIn> kr;
  kr.load(Kp, 0, T);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    kr.store(sm.Ks, LDK, 1.0f);
    __syncthreads();
    if (kt + 1 < ntiles) kr.load(Kp, k0 + BN, T);  // next tile in flight during this one
    if (qw0 >= T || (a.causal && k0 > qlast_w)) continue;
    d4v acc[2][2];
    score_tile_f64<D>(sm.Ks, LDK, qr, acc);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float x = (float)(a.scale * acc[kb][qb][v]);
          const int klo = 16 * kb + 4 * v + G, qlo = 16 * qb + c16;
          const int key = k0 + klo, query = qw0 + qlo;
          const bool ok = query < T && key < T && (!a.causal || key <= query);
          Ext& e = ex[qb];
          if (ok) {
            if (x > e.mx) { e.mx = x; e.ax = key; e.cx = 1; } else if (x == e.mx) { ++e.cx; }
            if (x < e.mn) { e.mn = x; e.an = key; e.cn = 1; } else if (x == e.mn) { ++e.cn; }
          }
          // re-layout into the stored tile order: (query qlo, key klo) -> v' * 64 + qlo + 32 g'
          const int gp = (klo >> 2) & 1, vp = 4 * (klo >> 3) + (klo & 3);
          scr[vp * SCR + qlo + 32 * gp] = x;
        }
    float* St = Sh + tile_index(qtw, kt, a.rec.nt, a.causal) * 1024;
#pragma unroll
    for (int v = 0; v < 16; ++v) St[v * 64 + l] = scr[v * SCR + l];
  }
  // merge the four lanes that share a query row (lanes c16 + 16 G)
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    ext_merge(ex[qb], 16);
    ext_merge(ex[qb], 32);
    if (G == 0) {
      const int r2 = 32 * w + 16 * qb + c16;
      sm.rowM[r2] = ex[qb].mx;
      sm.rowm[r2] = ex[qb].mn;
      sm.rowax[r2] = ex[qb].ax;
      sm.rowan[r2] = ex[qb].an;
      sm.rowcx[r2] = ex[qb].cx;
      sm.rowcn[r2] = ex[qb].cn;
    }
  }
  // pass 2 reads back the tiles stored above: complete the stores and drop stale L1 lines
  __threadfence();
  __syncthreads();
  // from here on lane l works on query row l%32 of the wave
  const float M = sm.rowM[rl], m = sm.rowm[rl];

  // ---- calibration and grid table (K+1 exponentials per row)
  const RowCal rc = row_calibration<CAL>(M, m, K, a.tau);
  float* tbl = reinterpret_cast<float*>(smem_raw + sizeof(FwdSmem<D>));
  float* trow = tbl + rl * ts;
  for (int r = g; r <= K; r += 2) trow[r] = grid_value<CAL>(M, m, K, a.tau, r);

  // ---- pass 2: reconstruct, normalize, multiply by V
  double sumL = 0.0, sumN = 0.0;  // row sums of positive weights: double, no absorption of small terms
  f16v o[D / 32], ol[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) { o[nb] = zero16(); ol[nb] = zero16(); }
  TileRegs<D, NT, TIn> vr;
  vr.load(Vp, 0, T);
  f16v snext;
  const bool act0 = qw0 < T;
  if (act0) {
    const float* St = Sh + tile_index(qtw, 0, a.rec.nt, a.causal) * 1024;
#pragma unroll
    for (int v = 0; v < 16; ++v) snext[v] = St[v * 64 + l];
  }
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    vr.store(sm.Vs, LDV, 1.0f);
    __syncthreads();
    const f16v s = snext;
    if (kt + 1 < ntiles) {  // next V tile and next score tile in flight during this one
      vr.load(Vp, k0 + BN, T);
      if (qw0 < T && (!a.causal || k0 + BN <= qlast_w)) {
        const float* St = Sh + tile_index(qtw, kt + 1, a.rec.nt, a.causal) * 1024;
#pragma unroll
        for (int v = 0; v < 16; ++v) snext[v] = St[v * 64 + l];
      }
    }
    if (qw0 >= T || (a.causal && k0 > qlast_w)) continue;
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
      sumL += (double)wl;
      sumN += (double)wn;
      p[v] = (MODE == LERP) ? wl : wn;
      pl[v] = wl;
    }
    // each tile's P V goes into a fresh accumulator, then into the running sum: the long
    // accumulation chain then holds one add per tile instead of one per MFMA step
    f16v ot[D / 32];
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) ot[nb] = zero16();
    tile_accum<D>(ot, p, sm.Vs, LDV);
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) o[nb] += ot[nb];
    if (MODE == NEAREST_P) {
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) ot[nb] = zero16();
      tile_accum<D>(ot, pl, sm.Vs, LDV);
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) ol[nb] += ot[nb];
    }
  }
  sumL += __shfl_xor(sumL, 32);
  sumN += __shfl_xor(sumN, 32);
  const float WLf = (float)sumL, WNf = (float)sumN;
  if (g == 0) {
    sm.rowW[rl] = (MODE == LERP) ? WLf : WNf;
    sm.rowWL[rl] = WLf;
    if (qvalid) {
      const size_t row = (size_t)head * T + qi;
      a.rec.M[row] = M;
      a.rec.m[row] = m;
      a.rec.amax[row] = sm.rowax[rl];
      a.rec.amin[row] = sm.rowan[rl];
      a.rec.nA[row] = sm.rowcx[rl];
      a.rec.nC[row] = sm.rowcn[rl];
      a.rec.WN[row] = WNf;
      a.rec.WL[row] = WLf;
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

template <int D>
size_t fwd_smem_bytes(int K) {
  return sizeof(FwdSmem<D>) + sizeof(float) * (FWD_BM * (K + 1));
}

// Test hook: the bin decision of every (query, key) pair, from the stored scores and row record.
template <int CAL, bool NEAREST>
__global__ __launch_bounds__(256) void bins_kernel(BinsArgs a) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, c = l & 31;
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
        const Decision d = decide<CAL>(St[v * 64 + l], rc, K, a.tau);
        val = d.tail ? 254 : (uint8_t)(NEAREST ? d.r + (d.t >= 0.5f ? 1 : 0) : d.r);
      }
      a.bins[(size_t)head * T * T + (size_t)qi * T + key] = val;
    }
  }
}

// ------------------------------------------------------------------------------- launchers
template <int D, int CAL, int MODE, typename TIn>
static hipError_t fwd_go(const Problem& p, const FwdArgs& a, hipStream_t s) {
  const int nqt = (p.T + FWD_BM - 1) / FWD_BM;
  const size_t smem = fwd_smem_bytes<D>(p.K);
  hipLaunchKernelGGL((fwd_kernel<D, CAL, MODE, TIn>), dim3(p.nheads * nqt), dim3(NT), smem, s, a);
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

template <int CAL, bool NEAREST>
static hipError_t bins_go(const Problem& p, const BinsArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bins_kernel<CAL, NEAREST>), dim3(p.nheads * a.rec.nt), dim3(256), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_bins(const Problem& p, const BinsArgs& a, hipStream_t s) {
  if (p.calib == FWM) return p.mode == LERP ? bins_go<FWM, false>(p, a, s) : bins_go<FWM, true>(p, a, s);
  return p.mode == LERP ? bins_go<MINMAX, false>(p, a, s) : bins_go<MINMAX, true>(p, a, s);
}

}  // namespace kia
