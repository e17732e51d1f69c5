// Backward kernels of K-interval attention for gfx950 (CDNA4).
//
// "Pretraining Transformers with Quantized Softmax in Attention", App. B:
//   gamma_j = (g_j - sum_i P_i g_i) / W at the surrogate's normalization point
//             ((P^N, W^N) for Weight-STE, (P^L, W^L) for Prob-STE and LERP),
//   Delta_j = (e^{b_{r+1}} - e^{b_r}) / h           (LERP secant slope),
//   dS_j    = gamma_j Delta_j  (+ the extremum terms in full mode),
// and the extremum terms of the full calibration gradient:
//   MinMax  a = sum_j gamma_j dw_j/dM, b = sum_j gamma_j dw_j/dm, with
//           dw/dM = X - w - rho Delta and dw/dm = w - X - (1 - rho) Delta
//           (rho = (r+t)/K, X = (r w + t e^{b_{r+1}})/K; the degenerate branch has
//           a constant h, which drops the rho Delta part), so a + b = -sum dS_self;
//   FWM     a = -sum_{window} gamma_j Delta_j;
// a is added to the score gradient of the arg-max key(s) and b to the arg-min
// key(s), split evenly among ties.
//
// Both kernels read the scores the forward stored (no score recomputation):
//   dq kernel   (query-major, 64 rows per workgroup): D_i, dQ_self = sum dS_self K
//               on the MFMA, the row sums a_i, b_i; then the extremum terms of dQ
//               (gathered rows of K at the arg-max / arg-min; a second sweep adds
//               extra tied keys when a row has any); writes dQ and, per row, the
//               record the key-major pass needs (calibration, 1/W, D_i,
//               alpha = a/nA, beta = b/nC) and the grid table.
//   dkdv kernel (key-major, 64 keys per workgroup): dV += P^T dO, dK += dS^T Q,
//               where dS carries alpha / beta on the arg-max / arg-min keys, so the
//               scatter of the calibration gradient into dK needs no atomics.  Each
//               wave transposes its stored score tile through LDS.
// Both sweep their tiles while the next tile's operands are already being loaded.
#include "kia_device.hpp"
#include "kia_launch.hpp"

namespace kia {

constexpr int NW = 2;         // waves per workgroup
constexpr int NT = 64 * NW;   // threads per workgroup
constexpr int BN = 32;        // keys per tile (dq kernel) / queries per tile (dkdv kernel)
constexpr int DQ_BM = 32 * NW;  // query rows per dq workgroup
constexpr int KV_BN = 32 * NW;  // key rows per dkdv workgroup
constexpr int TLD = 33;       // row stride of the LDS tile transpose
constexpr int TBL_CH = (BN * (KMAX + 1) + NT - 1) / NT;  // grid-table floats per thread per tile

// Per query row, written by the dq kernel for the key-major pass (64 bytes).
struct RowP {
  double origin, inv_h;
  float inv_hf, invWf, invWg, Di;
  float alpha, beta, M, m;
  int amax, amin, pad0, pad1;
};

template <typename T> __device__ __forceinline__ float ld1(const T* p);
template <> __device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p) {
  return __uint_as_float(((uint32_t)*p) << 16);
}

// ============================================================================ dq kernel
template <int D>
struct DqSmem {
  float Ks[BN * (D + 4)];
  float Vs[BN * (D + 4)];
  float alpha[DQ_BM], beta[DQ_BM];
  int amax[DQ_BM], amin[DQ_BM];
  // followed in dynamic LDS by the grid table: DQ_BM rows x (K + 1) floats
};

template <int D, int CAL, int MODE, bool FULL, typename TIn>
__global__ __launch_bounds__(NT) void dq_kernel(BwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  DqSmem<D>& sm = *reinterpret_cast<DqSmem<D>*>(smem_raw);
  float* tbl = reinterpret_cast<float*>(smem_raw + sizeof(DqSmem<D>));
  constexpr int LD = D + 4;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, c = l & 31;
  const int T = a.T, K = a.K, ts = K + 1;
  const int nqt = (T + DQ_BM - 1) / DQ_BM;
  int head, rank;
  block_work(a.nheads, head, rank);
  const int qt = a.causal ? nqt - 1 - rank : rank;
  const size_t hb = (size_t)head * T * D;
  const TIn* Kp = reinterpret_cast<const TIn*>(a.k) + hb;
  const TIn* Vp = reinterpret_cast<const TIn*>(a.v) + hb;
  const TIn* dOp = reinterpret_cast<const TIn*>(a.dO) + hb;
  const int qb0 = qt * DQ_BM, qw0 = qb0 + 32 * w, qi = qw0 + c;
  const int qtw = qw0 / BN;
  const bool qvalid = qi < T;
  const int qlast_w = min(qw0 + 31, T - 1);
  const int kend = a.causal ? min(T, qb0 + DQ_BM) : T;
  const int ntiles = (kend + BN - 1) / BN;
  const int rl = 32 * w + c;
  const size_t row = (size_t)head * T + (qvalid ? qi : 0);
  const float* Sh = a.rec.S + (size_t)head * a.rec.tiles_per_head * 1024;
  auto active = [&](int kt) { return qw0 < T && (!a.causal || kt * BN <= qlast_w); };

  float doreg[D / 2];
  load_row_operand<D>(doreg, dOp + (size_t)qi * D, qvalid, 1.0f);

  // row record of the forward
  const float M = a.rec.M[row], m = a.rec.m[row];
  const int amax = a.rec.amax[row], amin = a.rec.amin[row];
  const int nA = a.rec.nA[row], nC = a.rec.nC[row];
  const float Wf = (MODE == LERP) ? a.rec.WL[row] : a.rec.WN[row];
  const float Wg = (MODE == NEAREST_W) ? a.rec.WN[row] : a.rec.WL[row];
  const float invWg = 1.0f / Wg;

  // D_i = dO_i . O_i (O^L_i for Nearest with Prob-STE): sum_j P_j g_j at the normalization point
  float Di;
  {
    const float* X = ((MODE == NEAREST_P) ? a.rec.OL : a.o) + hb + (size_t)qi * D + 4 * g;
    double part = 0.0;
    if (qvalid) {
#pragma unroll
      for (int q = 0; q < D / 8; ++q) {
        const f4v x = *reinterpret_cast<const f4v*>(X + 8 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) part = fma((double)doreg[4 * q + e], (double)x[e], part);
      }
    }
    Di = (float)(part + __shfl_xor(part, 32));
  }

  const RowCal rc = row_calibration<CAL>(M, m, K, a.tau);
  float* trow = tbl + rl * ts;
  float* gtab = a.tab + row * ts;
  if (qvalid)
    for (int r = g; r <= K; r += 2) {
      const float e = grid_value<CAL>(M, m, K, a.tau, r);
      trow[r] = e;
      gtab[r] = e;   // the key-major pass reads the table instead of recomputing it
    }
  // extra tied extrema (beyond the first index) need a second sweep to find them
  const bool rowties = FULL && qvalid && (M != m) && (nA > 1 || (CAL == MINMAX && nC > 1));
  const bool blockties = __syncthreads_or(rowties);

  double acc_a = 0.0, sds = 0.0;  // calibration sums: terms of both signs, summed in double
  f16v dq[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) dq[nb] = zero16();

  TileRegs<D, NT, TIn> kr, vr;
  kr.load(Kp, 0, T);
  vr.load(Vp, 0, T);
  f16v snext;
  if (active(0)) {
    const float* St = Sh + tile_index(qtw, 0, a.rec.nt, a.causal) * 1024;
#pragma unroll
    for (int v = 0; v < 16; ++v) snext[v] = St[v * 64 + l];
  }
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    kr.store(sm.Ks, LD, 1.0f);
    vr.store(sm.Vs, LD, 1.0f);
    __syncthreads();
    const f16v s = snext;  // S^T: row = key, column = query
    if (kt + 1 < ntiles) {
      kr.load(Kp, k0 + BN, T);
      vr.load(Vp, k0 + BN, T);
      if (active(kt + 1)) {
        const float* St = Sh + tile_index(qtw, kt + 1, a.rec.nt, a.causal) * 1024;
#pragma unroll
        for (int v = 0; v < 16; ++v) snext[v] = St[v * 64 + l];
      }
    }
    if (!active(kt)) continue;
    const f16v gt = tile_dot<D>(sm.Vs, LD, doreg);  // (dO V^T)^T: g_ij = dO_i . V_j
    f16v ds;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = k0 + crow(v, g);
      const bool ok = qvalid && key < T && (!a.causal || key <= qi);
      const Decision d = decide<CAL>(s[v], rc, K, a.tau);
      const Weights wt = weights(d, trow);
      const bool keep = ok && !d.tail;
      const float Delta = keep ? (wt.E1 - wt.E0) * rc.inv_hf : 0.f;
      const float gam = keep ? (gt[v] - Di) * invWg : 0.f;
      const float dS = gam * Delta;
      ds[v] = dS;
      if (FULL) {
        sds += (double)dS;
        if (CAL == MINMAX) {
          const float rf = (float)d.r;
          // K * dw/dM = (r - K) w + t e^{b_{r+1}} - kappa (r + t) Delta
          const float dMk = fmaf(rf - (float)K, wt.wL, d.t * wt.E1) - rc.kappa * (rf + d.t) * Delta;
          acc_a = fma((double)gam, (double)dMk, acc_a);
        }
      }
    }
    tile_accum<D>(dq, ds, sm.Ks, LD);
  }

  // extremum terms of the row: alpha per tied max key, beta per tied min key
  float alpha = 0.f, beta = 0.f;
  if (FULL) {
    acc_a += __shfl_xor(acc_a, 32);
    sds += __shfl_xor(sds, 32);
    if (qvalid && M != m) {  // M == m: every grid value is 1 and both terms vanish exactly
      if (CAL == MINMAX) {
        const double A = acc_a / (double)K;
        const double Bm = -sds - A;
        alpha = (float)(A / (double)nA);
        beta = (float)(Bm / (double)nC);
      } else {
        alpha = (float)(-sds / (double)nA);
      }
    }
  }
  if (FULL && blockties) {
    // second sweep: tied keys other than the first arg-max / arg-min
    for (int kt = 0; kt < ntiles; ++kt) {
      const int k0 = kt * BN;
      __syncthreads();
      kr.load(Kp, k0, T);
      kr.store(sm.Ks, LD, 1.0f);
      __syncthreads();
      if (!active(kt)) continue;
      const float* St = Sh + tile_index(qtw, kt, a.rec.nt, a.causal) * 1024;
      f16v inj;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float sv = St[v * 64 + l];
        const int key = k0 + crow(v, g);
        const bool ok = rowties && key < T && (!a.causal || key <= qi);
        float x = 0.f;
        if (ok && sv == M && key != amax) x += alpha;
        if (CAL == MINMAX && ok && sv == m && key != amin) x += beta;
        inj[v] = x;
      }
      tile_accum<D>(dq, inj, sm.Ks, LD);
    }
  }
  if (g == 0) {
    sm.alpha[rl] = alpha;
    sm.beta[rl] = beta;
    sm.amax[rl] = qvalid ? amax : 0;
    sm.amin[rl] = qvalid ? amin : 0;
    if (qvalid) {
      RowP rp;
      rp.origin = rc.origin;
      rp.inv_h = rc.inv_h;
      rp.inv_hf = rc.inv_hf;
      rp.invWf = 1.0f / Wf;
      rp.invWg = invWg;
      rp.Di = Di;
      rp.alpha = FULL ? alpha : 0.f;
      rp.beta = FULL ? beta : 0.f;
      rp.M = M;
      rp.m = m;
      rp.amax = amax;
      rp.amin = amin;
      rp.pad0 = rp.pad1 = 0;
      a.rowp[row] = rp;
    }
  }
  __syncthreads();
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int qrow = qw0 + crow(v, g);
    if (qrow < T) {
      const int r2 = 32 * w + crow(v, g);
      const float al = sm.alpha[r2], be = sm.beta[r2];
      const TIn* ka = Kp + (size_t)sm.amax[r2] * D + c;
      const TIn* kb = Kp + (size_t)sm.amin[r2] * D + c;
      float* out = a.dq + hb + (size_t)qrow * D + c;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) {
        float val = dq[nb][v];
        if (FULL) {
          val = fmaf(al, ld1<TIn>(ka + 32 * nb), val);
          if (CAL == MINMAX) val = fmaf(be, ld1<TIn>(kb + 32 * nb), val);
        }
        out[32 * nb] = val * a.scale;
      }
    }
  }
}

// ============================================================================ dkdv kernel
template <int D>
struct KvSmem {
  float Qs[BN * (D + 4)];
  float dOs[BN * (D + 4)];
  float St[NW][BN * TLD];  // per-wave transpose of the stored score tile
  RowP rp[BN];
  float tbl[BN * (KMAX + 1)];
};

// Operands of one query tile for the key-major pass, held in registers while the previous
// tile computes: Q and dO rows, the wave's stored score tile, the row records and grid tables.
template <int D, typename TIn>
struct KvPrefetch {
  TileRegs<D, NT, TIn> q, dO;
  float s[16];
  f4v rp;
  float tb[TBL_CH];
};

template <int D, typename TIn>
__device__ __forceinline__ void kv_load(KvPrefetch<D, TIn>& pf, const BwdArgs& a, const TIn* Qp, const TIn* dOp,
                                        const float* Sh, int head, int qt, int ktw, bool act) {
  const int T = a.T, ts = a.K + 1, q0 = qt * BN, tid = threadIdx.x, l = tid & 63;
  pf.q.load(Qp, q0, T);
  pf.dO.load(dOp, q0, T);
  if (act) {
    const float* Sg = Sh + tile_index(qt, ktw, a.rec.nt, a.causal) * 1024;
#pragma unroll
    for (int v = 0; v < 16; ++v) pf.s[v] = Sg[v * 64 + l];
  }
  {  // 32 rows x 64 bytes: one float4 per thread
    const int rr = tid >> 2, part = tid & 3;
    pf.rp = f4v{0.f, 0.f, 0.f, 0.f};
    if (q0 + rr < T)
      pf.rp = reinterpret_cast<const f4v*>(a.rowp + (size_t)head * T + q0 + rr)[part];
  }
  const int nvalid = max(0, min(BN, T - q0)) * ts;
  const float* gt = a.tab + ((size_t)head * T + q0) * ts;
#pragma unroll
  for (int i = 0; i < TBL_CH; ++i) {
    const int idx = tid + i * NT;
    pf.tb[i] = idx < nvalid ? gt[idx] : 0.f;
  }
}

template <int D, int CAL, int MODE, bool FULL, typename TIn>
__global__ __launch_bounds__(NT) void dkdv_kernel(BwdArgs a) {
  __shared__ KvSmem<D> sm;
  constexpr int LD = D + 4;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, c = l & 31;
  const int T = a.T, K = a.K, ts = K + 1, nt = a.rec.nt;
  const int nkt = (T + KV_BN - 1) / KV_BN;
  int head, kt;
  block_work(a.nheads, head, kt);  // low key tiles see the most queries: heaviest first
  const size_t hb = (size_t)head * T * D;
  const TIn* Qp = reinterpret_cast<const TIn*>(a.q) + hb;
  const TIn* Vp = reinterpret_cast<const TIn*>(a.v) + hb;
  const TIn* dOp = reinterpret_cast<const TIn*>(a.dO) + hb;
  const int kb0 = kt * KV_BN, kw0 = kb0 + 32 * w, kj = kw0 + c;
  const int ktw = kw0 / BN;  // the wave's key tile
  const bool kvalid = kj < T;
  const float* Sh = a.rec.S + (size_t)head * a.rec.tiles_per_head * 1024;
  float* tr = sm.St[w];
  auto active = [&](int qt) { return kw0 < T && (!a.causal || ktw <= qt); };  // wave-uniform
  (void)nkt;

  float vreg[D / 2];
  load_row_operand<D>(vreg, Vp + (size_t)kj * D, kvalid, 1.0f);
  f16v dk[D / 32], dv[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) { dk[nb] = zero16(); dv[nb] = zero16(); }

  const int qt_first = a.causal ? kb0 / BN : 0;
  KvPrefetch<D, TIn> pf;
  if (qt_first < nt) kv_load<D, TIn>(pf, a, Qp, dOp, Sh, head, qt_first, ktw, active(qt_first));
  for (int qt = qt_first; qt < nt; ++qt) {
    const int q0 = qt * BN;
    const bool act = active(qt);
    __syncthreads();
    pf.q.store(sm.Qs, LD, a.scale);
    pf.dO.store(sm.dOs, LD, 1.0f);
    if (act) {
      // stored tile (qt, ktw): element (query l%32, key crow(v, g)) at v * 64 + l
#pragma unroll
      for (int v = 0; v < 16; ++v) tr[c * TLD + crow(v, g)] = pf.s[v];
    }
    reinterpret_cast<f4v*>(sm.rp)[tid] = pf.rp;
#pragma unroll
    for (int i = 0; i < TBL_CH; ++i) {
      const int idx = tid + i * NT;
      if (idx < BN * ts) sm.tbl[idx] = pf.tb[i];
    }
    __syncthreads();
    if (qt + 1 < nt) kv_load<D, TIn>(pf, a, Qp, dOp, Sh, head, qt + 1, ktw, active(qt + 1));
    if (!act) continue;
    f16v s;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = tr[crow(v, g) * TLD + c];  // S: row = query, column = key
    const f16v gg = tile_dot<D>(sm.dOs, LD, vreg);                 // g_ij = dO_i . V_j
    f16v p, ds;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rr = crow(v, g), qr = q0 + rr;
      const RowP& rp = sm.rp[rr];
      const bool ok = qr < T && kvalid && (!a.causal || kj <= qr);
      RowCal rc;
      rc.origin = rp.origin;
      rc.inv_h = rp.inv_h;
      rc.inv_hf = rp.inv_hf;
      rc.kappa = 1.f;
      const Decision d = decide<CAL>(s[v], rc, K, a.tau);
      const Weights wt = weights(d, sm.tbl + rr * ts);
      const bool keep = ok && !d.tail;
      const float wf = (MODE == LERP) ? wt.wL : wt.wN;
      const float Delta = (wt.E1 - wt.E0) * rp.inv_hf;
      float dS = (gg[v] - rp.Di) * rp.invWg * Delta;
      if (FULL) {
        if (s[v] == rp.M || kj == rp.amax) dS += rp.alpha;
        if (CAL == MINMAX && (s[v] == rp.m || kj == rp.amin)) dS += rp.beta;
      }
      p[v] = keep ? wf * rp.invWf : 0.f;
      ds[v] = ok ? (d.tail ? 0.f : dS) : 0.f;
    }
    tile_accum<D>(dv, p, sm.dOs, LD);
    tile_accum<D>(dk, ds, sm.Qs, LD);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int key = kw0 + crow(v, g);
    if (key < T) {
      float* pk = a.dk + hb + (size_t)key * D + c;
      float* pv = a.dv + hb + (size_t)key * D + c;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) {
        pk[32 * nb] = dk[nb][v];
        pv[32 * nb] = dv[nb][v];
      }
    }
  }
}

// ------------------------------------------------------------------------------- launchers
template <int D, int CAL, int MODE, bool FULL, typename TIn>
static hipError_t bwd_go(const Problem& p, const BwdArgs& a, hipStream_t s, int stage) {
  if (stage & 1) {
    const int nqt = (p.T + DQ_BM - 1) / DQ_BM;
    const size_t smem = sizeof(DqSmem<D>) + sizeof(float) * DQ_BM * (p.K + 1);
    hipLaunchKernelGGL((dq_kernel<D, CAL, MODE, FULL, TIn>), dim3(p.nheads * nqt), dim3(NT), smem, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage & 2) {
    const int nkt = (p.T + KV_BN - 1) / KV_BN;
    hipLaunchKernelGGL((dkdv_kernel<D, CAL, MODE, FULL, TIn>), dim3(p.nheads * nkt), dim3(NT), 0, s, a);
    return hipGetLastError();
  }
  return hipSuccess;
}
template <int D, int CAL, int MODE, bool FULL>
static hipError_t bwd_dt(const Problem& p, const BwdArgs& a, hipStream_t s, int st) {
  return p.bf16 ? bwd_go<D, CAL, MODE, FULL, uint16_t>(p, a, s, st) : bwd_go<D, CAL, MODE, FULL, float>(p, a, s, st);
}
template <int D, int CAL, int MODE>
static hipError_t bwd_fl(const Problem& p, const BwdArgs& a, hipStream_t s, int st) {
  return p.full ? bwd_dt<D, CAL, MODE, true>(p, a, s, st) : bwd_dt<D, CAL, MODE, false>(p, a, s, st);
}
template <int D, int CAL>
static hipError_t bwd_md(const Problem& p, const BwdArgs& a, hipStream_t s, int st) {
  switch (p.mode) {
    case LERP: return bwd_fl<D, CAL, LERP>(p, a, s, st);
    case NEAREST_W: return bwd_fl<D, CAL, NEAREST_W>(p, a, s, st);
    default: return bwd_fl<D, CAL, NEAREST_P>(p, a, s, st);
  }
}
template <int D>
static hipError_t bwd_cl(const Problem& p, const BwdArgs& a, hipStream_t s, int st) {
  return p.calib == FWM ? bwd_md<D, FWM>(p, a, s, st) : bwd_md<D, MINMAX>(p, a, s, st);
}
hipError_t launch_backward(const Problem& p, const BwdArgs& a, hipStream_t s, int stages) {
  return p.D == 128 ? bwd_cl<128>(p, a, s, stages) : bwd_cl<64>(p, a, s, stages);
}

}  // namespace kia
