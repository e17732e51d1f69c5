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
//   dq kernel   (query-major, 128 rows per workgroup): D_i, dQ_self = sum dS_self K
//               on the MFMA, the row sums a_i, b_i; then the extremum terms of dQ
//               (gathered rows of K at the arg-max / arg-min; a second sweep adds
//               extra tied keys when a row has any); writes dQ, alpha = a/nA,
//               beta = b/nC and D_i.
//   dkdv kernel (key-major, 128 keys per workgroup): dV += P^T dO, dK += dS^T Q,
//               where dS carries alpha / beta on the arg-max / arg-min keys, so the
//               scatter of the calibration gradient into dK needs no atomics.  Each
//               wave transposes its stored score tile through LDS.
#include "kia_device.hpp"
#include "kia_launch.hpp"

namespace kia {

constexpr int BN = 32;        // keys per tile (dq kernel) / queries per tile (dkdv kernel)
constexpr int DQ_BM = 128;    // query rows per dq workgroup
constexpr int KV_BN = 128;    // key rows per dkdv workgroup
constexpr int TLD = 33;       // row stride of the LDS tile transpose

template <typename T> __device__ __forceinline__ float ld1(const T* p);
template <> __device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p) {
  return __uint_as_float(((uint32_t)*p) << 16);
}

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
__global__ __launch_bounds__(256) void dq_kernel(BwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  DqSmem<D>& sm = *reinterpret_cast<DqSmem<D>*>(smem_raw);
  float* tbl = reinterpret_cast<float*>(smem_raw + sizeof(DqSmem<D>));
  constexpr int LD = D + 4;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, c = l & 31;
  const int T = a.T, K = a.K, ts = K + 1;
  const int nqt = (T + DQ_BM - 1) / DQ_BM;
  const int L = logical_block();
  const int head = L / nqt;
  const int qt = nqt - 1 - (L % nqt);
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

  float doreg[D / 2];
  load_row_operand<D>(doreg, dOp + (size_t)qi * D, qvalid, 1.0f);

  // row record of the forward
  const float M = a.rec.M[row], m = a.rec.m[row];
  const int amax = a.rec.amax[row], amin = a.rec.amin[row];
  const int nA = a.rec.nA[row], nC = a.rec.nC[row];
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
  if (g == 0 && qvalid) a.Dvec[row] = Di;

  const RowCal rc = row_calibration<CAL>(M, m, K, a.tau);
  float* trow = tbl + rl * ts;
  if (qvalid)
    for (int r = g; r <= K; r += 2) trow[r] = grid_value<CAL>(M, m, K, a.tau, r);
  // extra tied extrema (beyond the first index) need a second sweep to find them
  const bool rowties = FULL && qvalid && (M != m) && (nA > 1 || (CAL == MINMAX && nC > 1));
  const bool blockties = __syncthreads_or(rowties);

  double acc_a = 0.0, sds = 0.0;  // calibration sums: terms of both signs, summed in double
  f16v dq[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) dq[nb] = zero16();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    stage_rows<D>(sm.Ks, LD, Kp, k0, T, 1.0f);
    stage_rows<D>(sm.Vs, LD, Vp, k0, T, 1.0f);
    __syncthreads();
    if (qw0 >= T || (a.causal && k0 > qlast_w)) continue;
    const float* St = Sh + tile_index(qtw, kt, a.rec.nt, a.causal) * 1024;
    f16v s;
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = St[v * 64 + l];  // S^T: row = key, column = query
    const f16v gt = tile_dot<D>(sm.Vs, LD, doreg);          // (dO V^T)^T: g_ij = dO_i . V_j
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
      stage_rows<D>(sm.Ks, LD, Kp, k0, T, 1.0f);
      __syncthreads();
      if (qw0 >= T || (a.causal && k0 > qlast_w)) continue;
      const float* St = Sh + tile_index(qtw, kt, a.rec.nt, a.causal) * 1024;
      f16v inj;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float s = St[v * 64 + l];
        const int key = k0 + crow(v, g);
        const bool ok = rowties && key < T && (!a.causal || key <= qi);
        float x = 0.f;
        if (ok && s == M && key != amax) x += alpha;
        if (CAL == MINMAX && ok && s == m && key != amin) x += beta;
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
      a.alpha[row] = alpha;
      a.beta[row] = beta;
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
struct RowP {         // per query row, 64 bytes
  double origin, inv_h;
  float inv_hf, invWf, invWg, Di;
  float alpha, beta, M, m;
  int amax, amin;
};

template <int D>
struct KvSmem {
  float Qs[BN * (D + 4)];
  float dOs[BN * (D + 4)];
  float St[4][BN * TLD];  // per-wave transpose of the stored score tile
  RowP rp[BN];
  // followed in dynamic LDS by the grid table: BN rows x (K + 1) floats
};

template <int D, int CAL, int MODE, bool FULL, typename TIn>
__global__ __launch_bounds__(256) void dkdv_kernel(BwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  KvSmem<D>& sm = *reinterpret_cast<KvSmem<D>*>(smem_raw);
  float* tbl = reinterpret_cast<float*>(smem_raw + sizeof(KvSmem<D>));
  constexpr int LD = D + 4;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, c = l & 31;
  const int T = a.T, K = a.K, ts = K + 1, nt = a.rec.nt;
  const int nkt = (T + KV_BN - 1) / KV_BN;
  const int L = logical_block();
  const int head = L / nkt;
  const int kt = L % nkt;  // low key tiles see the most queries: heaviest first
  const size_t hb = (size_t)head * T * D;
  const TIn* Qp = reinterpret_cast<const TIn*>(a.q) + hb;
  const TIn* Vp = reinterpret_cast<const TIn*>(a.v) + hb;
  const TIn* dOp = reinterpret_cast<const TIn*>(a.dO) + hb;
  const int kb0 = kt * KV_BN, kw0 = kb0 + 32 * w, kj = kw0 + c;
  const int ktw = kw0 / BN;  // the wave's key tile
  const bool kvalid = kj < T;
  const float* Sh = a.rec.S + (size_t)head * a.rec.tiles_per_head * 1024;
  float* tr = sm.St[w];

  float vreg[D / 2];
  load_row_operand<D>(vreg, Vp + (size_t)kj * D, kvalid, 1.0f);
  f16v dk[D / 32], dv[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) { dk[nb] = zero16(); dv[nb] = zero16(); }

  const int qt_first = a.causal ? kb0 / BN : 0;
  for (int qt = qt_first; qt < nt; ++qt) {
    const int q0 = qt * BN;
    const bool active = kw0 < T && (!a.causal || ktw <= qt);  // wave-uniform
    __syncthreads();
    stage_rows<D>(sm.Qs, LD, Qp, q0, T, a.scale);
    stage_rows<D>(sm.dOs, LD, dOp, q0, T, 1.0f);
    if (active) {
      // stored tile (qt, ktw): element (query l%32, key crow(v, g)) at v * 64 + l
      const float* Sg = Sh + tile_index(qt, ktw, nt, a.causal) * 1024;
#pragma unroll
      for (int v = 0; v < 16; ++v) tr[c * TLD + crow(v, g)] = Sg[v * 64 + l];
    }
    if (tid < BN) {
      const int qr = q0 + tid;
      RowP rp;
      if (qr < T) {
        const size_t row = (size_t)head * T + qr;
        const float M = a.rec.M[row], m = a.rec.m[row];
        const RowCal rc = row_calibration<CAL>(M, m, K, a.tau);
        rp.origin = rc.origin;
        rp.inv_h = rc.inv_h;
        rp.inv_hf = rc.inv_hf;
        rp.invWf = 1.0f / ((MODE == LERP) ? a.rec.WL[row] : a.rec.WN[row]);
        rp.invWg = 1.0f / ((MODE == NEAREST_W) ? a.rec.WN[row] : a.rec.WL[row]);
        rp.Di = a.Dvec[row];
        rp.alpha = FULL ? a.alpha[row] : 0.f;
        rp.beta = FULL ? a.beta[row] : 0.f;
        rp.M = M;
        rp.m = m;
        rp.amax = a.rec.amax[row];
        rp.amin = a.rec.amin[row];
      } else {
        rp.origin = 0.0; rp.inv_h = 1.0; rp.inv_hf = 1.f; rp.invWf = 0.f; rp.invWg = 0.f;
        rp.Di = 0.f; rp.alpha = 0.f; rp.beta = 0.f; rp.M = 0.f; rp.m = 0.f;
        rp.amax = -1; rp.amin = -1;
      }
      sm.rp[tid] = rp;
    }
    __syncthreads();
    for (int idx = tid; idx < BN * ts; idx += 256) {
      const int rr = idx / ts, r = idx - rr * ts;
      tbl[idx] = (q0 + rr < T) ? grid_value<CAL>(sm.rp[rr].M, sm.rp[rr].m, K, a.tau, r) : 0.f;
    }
    __syncthreads();
    if (!active) continue;
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
      const Weights wt = weights(d, tbl + rr * ts);
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
    hipLaunchKernelGGL((dq_kernel<D, CAL, MODE, FULL, TIn>), dim3(p.nheads * nqt), dim3(256), smem, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage & 2) {
    const int nkt = (p.T + KV_BN - 1) / KV_BN;
    const size_t smem = sizeof(KvSmem<D>) + sizeof(float) * BN * (p.K + 1);
    hipLaunchKernelGGL((dkdv_kernel<D, CAL, MODE, FULL, TIn>), dim3(p.nheads * nkt), dim3(256), smem, s, a);
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
