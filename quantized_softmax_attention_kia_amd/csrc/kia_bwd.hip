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
//   FWM     a = -sum_{window} gamma_j Delta_j (every key of the resolved grid of App. D.4 is in
//           the window; a key floored onto the window edge has no slope and adds nothing);
// a is added to the score gradient of the arg-max key(s) and b to the arg-min
// key(s), split evenly among ties.
//
// The dq kernel reads the scores the forward stored (no score recomputation) and takes
// every bin decision of the backward; the dkdv kernel only contracts what it wrote:
//   dq kernel   (query-major, 64 rows per workgroup): D_i, g = dO V^T and dS on the MFMA
//               and the VALU, dQ_self = sum dS_self K, the row sums a_i, b_i, then the
//               extremum terms of dQ (gathered rows of K at the arg-max / arg-min; a second
//               sweep adds extra tied keys when a row has any).  Per tile it also writes the
//               normalized forward weights P and the score gradients dS, in the tile order of
//               the stored scores, and after the sweep adds alpha_i = a_i/nA_i and
//               beta_i = b_i/nC_i into dS at the row's extremum keys (each element is patched
//               by the lane that wrote it).
//   dkdv kernel (key-major, 128 keys per workgroup, four waves of 32 that share each staged
//               query tile): dV += P^T dO, dK += dS^T Q from those tiles: no decisions, no
//               row records, no atomics.
// Both sweep their tiles while the next tile's operands are already being loaded.
// Built once per calibration: KIA_CAL (a kia::Calib value) selects the dq kernels this build
// supplies; the build with KIA_CAL = 0 also supplies the dkdv kernel.
#include "kia_device.hpp"
#include "kia_launch.hpp"

#ifndef KIA_CAL
#error "build with -DKIA_CAL=<calibration>"
#endif

namespace kia {

constexpr int NW = 2;         // waves per dq workgroup
constexpr int NT = 64 * NW;   // threads per dq workgroup
constexpr int BN = 32;        // keys per tile (dq kernel) / queries per tile (dkdv kernel)
constexpr int DQ_BM = 32 * NW;  // query rows per dq workgroup
constexpr int KV_NW = 4;        // waves per dkdv workgroup: one staged query tile serves four key tiles
constexpr int KV_NT = 64 * KV_NW;
constexpr int KV_BN = 32 * KV_NW;  // key rows per dkdv workgroup

template <typename T> __device__ __forceinline__ float ld1(const T* p);
template <> __device__ __forceinline__ float ld1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ld1<uint16_t>(const uint16_t* p) {
  return __uint_as_float(((uint32_t)*p) << 16);
}

// Offset of element (query a, key b) inside a stored tile (scores, P, dS): v * 64 + a + 32 g
// where b = crow(v, g).  Lane l = a + 32 g of the wave owning the query tile holds it.
__device__ __forceinline__ int stored_offset(int a, int b) {
  const int g = (b >> 2) & 1, v = 4 * (b >> 3) + (b & 3);
  return v * 64 + a + 32 * g;
}
__device__ __forceinline__ int stored_lane_group(int b) { return (b >> 2) & 1; }

// ============================================================================ dq kernel
// BF16-exp forms g = dO V^T in double (fp64 MFMA): V rows as floats, row stride D + 4 (operand
// reads free of bank conflicts), and each wave's 32 x 32 tile of g, transposed through LDS
template <int D> constexpr int vns() { return D + 4; }
template <int D, int NS, bool F64>
constexpr int dq_vn_elems() {
  return F64 && 2 * BN * vns<D>() > NS * BN * np<D>() ? 2 * BN * vns<D>() : NS * BN * np<D>();
}
template <int D, int NS, bool F64>
struct DqSmem {
  __align__(16) __bf16 KT[NS * D * TP];         // K^T of the key tile, bf16 slices (dQ += dS K)
  __align__(16) __bf16 VN[dq_vn_elems<D, NS, F64>()];  // V rows of the key tile, bf16 slices (g = V dO^T)
  double GX[F64 ? NW : 1][F64 ? 32 * 33 : 1];
  float alpha[DQ_BM], beta[DQ_BM], mean[DQ_BM];
  int amax[DQ_BM], amin[DQ_BM];
  // followed in dynamic LDS by the grid table: MinMax DQ_BM rows x (K + 3) floats, FWM one
  // row of lres + K + 3 floats
};

__host__ __device__ constexpr int dq_table_floats(int CAL, int K, int lres) {
  return CAL == MINMAX ? DQ_BM * (K + 3) : (CAL == EXPB ? 0 : lres + K + 3);
}
// bin-mean modes: after the grid table, per row the bins' means of e^z and of g
template <int D, int CAL, int MODE, typename TIn>
size_t dq_smem_bytes(int K, int lres) {
  return sizeof(DqSmem<D, nslices<TIn>(), MODE == EXPBF>) +
         sizeof(float) * (dq_table_floats(CAL, K, lres) + (is_binmean(MODE) ? 2 * DQ_BM * BINM_MAXB : 0));
}

// GK: GK_SUMS (full, max_only, min_only: the calibration sums, with the extremum terms that
// a.keepM / a.keepm select), GK_DETACHED, or GK_P1 (detached; each row's dS mean over its visible
// keys is recorded for the dkdv kernel and taken out of dQ through the sum of the visible K rows).
// At D = 64 the register budget is held to two waves per SIMD.
template <int D, int CAL, int MODE, int GK, typename TIn, int NB = BINM_MAXB>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void dq_kernel(BwdArgs a) {
  constexpr bool SUMS = GK == GK_SUMS, P1 = GK == GK_P1;
  constexpr bool PC = p_coded(CAL, MODE);  // P written as table indices beside the row's table
  constexpr int NS = nslices<TIn>();
  // BF16-exp: dL/dw is rounded to bfloat16, so it is formed from exact parts: g in double (fp64
  // MFMA), D_i from the forward's double output (O and its residual), W from its float and residual
  constexpr bool F64 = MODE == EXPBF;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  DqSmem<D, NS, F64>& sm = *reinterpret_cast<DqSmem<D, NS, F64>*>(smem_raw);
  float* tbl = reinterpret_cast<float*>(smem_raw + sizeof(DqSmem<D, NS, F64>));
  float* VF = reinterpret_cast<float*>(sm.VN);  // F64: V rows as floats
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 5, c = l & 31;
  const int T = a.T, K = a.K;  // grid table: e^{b_0} .. e^{b_K}, then two zeros
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
  const size_t tbase = (size_t)head * a.rec.tiles_per_head;
  const float* Sh = a.rec.S + tbase * 1024;
  float* Ph = a.pt + tbase * 1024;
  uint8_t* Pch = a.pcode + tbase * 1024;
  float* dSh = a.dst + tbase * 1024;
  auto active = [&](int kt) { return qw0 < T && (!a.causal || kt * BN <= qlast_w); };

  // the row's loads first (record, the rows of O and dO), so that their latencies overlap;
  // rows past T read row 0 of the head and are zeroed or never used
  const float M = a.rec.M[row], m = a.rec.m[row];
  const int amax = a.rec.amax[row], amin = a.rec.amin[row];
  const int nA = a.rec.nA[row], nC = a.rec.nC[row];
  const float Wf = is_nearest(MODE) ? a.rec.WN[row] : a.rec.WL[row];
  const float Wg = (MODE == NEAREST_W) ? a.rec.WN[row] : a.rec.WL[row];
  f4v xo[D / 8], yo[D / 8], xr[F64 ? D / 8 : 1];  // xr: F64, the residual of O
  {
    const int qc = qvalid ? qi : 0;
    const float* X = ((MODE == NEAREST_P) ? a.rec.OL : a.o) + hb + (size_t)qc * D + 4 * g;
    const TIn* Y = dOp + (size_t)qc * D + 4 * g;
#pragma unroll
    for (int q = 0; q < D / 8; ++q) {
      xo[q] = *reinterpret_cast<const f4v*>(X + 8 * q);
      yo[q] = Ld<TIn>::four(Y + 8 * q);
      if (F64) xr[q] = *reinterpret_cast<const f4v*>(a.rec.OL + hb + (size_t)qc * D + 4 * g + 8 * q);
    }
  }
  const double Wgd = F64 ? (double)Wg + (double)a.rec.WN[row] : (double)Wg;
  // F64: the A operand of g = dO V^T, dO[qw0 + 16 qh + l%16][4 s + l/16] (zero past T)
  float doA[F64 ? 2 : 1][F64 ? D / 4 : 1];
  if constexpr (F64) {
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      const int r = qw0 + 16 * qh + (l & 15);
#pragma unroll
      for (int s4 = 0; s4 < D / 4; ++s4) doA[qh][s4] = r < T ? Ld<TIn>::one(dOp + (size_t)r * D + 4 * s4 + (l >> 4)) : 0.f;
    }
  }
  // the lane's dO row as bf16 slices, columns 16 kb + 8 g ..: the B operand of every g = V dO^T
  Split8 dos[D / 16];
  {
    RowOp<D, TIn> dr;
    dr.load(dOp, qi, T);
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) dos[kb] = dr.split(kb);
  }
  const float invWf = 1.0f / Wf, invWg = 1.0f / Wg;

  // D_i = dO_i . O_i (O^L_i for Nearest with Prob-STE): sum_j P_j g_j at the normalization point
  float Di;
  double Did;  // F64: in double, from O and its residual
  {
    double part = 0.0;
#pragma unroll
    for (int q = 0; q < D / 8; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = fma((double)yo[q][e], (double)xo[q][e], part);
        if (F64) part = fma((double)yo[q][e], (double)xr[q][e], part);
      }
    if (!qvalid) part = 0.0;
    Did = part + __shfl_xor(part, 32);
    Di = (float)Did;
  }

  const RowCal rc = row_calibration<CAL>(M, m, K, a.tau);
  // MinMax: one table row per query row (zero for rows past T); FWM: one table for all rows, from
  // lres levels below the window (resolved grid) to K (rows past T see no visible key)
  float* trow = tbl;
  if (CAL == MINMAX) {
    trow = tbl + rl;  // interval-major: entry r of row rl at r * DQ_BM + rl
    for (int r = g; r <= K + 2; r += 2) trow[r * DQ_BM] = qvalid && r <= K ? grid_value<CAL>(M, m, K, a.tau, r) : 0.f;
  } else if (CAL != EXPB) {  // the exponential baselines have no grid
    trow = tbl + a.lres;
    for (int i = tid; i <= a.lres + K + 2; i += NT) tbl[i] = i <= a.lres + K ? grid_value<CAL>(M, m, K, a.tau, i - a.lres) : 0.f;
  }
  // extra tied extrema (beyond the first index) need a second sweep to find them
  // (a MinMax row with M == m has every grid value 1: both extremum terms vanish; FWM records m = M)
  const bool flat = CAL == MINMAX && M == m;
  const bool rowties = SUMS && qvalid && !flat && ((a.keepM && nA > 1) || (CAL == MINMAX && a.keepm && nC > 1));
  const bool blockties = __syncthreads_or(rowties);

  double acc_a = 0.0, sds = 0.0;  // calibration sums of the row (terms of both signs)
  // A row whose maximum is attained by one key: that key's own score gradient gamma Delta and the
  // maximum's calibration term alpha cancel (the key's own dw/dM is -Delta at t = 1), so both are
  // formed together from the other keys' terms, without that cancellation.  The key stays out of
  // the sums and of the dQ products; xself / xown keep its own gamma Delta and gamma K (Delta +
  // dw/dM), and after the sweep its coefficient (self plus alpha) goes into dS and dQ at once.
  const bool xrow = SUMS && qvalid && !flat && nA == 1;
  float xself = 0.f, xown = 0.f;
  f16v dq[D / 32], pk[P1 ? D / 32 : 1];  // pk: P1 only, the sum of the visible K rows
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) dq[nb] = zero16();
  if (P1) {
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) pk[nb] = zero16();
  }

  constexpr bool BM = is_binmean(MODE);
  // stored scores of a tile: query c, key k0 + crow(v, g); loaded one tile ahead
  auto load_s = [&](int kt, float (&dst)[16]) {
    const float* St = Sh + tile_index(qtw, kt, a.rec.nt, a.causal) * 1024 + l;
#pragma unroll
    for (int v = 0; v < 16; ++v) dst[v] = St[v * 64];
  };

  // bin-mean modes (§5, App. I): a first sweep sums, per Nearest bin of the row, e^{s - M}, the
  // member count and the upstream gradient g (keys below an FWM window belong to no bin), per
  // lane in registers and then over the row's two lanes; per row it keeps the bins' means of e^z
  // and, for dS_k = e^{z_k} / W^C (gbar_b(k) - D^C), the differences gbar_b - D^C (W^C = sum_b S_b,
  // D^C = sum_j P^C_j g_j).  The sums are kept in double: D^C is a weighted mean of the bins' mean
  // gradients, which can be large beside the differences it is taken from
  float* bmean = tbl + dq_table_floats(CAL, K, a.lres) + rl * BINM_MAXB;  // [DQ_BM][BINM_MAXB]
  float* bgd = bmean + DQ_BM * BINM_MAXB;
  float invWC = 0.f;
  if constexpr (BM) {
    double bs[NB], bg[NB];
    float bn[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) { bs[q] = 0.0; bn[q] = 0.f; bg[q] = 0.0; }
    RowRegs<D, TIn, NT> vp;
    vp.load(Vp, 0, T);
    for (int kt = 0; kt < ntiles; ++kt) {
      const int k0 = kt * BN;
      __syncthreads();
      vp.template store<NS>(sm.VN);
      __syncthreads();
      if (kt + 1 < ntiles) vp.load(Vp, k0 + BN, T);
      if (!active(kt)) continue;
      float s[16];
      load_s(kt, s);
      f16v gt = zero16();
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) gt = mfma_split<NS, NS>(load_an<D, NS>(sm.VN, c, kb), dos[kb], gt);
      const int lim = (qvalid ? (a.causal ? min(qi, T - 1) : T - 1) : -1) - k0 - 4 * g;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const Decision d = decide<CAL>(s[v], rc, K, a.tau);
        const bool in = (crow(v, 0) <= lim) & !d.tail;
        const int ell = d.r + (d.t >= 0.5f ? 1 : 0);
        const float x = __expf(s[v] - M);
#pragma unroll
        for (int q = 0; q < NB; ++q) {
          const bool hit = in && ell == q;
          bs[q] += hit ? (double)x : 0.0;
          bn[q] += hit ? 1.f : 0.f;
          bg[q] += hit ? (double)gt[v] : 0.0;
        }
      }
    }
    double WC = 0.0, GC = 0.0, gbar[NB];  // bins past K hold nothing: NB of them cover every member
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      bs[q] += __shfl_xor(bs[q], 32);
      bn[q] += __shfl_xor(bn[q], 32);
      bg[q] += __shfl_xor(bg[q], 32);
      gbar[q] = bn[q] > 0.f ? bg[q] / (double)bn[q] : 0.0;
      WC += bs[q];
      GC = fma(bs[q], gbar[q], GC);
    }
    const double DC = WC > 0.0 ? GC / WC : 0.0;
    if (g == 0) {
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        bmean[q] = bn[q] > 0.f ? (float)(bs[q] / (double)bn[q]) : 0.f;
        bgd[q] = (float)(gbar[q] - DC);
      }
    }
    invWC = WC > 0.0 ? (float)(1.0 / WC) : 0.f;
  }

  if constexpr (PC) {
    // the row's P by table index (bin means under bin mean, else the grid), index K + 1 zero
    if (qvalid) {
      float* pr = a.ptab + row * (size_t)(K + 2);
      for (int j = g; j <= K + 1; j += 2) {
        float e = 0.f;
        if (j <= K) e = MODE == BINM ? bmean[j] : trow[j * (CAL == MINMAX ? DQ_BM : 1)];
        pr[j] = e * invWf;
      }
    }
  }

  PairRegs<D, TIn, NT> kr;  // K rows of the next key tile, staged as the workgroup's K^T slices
  RowRegs<D, TIn, NT> vr;   // V rows of the next key tile, staged as natural-layout slices
  kr.load(Kp, 0, T);
  if (!BM) vr.load(Vp, 0, T);
  float snext[16];
  if (active(0)) load_s(0, snext);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * BN;
    const bool act = active(kt);
    const size_t to = tile_index(qtw, act ? kt : 0, a.rec.nt, a.causal) * 1024;
    float s[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = snext[v];
    if (kt + 1 < ntiles && active(kt + 1)) load_s(kt + 1, snext);
    __syncthreads();
    kr.template store_t<NS>(sm.KT);
    if (F64) vr.store_f32(VF, vns<D>());
    else if (!BM) vr.template store<NS>(sm.VN);
    __syncthreads();
    if (kt + 1 < ntiles) {
      kr.load(Kp, k0 + BN, T);
      if (!BM) vr.load(Vp, k0 + BN, T);
    }
    if (!act) continue;
    float* Pw = Ph + to;
    uint8_t* Pcw = Pch + to;
    float* dSw = dSh + to;
    // (dO V^T)^T as bf16 slice products: register v holds g = dO_i . V_j for query c, key k0 + crow(v, g)
    f16v gt = zero16();
    if (!BM && !F64) {
#pragma unroll
      for (int kb = 0; kb < D / 16; ++kb) gt = mfma_split<NS, NS>(load_an<D, NS>(sm.VN, c, kb), dos[kb], gt);
    }
    // F64: g in double, block (qh, kh) element i at query 16 qh + l/16 + 4 i, key 16 kh + l%16, then
    // through LDS to the lane's own elements (query c, key crow(v, g))
    double g64[F64 ? 16 : 1];
    if constexpr (F64) {
      d4v gx[2][2];
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) { gx[qh][0] = zero4d(); gx[qh][1] = zero4d(); }
#pragma unroll
      for (int s4 = 0; s4 < D / 4; ++s4) {
        const int d = 4 * s4 + (l >> 4);
        const double b0 = VF[(l & 15) * vns<D>() + d], b1 = VF[(16 + (l & 15)) * vns<D>() + d];
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
          gx[qh][0] = mfma_f64(doA[qh][s4], b0, gx[qh][0]);
          gx[qh][1] = mfma_f64(doA[qh][s4], b1, gx[qh][1]);
        }
      }
      double* G = sm.GX[w];
#pragma unroll
      for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 4; ++i) G[(16 * qh + (l >> 4) + 4 * i) * 33 + 16 * kh + (l & 15)] = gx[qh][kh][i];
      wave_lds_sync();
#pragma unroll
      for (int v = 0; v < 16; ++v) g64[v] = G[c * 33 + crow(v, g)];
      wave_lds_sync();  // read before the next tile's g is written
    }
    // half tiles (keys crow(v, g), v = 8 b .. 8 b + 7): decisions, weights and dS, then their share of
    // dQ += dS K as bf16 slice products (dS in the A layout: query c, keys crow(8 b + e, g)).  A key
    // that is not visible, or in the FWM tail, takes the table's two zero entries (r = K + 1): its
    // weight, slope, dS and calibration terms are then exactly zero.  A floored tail key keeps the
    // window edge's weight and has no slope, hence no dS and no calibration term.
    const int lim = (qvalid ? (a.causal ? min(qi, T - 1) : T - 1) : -1) - k0 - 4 * g;  // crow(v, 0) <= lim
    // at D = 128 (one wave per SIMD, registers to spare) each key tile's dS K goes into a fresh
    // accumulator that joins the running dQ once: a long row (T = 8192: 256 key tiles) then takes one
    // rounding of its running sum per tile instead of one per slice product
    constexpr bool FRESH = D == 128 && !P1;
    f16v tq[FRESH ? D / 32 : 1];
    if (FRESH) {
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) tq[nb] = zero16();
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float ds[8];
      // the half tile's calibration terms, summed in float (8 terms) and then joined in double
      float hs = 0.f, ha = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int v = 8 * b + j;
        const float gam = (gt[v] - Di) * invWg;
        float dS, pw;
        int code = 0;  // PC: the index of pw in the row's table
        Decision d;
        Weights wt;
        float Delta = 0.f;
        if constexpr (BM) {
          // bin mean: dS_k = e^{z_k} / W^C (gbar_b(k) - D^C); the forward's weight is the bin's
          // mean (bin mean) or the grid value at the Nearest index (the hybrid)
          d = decide<CAL>(s[v], rc, K, a.tau);
          const bool in = (crow(v, 0) <= lim) & !d.tail;
          const int ell = min(d.r + (d.t >= 0.5f ? 1 : 0), NB - 1);
          dS = in ? __expf(s[v] - M) * invWC * bgd[ell] : 0.f;
          code = in ? ell : K + 1;
          if (MODE == BINM) pw = in ? bmean[ell] : 0.f;
          else pw = in ? weights_cal<CAL, CAL == MINMAX ? DQ_BM : 1>(d, trow, a.lres, a.res_far != 0, K, a.tau).wN : 0.f;
        } else if constexpr (CAL == EXPB) {
          // exponential baselines: the weight as the forward took it.  The forward's float form,
          // where the forward kept it, gave the exact form's value on the stored score; where it
          // retook it, the stored score is exact.  Here the float form is checked against its
          // arithmetic alone and the exact form taken where that cannot settle the rounding.
          // dL/dz = gamma dw/dz, for BF16-exp in bfloat16: gamma rounded where it enters the
          // bfloat16 weight, the product (exact in float) rounded once more
          const bool vis = crow(v, 0) <= lim;
          bool rs = false, re = false;
          ExpW ew = exp_weight_fast<MODE>(s[v], M, 0.f, &rs, &re);
          if (rs || re) ew = exp_weight_exact<MODE>(s[v], M);
          pw = vis ? ew.w : 0.f;
          if constexpr (F64) {
            // dL/dw in double, rounded once to bfloat16 (exact parts: the rounding is the exact
            // value's wherever that lies farther than double rounding error from a midpoint)
            const float gb = (float)bf16_round_d((g64[v] - Did) / Wgd);
            dS = vis ? bf16_round(gb * ew.d) : 0.f;
          } else {
            dS = vis ? gam * ew.d : 0.f;
          }
        } else {
          d = decide<CAL>(s[v], rc, K, a.tau);
          if ((crow(v, 0) > lim) | (CAL == FWM && d.tail)) d.r = K + 1;
          wt = weights_cal<CAL, CAL == MINMAX ? DQ_BM : 1>(d, trow, a.lres, a.res_far != 0, K, a.tau);
          Delta = (CAL == FWM_FLOOR && d.tail) ? 0.f : wt.E0 * rc.slope;
          dS = gam * Delta;
          pw = is_nearest(MODE) ? wt.wN : wt.wL;
          code = d.r > K ? K + 1 : d.r + (d.t >= 0.5f ? 1 : 0);  // wN is the table's entry there
        }
        // the forward's normalized weight: P^L for LERP, the hard P^N for Nearest
        if constexpr (PC) Pcw[v * 64 + l] = (uint8_t)code;
        else Pw[v * 64 + l] = pw * invWf;
        dSw[v * 64 + l] = dS;
        if (P1) hs += dS;
        if (SUMS) {
          const bool xk = xrow & (k0 + crow(v, g) == amax);  // the row's only arg-max key
          xself += xk ? dS : 0.f;
          hs += xk ? 0.f : dS;
          if (CAL == MINMAX) {
            const float rf = (float)d.r;
            // K * dw/dM = (r - K) w + t e^{b_{r+1}} - kappa (r + t) Delta
            const float dMk = fmaf(rf - (float)K, wt.wL, d.t * wt.E1) - rc.kappa * (rf + d.t) * Delta;
            ha = fmaf(gam, xk ? 0.f : dMk, ha);
            // K (Delta + dw/dM) = (K - kappa (r + t)) Delta + (r - K) w + t e^{b_{r+1}}: 0 at t = 1
            if (xk) xown += gam * fmaf((float)K - rc.kappa * (rf + d.t), Delta, fmaf(rf - (float)K, wt.wL, d.t * wt.E1));
          }
          dS = xk ? 0.f : dS;
        }
        ds[j] = dS;
      }
      if (SUMS || P1) sds += (double)hs;
      if (SUMS && CAL == MINMAX) acc_a += (double)ha;
      const Split8 dss = split8(ds);
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) {
        if (FRESH) tq[nb] = mfma_split<NS>(dss, load_bt<D, NS>(sm.KT, b, 32 * nb + c), tq[nb]);
        else dq[nb] = mfma_split<NS>(dss, load_bt<D, NS>(sm.KT, b, 32 * nb + c), dq[nb]);
      }
      if (P1) {
        // the sum of the row's visible K rows, for the mean's share of dQ: a 0 / 1 mask (exact in
        // bf16) times the K^T slices
        uint32_t mk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          mk[e] = (crow(8 * b + 2 * e, 0) <= lim ? 0x3f80u : 0u) | (crow(8 * b + 2 * e + 1, 0) <= lim ? 0x3f800000u : 0u);
        Split8 ms;
        __builtin_memcpy(&ms.h, mk, 16);
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) pk[nb] = mfma_split<NS, 1>(ms, load_bt<D, NS>(sm.KT, b, 32 * nb + c), pk[nb]);
      }
    }
    if (FRESH) {
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) dq[nb] += tq[nb];
    }
  }

  // extremum terms of the row: alpha per tied max key, beta per tied min key
  float alpha = 0.f, beta = 0.f;
  const bool inject = SUMS && qvalid && !flat;
  float mean = 0.f;  // P1: the row's mean of dS over its visible keys
  if (P1) {
    sds += __shfl_xor(sds, 32);
    mean = qvalid ? (float)(sds / (double)(a.causal ? qi + 1 : T)) : 0.f;
    if (g == 0 && qvalid) a.rowmean[row] = mean;
  }
  if (SUMS) {
    acc_a += __shfl_xor(acc_a, 32);
    sds += __shfl_xor(sds, 32);
    xself += __shfl_xor(xself, 32);  // the other lane of the row holds 0
    xown += __shfl_xor(xown, 32);
    if (inject) {
      if (xrow) {
        // alpha here is the arg-max key's whole coefficient: its own gamma Delta plus the
        // maximum's term (or its own term alone when that term is dropped)
        if (CAL == MINMAX) {
          const double comb = (acc_a + (double)xown) / (double)K;
          alpha = a.keepM ? (float)comb : xself;
          beta = a.keepm ? (float)((-sds - comb) / (double)nC) : 0.f;
        } else {
          alpha = a.keepM ? (float)(-sds) : xself;
        }
      } else if (CAL == MINMAX) {
        const double A = acc_a / (double)K;
        const double Bm = -sds - A;
        alpha = a.keepM ? (float)(A / (double)nA) : 0.f;
        beta = a.keepm ? (float)(Bm / (double)nC) : 0.f;
      } else {
        alpha = a.keepM ? (float)(-sds / (double)nA) : 0.f;
      }
    }
    // dS of the first arg-max / arg-min key of the row gains alpha / beta (the arg-max key of an
    // xrow row takes its coefficient), written by the lane that stored the element (program order
    // makes its own store visible to it)
    if (inject && (a.keepM || xrow) && g == stored_lane_group(amax % BN)) {
      float* e = dSh + tile_index(qtw, amax / BN, a.rec.nt, a.causal) * 1024 + stored_offset(c, amax % BN);
      *e = xrow ? alpha : *e + alpha;
    }
    if (CAL == MINMAX && inject && a.keepm && g == stored_lane_group(amin % BN)) {
      float* e = dSh + tile_index(qtw, amin / BN, a.rec.nt, a.causal) * 1024 + stored_offset(c, amin % BN);
      *e = *e + beta;
    }
  }
  if (SUMS && blockties) {
    // second sweep: tied keys other than the first arg-max / arg-min
    for (int kt = 0; kt < ntiles; ++kt) {
      const int k0 = kt * BN;
      __syncthreads();
      kr.load(Kp, k0, T);
      kr.template store_t<NS>(sm.KT);
      __syncthreads();
      if (!active(kt)) continue;
      const size_t to = tile_index(qtw, kt, a.rec.nt, a.causal) * 1024;
      const float* St = Sh + to;
      float inj[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float sv = St[v * 64 + l];
        const int key = k0 + crow(v, g);
        const bool ok = rowties && key < T && (!a.causal || key <= qi);
        float x = 0.f;
        if (ok && sv == M && key != amax) x += alpha;
        if (CAL == MINMAX && ok && sv == m && key != amin) x += beta;
        inj[v] = x;
        if (x != 0.f) dSh[to + v * 64 + l] += x;  // stored by this lane in the first sweep
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const Split8 is = split8(inj + 8 * b);
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) dq[nb] = mfma_split<NS>(is, load_bt<D, NS>(sm.KT, b, 32 * nb + c), dq[nb]);
      }
    }
  }
  if (g == 0) {
    sm.alpha[rl] = alpha;
    sm.beta[rl] = beta;
    sm.mean[rl] = mean;
    sm.amax[rl] = qvalid ? amax : 0;
    sm.amin[rl] = qvalid ? amin : 0;
  }
  __syncthreads();
  // the extremum keys' K rows of all 16 rows first (every row records valid keys, so no load
  // waits behind a row test), then the stores
  constexpr int NX = SUMS ? 16 : 1, NXM = SUMS && CAL == MINMAX ? 16 : 1;
  float xa[NX][D / 32], xb[NXM][D / 32];
  if (SUMS) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r2 = 32 * w + crow(v, g);
      const TIn* ka = Kp + (size_t)sm.amax[r2] * D + c;
      const TIn* kb = Kp + (size_t)sm.amin[r2] * D + c;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) {
        xa[v][nb] = ld1<TIn>(ka + 32 * nb);
        if (CAL == MINMAX) xb[v][nb] = ld1<TIn>(kb + 32 * nb);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int qrow = qw0 + crow(v, g);
    if (qrow < T) {
      const int r2 = 32 * w + crow(v, g);
      const float al = sm.alpha[r2], be = sm.beta[r2];
      float* out = a.dq + hb + (size_t)qrow * D + c;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) {
        float val = dq[nb][v];
        if (SUMS) {
          val = fmaf(al, xa[v][nb], val);
          if (CAL == MINMAX) val = fmaf(be, xb[v][nb], val);
        }
        if (P1) val = fmaf(-sm.mean[r2], pk[nb][v], val);
        out[32 * nb] = val * a.scale;
      }
    }
  }
}

// ============================================================================ dkdv kernel

// rows of a query tile times the longest table of P values by index (K <= 64)
constexpr int KV_PT = BN * 66;
template <int D, int NS, bool PC>
struct KvSmem {
  __bf16 QT[NS * D * TP];   // Q^T of the query tile, bf16 slices
  __bf16 dOT[NS * D * TP];  // dO^T of the query tile
  float pt[PC ? KV_PT : 1];  // coded P: the query tile's rows of P values by index
};

// Lane (c, g) loads, for its key c of the wave's key tile, the stored P and dS of the queries
// crow(v, g) (v = 0..15): in a stored tile they sit at v_c * 64 + 32 g_c + (query) with
// c = crow(v_c, g_c), so they form four aligned runs of four floats.
// Under P1 the tile also carries the rows' means of the detached dS (queries crow(v, g)).
// Coded P (PC): the same runs hold one byte per element, four to a 32-bit word.
template <bool P1, bool PC>
struct KvTile {
  f4v p[PC ? 1 : 4], ds[4];
  uint32_t pc[PC ? 4 : 1];
  float mean[P1 ? 16 : 1];
};
template <bool P1, bool PC>
__device__ __forceinline__ void kv_load(KvTile<P1, PC>& t, const BwdArgs& a, size_t tbase, int head, int qt,
                                        int ktw) {
  const int l = threadIdx.x & 63, g = l >> 5, c = l & 31;
  const size_t to = (tbase + tile_index(qt, ktw, a.rec.nt, a.causal)) * 1024 +
                    (4 * (c >> 3) + (c & 3)) * 64 + 32 * ((c >> 2) & 1) + 4 * g;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (PC) t.pc[q] = *reinterpret_cast<const uint32_t*>(a.pcode + to + 8 * q);
    else t.p[q] = *reinterpret_cast<const f4v*>(a.pt + to + 8 * q);
    t.ds[q] = *reinterpret_cast<const f4v*>(a.dst + to + 8 * q);
  }
  if (P1) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int query = qt * BN + crow(v, g);
      t.mean[v] = query < a.T ? a.rowmean[(size_t)head * a.T + query] : 0.f;
    }
  }
}

// P1: subtract each query row's mean of the detached dS from its visible elements.
// PC: P arrives as table indices and is looked up in the query rows' tables (staged with Q, dO).
// PT1: the query tile's table rows fit one element per thread (K <= 6).
template <int D, typename TIn, bool P1, bool PC, bool PT1 = false>
__global__ __launch_bounds__(KV_NT) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void dkdv_kernel(BwdArgs a) {
  constexpr int NS = nslices<TIn>();
  __shared__ KvSmem<D, NS, PC> sm;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 5, c = l & 31;
  const int T = a.T, nt = a.rec.nt;
  int head, kt;
  block_work(a.nheads, head, kt);  // low key tiles see the most queries: heaviest first
  const size_t hb = (size_t)head * T * D;
  const TIn* Qp = reinterpret_cast<const TIn*>(a.q) + hb;
  const TIn* dOp = reinterpret_cast<const TIn*>(a.dO) + hb;
  const int kb0 = kt * KV_BN, kw0 = kb0 + 32 * w;
  const int ktw = kw0 / BN;  // the wave's key tile
  const size_t tbase = (size_t)head * a.rec.tiles_per_head;
  auto active = [&](int qt) { return kw0 < T && (!a.causal || ktw <= qt); };  // wave-uniform

  // At D = 128 (long rows) the running sums are kept in double: a key that carries much of the
  // probability of many rows sums terms far larger than its result (dV_j = sum_i P_ij dO_i with P
  // near 1 in hundreds of rows), and float roundings of a running sum of 8192 rows would reach the
  // result.  Each query tile's products go into one fresh float accumulator, first dV's and then
  // dK's, and join the double sums once per tile.  (P1 keeps the float sums: its extra operands
  // leave no registers for them.)
  constexpr bool DSUM = D == 128 && !P1;
  f16v dk[DSUM ? 1 : D / 32], dv[DSUM ? 1 : D / 32];
  double dkd[DSUM ? D / 32 : 1][DSUM ? 16 : 1], dvd[DSUM ? D / 32 : 1][DSUM ? 16 : 1];
  if constexpr (DSUM) {
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) { dkd[nb][v] = 0.0; dvd[nb][v] = 0.0; }
  } else {
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) { dk[nb] = zero16(); dv[nb] = zero16(); }
  }

  const int qt_first = a.causal ? kb0 / BN : 0;
  // the workgroup's Q and dO rows of the next query tile, staged through LDS as bf16 slices;
  // the wave's P and dS of a tile, in two buffers taken in turn
  PairRegs<D, TIn, KV_NT> qr, dr;
  KvTile<P1, PC> t0, t1;
  // coded P: the query tile's table rows are contiguous (rows past T are never looked up)
  constexpr int PT_PER = PC && !PT1 ? (KV_PT + KV_NT - 1) / KV_NT : 1;
  const int K2 = a.K + 2;
  float ptr[PT_PER];
  auto pt_load = [&](int qt) {
    const float* src = a.ptab + ((size_t)head * T + (size_t)qt * BN) * K2;
    const int n = min(BN, T - qt * BN) * K2;
#pragma unroll
    for (int u = 0; u < PT_PER; ++u) {
      const int i = tid + u * KV_NT;
      ptr[u] = i < n ? src[i] : 0.f;
    }
  };
  if (PC && qt_first < nt) pt_load(qt_first);
  auto stage = [&](int qt) {
    __syncthreads();
    qr.template store_t<NS>(sm.QT);
    dr.template store_t<NS>(sm.dOT);
    if (PC) {
#pragma unroll
      for (int u = 0; u < PT_PER; ++u) {
        const int i = tid + u * KV_NT;
        if (i < BN * K2) sm.pt[i] = ptr[u];
      }
    }
    __syncthreads();
    if (qt + 1 < nt) {
      qr.load(Qp, (qt + 1) * BN, T);
      dr.load(dOp, (qt + 1) * BN, T);
      if (PC) pt_load(qt + 1);
    }
  };
  auto contract = [&](const KvTile<P1, PC>& t, int qt) {
    // element (query crow(v, g), key c) of P and dS; zero where masked
    float p[16], ds[16];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (PC) {
          // query 8 q + 4 g + e of the tile: index K + 1 (masked, tail) is P = 0
          const int code = (int)((t.pc[q] >> (8 * e)) & 0xffu);
          p[4 * q + e] = code <= a.K ? sm.pt[(8 * q + 4 * g + e) * K2 + code] : 0.f;
        } else {
          p[4 * q + e] = t.p[q][e];
        }
        ds[4 * q + e] = t.ds[q][e];
      }
    if (P1) {
      // the query row's mean of the detached dS comes off every visible element
      const int key = kw0 + c;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int query = qt * BN + crow(v, g);
        if (query < T && key < T && (!a.causal || key <= query)) ds[v] -= t.mean[v];
      }
    }
    if constexpr (DSUM) {
      f16v tf[D / 32];
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) tf[nb] = zero16();
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const Split8 ps = split8(p + 8 * b);
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) tf[nb] = mfma_split<NS>(ps, load_bt<D, NS>(sm.dOT, b, 32 * nb + c), tf[nb]);
      }
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) { dvd[nb][v] += (double)tf[nb][v]; tf[nb][v] = 0.f; }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const Split8 dss = split8(ds + 8 * b);
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) tf[nb] = mfma_split<NS>(dss, load_bt<D, NS>(sm.QT, b, 32 * nb + c), tf[nb]);
      }
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) dkd[nb][v] += (double)tf[nb][v];
      return;
    }
    // at D = 128 under P1 each query tile's products go into a fresh accumulator that joins the
    // float running sums once per tile
    constexpr bool FRESH = D == 128;
    f16v tv[FRESH ? D / 32 : 1], tk[FRESH ? D / 32 : 1];
    if (FRESH) {
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) { tv[nb] = zero16(); tk[nb] = zero16(); }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const Split8 ps = split8(p + 8 * b), dss = split8(ds + 8 * b);
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) {
        if (FRESH) {
          tv[nb] = mfma_split<NS>(ps, load_bt<D, NS>(sm.dOT, b, 32 * nb + c), tv[nb]);
          tk[nb] = mfma_split<NS>(dss, load_bt<D, NS>(sm.QT, b, 32 * nb + c), tk[nb]);
        } else {
          dv[nb] = mfma_split<NS>(ps, load_bt<D, NS>(sm.dOT, b, 32 * nb + c), dv[nb]);
          dk[nb] = mfma_split<NS>(dss, load_bt<D, NS>(sm.QT, b, 32 * nb + c), dk[nb]);
        }
      }
    }
    if (FRESH) {
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) { dv[nb] += tv[nb]; dk[nb] += tk[nb]; }
    }
  };
  if (qt_first < nt) {
    qr.load(Qp, qt_first * BN, T);
    dr.load(dOp, qt_first * BN, T);
    if (active(qt_first)) kv_load<P1, PC>(t0, a, tbase, head, qt_first, ktw);
  }
  for (int qt = qt_first; qt < nt; qt += 2) {
    stage(qt);
    if (qt + 1 < nt && active(qt + 1)) kv_load<P1, PC>(t1, a, tbase, head, qt + 1, ktw);
    if (active(qt)) contract(t0, qt);
    if (qt + 1 >= nt) break;
    stage(qt + 1);
    if (qt + 2 < nt && active(qt + 2)) kv_load<P1, PC>(t0, a, tbase, head, qt + 2, ktw);
    if (active(qt + 1)) contract(t1, qt + 1);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int key = kw0 + crow(v, g);
    if (key < T) {
      float* pk = a.dk + hb + (size_t)key * D + c;
      float* pv = a.dv + hb + (size_t)key * D + c;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) {
        if constexpr (DSUM) {
          pk[32 * nb] = (float)(dkd[nb][v] * a.scale);
          pv[32 * nb] = (float)dvd[nb][v];
        } else {
          pk[32 * nb] = dk[nb][v] * a.scale;
          pv[32 * nb] = dv[nb][v];
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------- launchers
#if KIA_CAL == 0
template <int D, typename TIn>
static hipError_t dkdv_go(const Problem& p, const BwdArgs& a, hipStream_t s) {
  const int nkt = (p.T + KV_BN - 1) / KV_BN;
  const dim3 grid(p.nheads * nkt), block(KV_NT);
  if (a.pc && BN * (p.K + 2) <= KV_NT) {
    if (a.p1) hipLaunchKernelGGL((dkdv_kernel<D, TIn, true, true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((dkdv_kernel<D, TIn, false, true, true>), grid, block, 0, s, a);
  } else if (a.pc) {
    if (a.p1) hipLaunchKernelGGL((dkdv_kernel<D, TIn, true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((dkdv_kernel<D, TIn, false, true>), grid, block, 0, s, a);
  } else {
    if (a.p1) hipLaunchKernelGGL((dkdv_kernel<D, TIn, true, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((dkdv_kernel<D, TIn, false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}
hipError_t launch_dkdv(const Problem& p, const BwdArgs& a, hipStream_t s) {
  if (p.D == 128) return p.bf16 ? dkdv_go<128, uint16_t>(p, a, s) : dkdv_go<128, float>(p, a, s);
  return p.bf16 ? dkdv_go<64, uint16_t>(p, a, s) : dkdv_go<64, float>(p, a, s);
}
#endif
template <int D, int CAL, int MODE, int GK, typename TIn>
static hipError_t dq_go(const Problem& p, const BwdArgs& a, hipStream_t s) {
  const int nqt = (p.T + DQ_BM - 1) / DQ_BM;
  const size_t smem = dq_smem_bytes<D, CAL, MODE, TIn>(p.K, p.lres);
  if constexpr (is_binmean(MODE)) {
    if (p.K < BINM_SMALLB) {
      hipLaunchKernelGGL((dq_kernel<D, CAL, MODE, GK, TIn, BINM_SMALLB>), dim3(p.nheads * nqt), dim3(NT), smem, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((dq_kernel<D, CAL, MODE, GK, TIn>), dim3(p.nheads * nqt), dim3(NT), smem, s, a);
  return hipGetLastError();
}
template <int D, int CAL, int MODE, int GK>
static hipError_t dq_dt(const Problem& p, const BwdArgs& a, hipStream_t s) {
  return p.bf16 ? dq_go<D, CAL, MODE, GK, uint16_t>(p, a, s) : dq_go<D, CAL, MODE, GK, float>(p, a, s);
}
template <int D, int CAL, int MODE>
static hipError_t dq_gk(const Problem& p, const BwdArgs& a, hipStream_t s) {
  switch (p.gk) {
    case GK_SUMS: return dq_dt<D, CAL, MODE, GK_SUMS>(p, a, s);
    case GK_DETACHED: return dq_dt<D, CAL, MODE, GK_DETACHED>(p, a, s);
    default: return dq_dt<D, CAL, MODE, GK_P1>(p, a, s);
  }
}
template <int D, int CAL>
static hipError_t dq_md(const Problem& p, const BwdArgs& a, hipStream_t s) {
  if constexpr (CAL == EXPB) {
    if (p.mode == EXPF8) return dq_gk<D, CAL, EXPF8>(p, a, s);
    return p.mode == EXPBF ? dq_gk<D, CAL, EXPBF>(p, a, s) : dq_gk<D, CAL, EXP32>(p, a, s);
  } else {
    switch (p.mode) {
      case LERP: return dq_gk<D, CAL, LERP>(p, a, s);
      case NEAREST_W: return dq_gk<D, CAL, NEAREST_W>(p, a, s);
      case NEAREST_P: return dq_gk<D, CAL, NEAREST_P>(p, a, s);
      default:
        // bin mean and the hybrid: no extremum terms (their values do not depend on the
        // extrema), so only the detached and P1 kernels
        if constexpr (CAL == MINMAX || CAL == FWM) {
          if (p.mode == BINM)
            return p.gk == GK_P1 ? dq_dt<D, CAL, BINM, GK_P1>(p, a, s) : dq_dt<D, CAL, BINM, GK_DETACHED>(p, a, s);
          return p.gk == GK_P1 ? dq_dt<D, CAL, NEARB, GK_P1>(p, a, s) : dq_dt<D, CAL, NEARB, GK_DETACHED>(p, a, s);
        } else {
          return hipErrorInvalidValue;
        }
    }
  }
}
template <>
hipError_t dq_cal<KIA_CAL>(const Problem& p, const BwdArgs& a, hipStream_t s) {
  return p.D == 128 ? dq_md<128, KIA_CAL>(p, a, s) : dq_md<64, KIA_CAL>(p, a, s);
}

}  // namespace kia
