// One-pass (online-rescale) exact softmax attention for gfx950 (CDNA4): the same-hardware speed
// reference for the K-interval operator.
//
// "Pretraining Transformers with Quantized Softmax in Attention", App. B "Softmax": the weights are
// e^{s - M} over their row sum.  The exponential is shift-invariant, so any shift gives the same
// probabilities: a row need not know its maximum before its first weight, and the forward sweeps
// the keys once, keeping a running maximum m, the running weight sum l and the running output,
// both rescaled by e^{m_old - m_new} when m grows.  Nothing of size T x T is stored: the backward
// recomputes the scores tile by tile from Q, K and the row's final (M, W).
//
//   forward     32 query rows per workgroup; its FLW waves split the key tiles (wave w takes every
//               FLW-th) and each keeps its own (m, l, O); they meet in LDS at the end.  Scores are
//               bf16 slice products on the matrix pipe (K^T Q as in the K-interval forward), and
//               O is accumulated transposed, O^T += V^T P^T, so that each lane's 16 accumulator
//               elements belong to its own query row: the rescale is one factor per lane.
//   dq          64 query rows per workgroup (two waves): per key tile S and dP = dO V^T from the
//               staged K and V rows, P = e^{s - M} / W, dS = P (dP - D_i), dQ += dS K.  Writes
//               D_i = dO_i . O_i for dkdv.
//   dkdv        128 keys per workgroup (four waves of 32): per query tile S and dP again from the
//               staged Q and dO rows against the wave's own K and V rows (kept in registers),
//               then dV += P^T dO and dK += dS^T Q.
// The calibration term of the row maximum is zero for softmax (its weights do not depend on the
// shift), so the backward has none.  No atomics: every output element has one writer.
#include "kia_device.hpp"
#include "kia_launch.hpp"

#include <climits>

namespace kia {

constexpr int FLW = 2;             // forward waves per workgroup
constexpr int FL_NT = 64 * FLW;
constexpr int FQ_NT = 128;          // dq: two waves, 64 query rows
constexpr int FQ_BM = 64;
constexpr int FK_NT = 256;          // dkdv: four waves, 128 keys
constexpr int FK_BN = 128;
// A weight that can reach 1/16 of its row's probability (with room for the faster score's error)
// is taken again on the exact score: such a key passes any ulp of its score's error into D_i and
// into every score gradient of the row.
constexpr float HEAVY_P = (1.0f / 16.0f) / (1.0f + 1e-3f);
// The same bound on a shifted score: P <= e^{s - m} for any running maximum m <= M (every weight
// sum is at least 1), so a key more than ln 16 (with the margin) below the running maximum is
// never heavy.
constexpr float LN16M = 2.7736f;
constexpr int FLH = 4;  // forward: candidate heavy keys tracked per lane

// ================================================================================ forward
template <int D> constexpr int fl_ost() { return D + 4; }  // row stride of the O tile written out
template <int D, int NS>
constexpr int fl_wave_bytes() {  // per wave: V^T slices of its key tile, at the end its partial O
  return NS * D * TP * 2 > 32 * fl_ost<D>() * 4 ? NS * D * TP * 2 : 32 * fl_ost<D>() * 4;
}
template <int D, int NS>
struct FlFwdSmem {
  __align__(16) unsigned char wave[FLW][fl_wave_bytes<D, NS>()];
  float m[FLW][32], l[FLW][32];
};

template <int D, typename TIn>
__global__ __launch_bounds__(FL_NT) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void flash_fwd_kernel(FlashArgs a) {
  constexpr int NS = nslices<TIn>();
  __shared__ FlFwdSmem<D, NS> sm;
  const int w = wave_id(), l = threadIdx.x & 63, g = l >> 5, c = l & 31;
  const int T = a.T, nt = (T + 31) / 32;
  int head, rank;
  block_work(a.nheads, head, rank);
  const int qt = a.causal ? nt - 1 - rank : rank;  // rank 0: the latest query tile, the most keys
  const size_t hb = (size_t)head * T * D;
  const TIn* Kp = reinterpret_cast<const TIn*>(a.k) + hb;
  const TIn* Vp = reinterpret_cast<const TIn*>(a.v) + hb;
  const int q0 = qt * 32, qi = q0 + c;
  const bool qvalid = qi < T;
  const int ntiles = a.causal ? qt + 1 : nt;
  __bf16* VT = reinterpret_cast<__bf16*>(sm.wave[w]);

  // K rows of the wave's current tile: reloaded with the next tile's as soon as the score products
  // have read them, so that the load overlaps the tile's weights and P V
  RowOp<D, TIn> kr;
  if (w < ntiles) kr.load(Kp, w * 32 + c, T);
  Split8 qs[D / 16];
  {
    RowOp<D, TIn> qr;
    qr.load(reinterpret_cast<const TIn*>(a.q) + hb, qi, T);
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) qs[kb] = qr.split(kb);
  }
  PairRegs<D, TIn, 64> vr;  // V rows of the tile, loaded at its start and staged after its scores

  const TIn* qrow = reinterpret_cast<const TIn*>(a.q) + hb + (size_t)(qvalid ? qi : 0) * D;
  float mrun = -INFINITY, lsum = 0.f;  // the row's running maximum, this lane's running weight sum
  // the lane's FLH largest fast scores within ln 16 of the running maximum (the only keys that can
  // end up heavy), and the smallest of them
  float cv[FLH];
  int ck[FLH];
#pragma unroll
  for (int i = 0; i < FLH; ++i) { cv[i] = -INFINITY; ck[i] = 0; }
  float cmin = -INFINITY;
  f16v o[D / 32];                      // O^T: element v of block nb is column 32 nb + crow(v, g) of row c
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) o[nb] = zero16();

  for (int kt = w; kt < ntiles; kt += FLW) {
    const int k0 = kt * 32;
    vr.load(Vp, k0, T);
    // scores S^T = K Q^T as bf16 slice products (the smaller products apart from h h')
    f16v acc = zero16(), asm_ = zero16();
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
    }
    if (NS == 3) acc += asm_;
    if (kt + FLW < ntiles) kr.load(Kp, k0 + FLW * 32 + c, T);
    vr.template store_t<NS>(VT);
    wave_lds_sync();
    const bool full = k0 + 32 <= T && q0 + 32 <= T && (!a.causal || kt < qt);
    float s[16], tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = k0 + crow(v, g);
      const bool ok = full || (qvalid & (key < T) & (!a.causal | (key <= qi)));
      s[v] = ok ? acc[v] * a.scale : -INFINITY;
      tmax = fmaxf(tmax, s[v]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mnew = fmaxf(mrun, tmax);
    {
      const float thr = fmaxf(cmin, mnew - LN16M);
      uint32_t ins = 0u;
#pragma unroll
      for (int v = 0; v < 16; ++v) ins |= s[v] > thr ? 1u << v : 0u;
      while (ins) {  // divergent, rare once the row's largest scores have been seen
        const int v = __builtin_ctz(ins);
        ins &= ins - 1u;
        float x = s[0];
#pragma unroll
        for (int u = 1; u < 16; ++u) x = u == v ? s[u] : x;
        if (x > cmin) {
          bool done = false;
#pragma unroll
          for (int i = 0; i < FLH; ++i) {
            const bool here = !done && cv[i] == cmin;
            cv[i] = here ? x : cv[i];
            ck[i] = here ? k0 + crow(v, g) : ck[i];
            done |= here;
          }
          cmin = cv[0];
#pragma unroll
          for (int i = 1; i < FLH; ++i) cmin = fminf(cmin, cv[i]);
        }
      }
    }
    // rescale of what the row has so far (0 before its first visible key; a row that has seen no
    // visible key yet keeps m = -inf and weighs nothing)
    const bool none = mnew == -INFINITY;
    const float alpha = none ? 1.f : __expf(mrun - mnew);
    float p[16], ts = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      p[v] = none ? 0.f : __expf(s[v] - mnew);
      ts += p[v];
    }
    lsum = fmaf(lsum, alpha, ts);
    mrun = mnew;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) o[nb] *= alpha;
    // O^T += V^T P^T: A = V^T (rows d = 32 nb + c of the staged tile), B = P^T (column: query c)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const Split8 pb = split8(p + 8 * b);
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) o[nb] = mfma_split<3, NS>(load_bt<D, NS>(VT, b, 32 * nb + c), pb, o[nb]);
    }
    wave_lds_sync();  // this tile's V^T reads come before the next tile's staging
  }

  // ---- heavy keys.  With the row's (M, W) known, a key whose weight reaches 1/16 of W is taken
  // again on its exact score: its weight change goes into this wave's l and O (relative to the
  // wave's own maximum).  Every such key is in its lane's list unless the list's smallest entry is
  // itself above the threshold (a key may have been left out): that wave sweeps its tiles again.
  {
    const float lrow = lsum + __shfl_xor(lsum, 32);
    if (g == 0) {
      sm.m[w][c] = mrun;
      sm.l[w][c] = lrow;
    }
    __syncthreads();
    float Mr = sm.m[0][c];
#pragma unroll
    for (int u = 1; u < FLW; ++u) Mr = fmaxf(Mr, sm.m[u][c]);
    float Wr = 0.f;
#pragma unroll
    for (int u = 0; u < FLW; ++u) Wr += sm.m[u][c] == -INFINITY ? 0.f : sm.l[u][c] * __expf(sm.m[u][c] - Mr);
    const float sthr = qvalid && Mr > -INFINITY ? Mr + __logf(Wr * (1.0f / 16.0f)) - 1e-3f : INFINITY;
    const bool incomplete = cmin >= sthr;
    // one key's change (this lane's or its partner's, same row) into this lane's columns of O
    auto apply = [&](int key, float dw) {
      const TIn* vrow = Vp + (size_t)key * D;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[nb][v] = fmaf(dw, Ld<TIn>::one(vrow + 32 * nb + crow(v, g)), o[nb][v]);
    };
    auto change = [&](int key, float sfast) {  // the weight change of a key retaken on its exact score
      const float xe = exact_score<D, TIn, 2>(qrow, Kp + (size_t)key * D, a.scale_d);
      return __expf(xe - mrun) - __expf(sfast - mrun);
    };
#pragma unroll
    for (int i = 0; i < FLH; ++i) {
      const bool heavy = !incomplete && cv[i] >= sthr;
      const float dw = heavy ? change(ck[i], cv[i]) : 0.f;
      lsum += dw;
      const float pdw = __shfl_xor(dw, 32);
      const int pk = __shfl_xor(ck[i], 32);
      if (dw != 0.f) apply(ck[i], dw);
      if (pdw != 0.f) apply(pk, pdw);
    }
    if (__any(incomplete)) {
      // the wave's tiles again: fast scores as in the sweep, every key at or above the threshold
      // in an incomplete lane retaken
      for (int kt = w; kt < ntiles; kt += FLW) {
        const int k0 = kt * 32;
        kr.load(Kp, k0 + c, T);
        f16v acc = zero16(), asm_ = zero16();
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
        }
        if (NS == 3) acc += asm_;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = k0 + crow(v, g);
          const bool ok = qvalid & (key < T) & (!a.causal | (key <= qi));
          const float sf = acc[v] * a.scale;
          const bool heavy = incomplete && ok && sf >= sthr;
          const float dw = heavy ? change(key, sf) : 0.f;
          lsum += dw;
          const float pdw = __shfl_xor(dw, 32);
          if (dw != 0.f) apply(key, dw);
          if (pdw != 0.f) apply(k0 + crow(v, g ^ 1), pdw);
        }
      }
    }
    __syncthreads();  // the lists' row sums are read before the merge writes its own
  }

  // the waves' (m, l, O) meet in LDS; wave 0 combines them in wave order
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();
  float* part = reinterpret_cast<float*>(sm.wave[w]);  // this wave's V^T is no longer read
  if (w > 0) {
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) part[(nb * 16 + v) * 64 + l] = o[nb][v];
    if (g == 0) {
      sm.m[w][c] = mrun;
      sm.l[w][c] = lsum;
    }
  }
  __syncthreads();
  if (w != 0) return;
  float M = mrun;
#pragma unroll
  for (int u = 1; u < FLW; ++u) M = fmaxf(M, sm.m[u][c]);
  const float f0 = mrun == -INFINITY ? 0.f : __expf(mrun - M);
  float W = lsum * f0;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) o[nb] *= f0;
#pragma unroll
  for (int u = 1; u < FLW; ++u) {
    const float mu = sm.m[u][c];
    const float fu = mu == -INFINITY ? 0.f : __expf(mu - M);
    W = fmaf(sm.l[u][c], fu, W);
    const float* op = reinterpret_cast<const float*>(sm.wave[u]);
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[nb][v] = fmaf(op[(nb * 16 + v) * 64 + l], fu, o[nb][v]);
  }
  if (g == 0 && qvalid) {
    const size_t row = (size_t)head * T + qi;
    a.rowM[row] = M;
    a.rowW[row] = W;
  }
  // O = num / W, through LDS so that the rows are written in whole lines
  float* X = part;  // wave 0's region: [32][fl_ost] floats
  const float inv = 1.0f / W;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int v = 0; v < 16; ++v) X[c * fl_ost<D>() + 32 * nb + crow(v, g)] = o[nb][v] * inv;
  wave_lds_sync();
  for (int i = 4 * l; i < 32 * D; i += 4 * 64) {
    const int r = i / D, col = i % D;
    if (q0 + r < T)
      *reinterpret_cast<f4v*>(a.o + hb + (size_t)(q0 + r) * D + col) = *reinterpret_cast<const f4v*>(X + r * fl_ost<D>() + col);
  }
}

// ================================================================================ dq
template <int D, int NS>
struct FlDqSmem {
  __align__(16) __bf16 KT[NS * D * TP];       // K^T of the key tile (dQ += dS K)
  __align__(16) __bf16 KN[NS * 32 * np<D>()];  // K rows (S^T = K Q^T)
  __align__(16) __bf16 VN[NS * 32 * np<D>()];  // V rows (dP^T = V dO^T)
};

template <int D, typename TIn>
__global__ __launch_bounds__(FQ_NT) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void flash_dq_kernel(FlashArgs a) {
  constexpr int NS = nslices<TIn>();
  __shared__ FlDqSmem<D, NS> sm;
  const int w = wave_id(), l = threadIdx.x & 63, g = l >> 5, c = l & 31;
  const int T = a.T;
  const int nqt = (T + FQ_BM - 1) / FQ_BM;
  int head, rank;
  block_work(a.nheads, head, rank);
  const int qt = a.causal ? nqt - 1 - rank : rank;
  const size_t hb = (size_t)head * T * D;
  const TIn* Kp = reinterpret_cast<const TIn*>(a.k) + hb;
  const TIn* Vp = reinterpret_cast<const TIn*>(a.v) + hb;
  const TIn* dOp = reinterpret_cast<const TIn*>(a.dO) + hb;
  const int qb0 = qt * FQ_BM, qw0 = qb0 + 32 * w, qi = qw0 + c;
  const bool qvalid = qi < T;
  const int qlast_w = min(qw0 + 31, T - 1);
  const int kend = a.causal ? min(T, qb0 + FQ_BM) : T;
  const int ntiles = (kend + 31) / 32;
  const size_t row = (size_t)head * T + (qvalid ? qi : 0);
  auto active = [&](int kt) { return qw0 < T && (!a.causal || kt * 32 <= qlast_w); };

  const float M = a.rowM[row], invW = 1.0f / a.rowW[row];
  // D_i = dO_i . O_i in double (the two lanes of the row take half the columns each)
  float Di;
  {
    const int qc = qvalid ? qi : 0;
    double part = 0.0;
#pragma unroll
    for (int q = 0; q < D / 8; ++q) {
      const f4v x = *reinterpret_cast<const f4v*>(a.o + hb + (size_t)qc * D + 8 * q + 4 * g);
      const f4v y = Ld<TIn>::four(dOp + (size_t)qc * D + 8 * q + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) part = fma((double)y[e], (double)x[e], part);
    }
    if (!qvalid) part = 0.0;
    Di = (float)(part + __shfl_xor(part, 32));
    if (g == 0 && qvalid) a.rowD[row] = Di;
  }
  const TIn* qrow = reinterpret_cast<const TIn*>(a.q) + hb + (size_t)(qvalid ? qi : 0) * D;
  // the lane's Q and dO rows, B operands of S^T and dP^T: dO split once, Q kept as loaded and
  // split where used (registers)
  RowOp<D, TIn> qr;
  qr.load(reinterpret_cast<const TIn*>(a.q) + hb, qi, T);
  Split8 dos[D / 16];
  {
    RowOp<D, TIn> dr;
    dr.load(dOp, qi, T);
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) dos[kb] = dr.split(kb);
  }
  f16v dq[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) dq[nb] = zero16();

  // the next key tile is loaded while this one computes, except with fp32 rows (three slices),
  // whose operands leave no registers for it: there each tile is loaded at its start
  constexpr bool PREFETCH = NS == 1;
  PairRegs<D, TIn, FQ_NT> kt_r;  // K rows of the next key tile, staged transposed
  RowRegs<D, TIn, FQ_NT> kn_r, vn_r;  // K and V rows of the next key tile, staged in their own layout
  auto load_tile = [&](int k0) {
    kt_r.load(Kp, k0, T);
    kn_r.load(Kp, k0, T);
    vn_r.load(Vp, k0, T);
  };
  if (PREFETCH) load_tile(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * 32;
    if (!PREFETCH) load_tile(k0);
    __syncthreads();
    kt_r.template store_t<NS>(sm.KT);
    kn_r.template store<NS>(sm.KN);
    vn_r.template store<NS>(sm.VN);
    __syncthreads();
    if (PREFETCH && kt + 1 < ntiles) load_tile(k0 + 32);
    if (!active(kt)) continue;
    // S^T and dP^T: register v holds (query c, key k0 + crow(v, g))
    f16v sacc = zero16(), gacc = zero16();
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      sacc = mfma_split<NS, NS>(load_an<D, NS>(sm.KN, c, kb), qr.split(kb), sacc);
      gacc = mfma_split<NS, NS>(load_an<D, NS>(sm.VN, c, kb), dos[kb], gacc);
    }
    const int lim = (qvalid ? (a.causal ? min(qi, T - 1) : T - 1) : -1) - k0 - 4 * g;  // crow(v, 0) <= lim
    float p[16];
    uint32_t heavy = 0u;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      p[v] = crow(v, 0) <= lim ? __expf(sacc[v] * a.scale - M) * invW : 0.f;
      heavy |= p[v] >= HEAVY_P ? 1u << v : 0u;
    }
    while (__any(heavy != 0u)) {  // rare: at most 16 keys of a row
      if (heavy) {
        const int v = __builtin_ctz(heavy);
        heavy &= heavy - 1u;
        const float xe = exact_score<D, TIn, 2>(qrow, Kp + (size_t)(k0 + crow(v, g)) * D, a.scale_d);
        const float pe = __expf(xe - M) * invW;
#pragma unroll
        for (int u = 0; u < 16; ++u) p[u] = u == v ? pe : p[u];
      }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float ds[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) ds[j] = p[8 * b + j] * (gacc[8 * b + j] - Di);
      const Split8 dss = split8(ds);
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) dq[nb] = mfma_split<NS>(dss, load_bt<D, NS>(sm.KT, b, 32 * nb + c), dq[nb]);
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int qrow = qw0 + crow(v, g);
    if (qrow < T) {
      float* out = a.dq + hb + (size_t)qrow * D + c;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) out[32 * nb] = dq[nb][v] * a.scale;
    }
  }
}

// ================================================================================ dkdv
template <int D, int NS>
struct FlKvSmem {
  __bf16 QT[NS * D * TP];        // Q^T of the query tile (dK += dS^T Q)
  __bf16 dOT[NS * D * TP];       // dO^T (dV += P^T dO)
  __align__(16) __bf16 QN[NS * 32 * np<D>()];   // Q rows (S = Q K^T)
  __align__(16) __bf16 dON[NS * 32 * np<D>()];  // dO rows (dP = dO V^T)
  float rM[32], rW[32], rD[32];  // the query tile's rows: shift, weight sum, D_i
};

template <int D, typename TIn>
__global__ __launch_bounds__(FK_NT) __attribute__((amdgpu_waves_per_eu(1))) void flash_dkdv_kernel(FlashArgs a) {
  constexpr int NS = nslices<TIn>();
  __shared__ FlKvSmem<D, NS> sm;
  const int tid = threadIdx.x, w = wave_id(), l = tid & 63, g = l >> 5, c = l & 31;
  const int T = a.T, nt = (T + 31) / 32;
  int head, kt;
  block_work(a.nheads, head, kt);  // low key tiles see the most queries: heaviest first
  const size_t hb = (size_t)head * T * D;
  const TIn* Qp = reinterpret_cast<const TIn*>(a.q) + hb;
  const TIn* dOp = reinterpret_cast<const TIn*>(a.dO) + hb;
  const int kb0 = kt * FK_BN, kw0 = kb0 + 32 * w, key = kw0 + c;
  const int ktw = kw0 / 32;
  auto active = [&](int qt) { return kw0 < T && (!a.causal || ktw <= qt); };  // wave-uniform

  // the lane's K and V rows, the B operands of S and dP: kept as loaded and split where used
  RowOp<D, TIn> kown, vown;
  const TIn* Kp_own = reinterpret_cast<const TIn*>(a.k) + hb + (size_t)(key < T ? key : 0) * D;
  kown.load(reinterpret_cast<const TIn*>(a.k) + hb, key, T);
  vown.load(reinterpret_cast<const TIn*>(a.v) + hb, key, T);
  f16v dk[D / 32], dv[D / 32];
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb) { dk[nb] = zero16(); dv[nb] = zero16(); }

  const int qt_first = a.causal ? kb0 / 32 : 0;
  // the next query tile is loaded while this one computes, except with fp32 rows at D = 128, whose
  // own K and V rows leave no registers for it: there each tile is loaded at its start
  constexpr bool PREFETCH = !(D == 128 && NS == 3);
  PairRegs<D, TIn, FK_NT> qt_r, dt_r;  // the next query tile's Q and dO rows, staged transposed
  RowRegs<D, TIn, FK_NT> qn_r, dn_r;   // ... and in their own layout
  float st_r = 0.f;                     // thread t < 96: one of the next tile's row numbers
  auto load_tile = [&](int qt) {
    qt_r.load(Qp, qt * 32, T);
    dt_r.load(dOp, qt * 32, T);
    qn_r.load(Qp, qt * 32, T);
    dn_r.load(dOp, qt * 32, T);
    if (tid < 96) {
      const int r = qt * 32 + (tid & 31);
      const size_t at = (size_t)head * T + (r < T ? r : 0);
      st_r = tid < 32 ? a.rowM[at] : (tid < 64 ? a.rowW[at] : a.rowD[at]);
    }
  };
  if (PREFETCH && qt_first < nt) load_tile(qt_first);
  for (int qt = qt_first; qt < nt; ++qt) {
    const int q0 = qt * 32;
    if (!PREFETCH) load_tile(qt);
    __syncthreads();
    qt_r.template store_t<NS>(sm.QT);
    dt_r.template store_t<NS>(sm.dOT);
    qn_r.template store<NS>(sm.QN);
    dn_r.template store<NS>(sm.dON);
    if (tid < 32) sm.rM[tid] = st_r;
    else if (tid < 64) sm.rW[tid - 32] = st_r;
    else if (tid < 96) sm.rD[tid - 64] = st_r;
    __syncthreads();
    if (PREFETCH && qt + 1 < nt) load_tile(qt + 1);
    if (!active(qt)) continue;
    // S and dP: register v holds (query q0 + crow(v, g), key c of the wave's tile)
    f16v sacc = zero16(), gacc = zero16();
#pragma unroll
    for (int kb = 0; kb < D / 16; ++kb) {
      sacc = mfma_split<NS, NS>(load_an<D, NS>(sm.QN, c, kb), kown.split(kb), sacc);
      gacc = mfma_split<NS, NS>(load_an<D, NS>(sm.dON, c, kb), vown.split(kb), gacc);
    }
    float p[16], ds[16];
    uint32_t heavy = 0u;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = crow(v, g), query = q0 + r;
      const bool ok = query < T && key < T && (!a.causal || key <= query);
      p[v] = ok ? __expf(sacc[v] * a.scale - sm.rM[r]) / sm.rW[r] : 0.f;
      heavy |= p[v] >= HEAVY_P ? 1u << v : 0u;
    }
    while (__any(heavy != 0u)) {
      if (heavy) {
        const int v = __builtin_ctz(heavy);
        heavy &= heavy - 1u;
        const int r = crow(v, g);
        const float xe = exact_score<D, TIn, 2>(Qp + (size_t)(q0 + r) * D, Kp_own, a.scale_d);
        const float pe = __expf(xe - sm.rM[r]) / sm.rW[r];
#pragma unroll
        for (int u = 0; u < 16; ++u) p[u] = u == v ? pe : p[u];
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) ds[v] = p[v] * (gacc[v] - sm.rD[crow(v, g)]);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const Split8 ps = split8(p + 8 * b), dss = split8(ds + 8 * b);
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) {
        dv[nb] = mfma_split<NS>(ps, load_bt<D, NS>(sm.dOT, b, 32 * nb + c), dv[nb]);
        dk[nb] = mfma_split<NS>(dss, load_bt<D, NS>(sm.QT, b, 32 * nb + c), dk[nb]);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int kr = kw0 + crow(v, g);
    if (kr < T) {
      float* pk = a.dk + hb + (size_t)kr * D + c;
      float* pv = a.dv + hb + (size_t)kr * D + c;
#pragma unroll
      for (int nb = 0; nb < D / 32; ++nb) {
        pk[32 * nb] = dk[nb][v] * a.scale;
        pv[32 * nb] = dv[nb][v];
      }
    }
  }
}

// ================================================================================ launchers
template <int D, typename TIn>
static hipError_t flash_fwd_go(const Problem& p, const FlashArgs& a, hipStream_t s) {
  const int nqt = (p.T + 31) / 32;
  hipLaunchKernelGGL((flash_fwd_kernel<D, TIn>), dim3(p.nheads * nqt), dim3(FL_NT), 0, s, a);
  return hipGetLastError();
}
template <int D, typename TIn>
static hipError_t flash_bwd_go(const Problem& p, const FlashArgs& a, hipStream_t s) {
  const int nq = (p.T + FQ_BM - 1) / FQ_BM, nk = (p.T + FK_BN - 1) / FK_BN;
  hipLaunchKernelGGL((flash_dq_kernel<D, TIn>), dim3(p.nheads * nq), dim3(FQ_NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((flash_dkdv_kernel<D, TIn>), dim3(p.nheads * nk), dim3(FK_NT), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_flash_forward(const Problem& p, const FlashArgs& a, hipStream_t s) {
  if (p.D == 128) return p.bf16 ? flash_fwd_go<128, uint16_t>(p, a, s) : flash_fwd_go<128, float>(p, a, s);
  return p.bf16 ? flash_fwd_go<64, uint16_t>(p, a, s) : flash_fwd_go<64, float>(p, a, s);
}
hipError_t launch_flash_backward(const Problem& p, const FlashArgs& a, hipStream_t s) {
  if (p.D == 128) return p.bf16 ? flash_bwd_go<128, uint16_t>(p, a, s) : flash_bwd_go<128, float>(p, a, s);
  return p.bf16 ? flash_bwd_go<64, uint16_t>(p, a, s) : flash_bwd_go<64, float>(p, a, s);
}

}  // namespace kia
