// Internal interface between the C ABI (kia_api.hip) and the kernel launchers.  The forward and
// dq kernels are compiled once per calibration (kia_fwd.hip, kia_bwd.hip built with KIA_CAL = 0..3),
// each build supplying that calibration's specializations declared below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kia {

// MinMax, and FWM under its three tail policies: keys below the window weigh 0 (FWM), sit on
// the window edge with weight e^{-tau} and no slope (FWM_FLOOR), or stay on the grid continued
// below -tau (FWM_RES)
// EXPB: the exponential baselines (no grid: the row maximum alone shifts the scores)
enum Calib { MINMAX = 0, FWM = 1, FWM_FLOOR = 2, FWM_RES = 3, EXPB = 4 };
constexpr int NCALIB = 5;
// grid levels below the window held in the FWM_RES table (lower ones are computed on the fly)
constexpr int LRES_MAX = 1024;
// reconstruction and surrogate: LERP; Nearest with the Weight-STE point (P^N, W^N);
// Nearest with the Prob-STE point (P^L, W^L)
enum Mode { LERP = 0, NEAREST_W = 1, NEAREST_P = 2,
            // under EXPB: softmax, BF16-exp, FP8-rounded exp
            EXP32 = 3, EXPBF = 4, EXPF8 = 5,
            // bin mean (each Nearest bin weighs the mean of e^z over its members), and the strict
            // Nearest forward with the bin-mean backward (its forward runs as NEAREST_W)
            BINM = 6, NEARB = 7 };
constexpr bool is_nearest(int mode) {
  return mode == NEAREST_W || mode == NEAREST_P || mode == BINM || mode == NEARB;
}
constexpr bool is_binmean(int mode) { return mode == BINM || mode == NEARB; }
// The forward's normalized weight P reaches the dkdv kernel as a float per element, or, where
// every P of a row is one of K + 1 table values times 1/W (the Nearest forward, bin mean and the
// hybrid, under MinMax or FWM with a zero or floored tail), as a one-byte table index per element
// (K + 1: P = 0) beside each row's table of the K + 2 values.
constexpr bool p_coded(int calib, int mode) {
  return is_nearest(mode) && (calib == MINMAX || calib == FWM || calib == FWM_FLOOR);
}
// bins of the bin-mean modes: at most 9 (K <= 8), kept per lane in registers
constexpr int BINM_MAXB = 9;
// bins held when K <= 4 (the bin-mean kernels are also built for this count: fewer registers and
// per-key compares); LDS layouts keep the BINM_MAXB stride
constexpr int BINM_SMALLB = 5;
// backward kernels by gradient mode: the calibration sums (full, max_only, min_only), the
// detached extrema, or the detached gradient projected onto zero-sum rows (P1)
enum GradKind { GK_SUMS = 0, GK_DETACHED = 1, GK_P1 = 2 };

// Per-row record written by the forward and read by the backward (struct of arrays).
struct RowRec {
  float* M;
  float* m;
  int32_t* amax;
  int32_t* amin;
  int32_t* nA;
  int32_t* nC;
  float* WN;
  float* WL;
  float* E;   // the rigorous error bound of the row's stored scores (pass 1 for pass 2)
  float* OL;  // [N, D]: Nearest + Prob-STE O^L, BF16-exp O's residual (else nullptr)
  float* S;   // stored score tiles: per head, tiles_per_head tiles of 1024 floats
  int nt;     // number of 32-row tiles along T
  size_t tiles_per_head;
};

struct Problem {
  int nheads;   // B * H
  int T, D, K;
  int causal;
  float tau;
  double scale;
  int calib, mode, bf16;  // mode: LERP / NEAREST_W / NEAREST_P
  int gk;                 // GradKind
  int keepM, keepm;       // GK_SUMS: which extremum terms are injected (max_only / min_only drop one)
  int lres;               // FWM_RES: grid levels below the window in the table (0 otherwise)
  int res_far;            // FWM_RES: the table stops above b = -104 (lres hit LRES_MAX)
};

struct FwdArgs {
  int nheads;
  const void* q;
  const void* k;
  const void* v;
  float* o;
  RowRec rec;
  int T, K, causal;
  float tau;
  double scale;  // score scale, applied in double to the exact scores
  int lres;      // FWM_RES: grid levels below the window in the table
  int res_far;   // FWM_RES: keys below the table need computed grid values
  int phase;     // 0: the whole forward; 1: pass 1 and the exact extrema; 2: the rest
};

struct BwdArgs {
  int nheads;
  const void* q;
  const void* k;
  const void* v;
  const float* o;
  const void* dO;
  RowRec rec;  // read only
  float* dq;
  float* dk;
  float* dv;
  float* pt;     // key-major tiles of the forward's P, written by the dq kernel
  uint8_t* pcode;  // the same tiles as table indices, one byte per element (pc: p_coded)
  float* ptab;     // pc: per row, the K + 2 values of P by index (the last is 0)
  int pc;
  float* dst;    // key-major tiles of dS (extremum terms included), written by the dq kernel
  float* rowmean;  // P1: per row, the mean of the detached dS over the visible keys (dq writes it)
  int T, K, causal;
  float tau, scale;
  int keepM, keepm;  // GK_SUMS: inject the maximum's / minimum's term
  int p1;            // dkdv: subtract rowmean from the visible dS elements
  int lres;          // FWM_RES: grid levels below the window in the table
  int res_far;       // FWM_RES: keys below the table need computed grid values
};

// The one-pass exponential baselines (kia_flash.hip): per row the shift M of the scores and the
// weight sum W the forward ends with, and D_i = dO_i . O_i, which the dq kernel writes for dkdv.
struct FlashArgs {
  int nheads;
  const void* q;
  const void* k;
  const void* v;
  const void* dO;
  float* o;        // forward: written; backward: read
  float* rowM;
  float* rowW;
  float* rowD;
  float* dq;
  float* dk;
  float* dv;
  int T, causal;
  float scale;
  double scale_d;  // the same scale in double, for exact scores
};

struct BinsArgs {
  RowRec rec;
  uint8_t* bins;
  int T, K, causal;
  float tau;
};

// per-calibration launchers, one specialization per build of kia_fwd.hip / kia_bwd.hip
template <int CAL> hipError_t forward_cal(const Problem& p, const FwdArgs& a, hipStream_t s);
template <int CAL> hipError_t bins_cal(const Problem& p, const BinsArgs& a, hipStream_t s);
template <int CAL> hipError_t dq_cal(const Problem& p, const BwdArgs& a, hipStream_t s);
#define KIA_DECLARE_CAL(C)                                                                   \
  template <> hipError_t forward_cal<C>(const Problem& p, const FwdArgs& a, hipStream_t s); \
  template <> hipError_t bins_cal<C>(const Problem& p, const BinsArgs& a, hipStream_t s);   \
  template <> hipError_t dq_cal<C>(const Problem& p, const BwdArgs& a, hipStream_t s);
KIA_DECLARE_CAL(MINMAX)
KIA_DECLARE_CAL(FWM)
KIA_DECLARE_CAL(FWM_FLOOR)
KIA_DECLARE_CAL(FWM_RES)
KIA_DECLARE_CAL(EXPB)
#undef KIA_DECLARE_CAL
// the dK, dV kernel (independent of the calibration; built with KIA_CAL = 0)
hipError_t launch_dkdv(const Problem& p, const BwdArgs& a, hipStream_t s);

hipError_t launch_flash_forward(const Problem& p, const FlashArgs& a, hipStream_t s);
hipError_t launch_flash_backward(const Problem& p, const FlashArgs& a, hipStream_t s);

inline hipError_t launch_forward(const Problem& p, const FwdArgs& a, hipStream_t s) {
  switch (p.calib) {
    case MINMAX: return forward_cal<MINMAX>(p, a, s);
    case FWM: return forward_cal<FWM>(p, a, s);
    case FWM_FLOOR: return forward_cal<FWM_FLOOR>(p, a, s);
    case FWM_RES: return forward_cal<FWM_RES>(p, a, s);
    default: return forward_cal<EXPB>(p, a, s);
  }
}
// stages: bit 0 = dq kernel (dQ and the P, dS tiles), bit 1 = dkdv kernel (dK, dV)
inline hipError_t launch_backward(const Problem& p, const BwdArgs& a, hipStream_t s, int stages) {
  if (stages & 1) {
    hipError_t e;
    switch (p.calib) {
      case MINMAX: e = dq_cal<MINMAX>(p, a, s); break;
      case FWM: e = dq_cal<FWM>(p, a, s); break;
      case FWM_FLOOR: e = dq_cal<FWM_FLOOR>(p, a, s); break;
      case FWM_RES: e = dq_cal<FWM_RES>(p, a, s); break;
      default: e = dq_cal<EXPB>(p, a, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return (stages & 2) ? launch_dkdv(p, a, s) : hipSuccess;
}
inline hipError_t launch_bins(const Problem& p, const BinsArgs& a, hipStream_t s) {
  switch (p.calib) {
    case MINMAX: return bins_cal<MINMAX>(p, a, s);
    case FWM: return bins_cal<FWM>(p, a, s);
    case FWM_FLOOR: return bins_cal<FWM_FLOOR>(p, a, s);
    case FWM_RES: return bins_cal<FWM_RES>(p, a, s);
    default: return bins_cal<EXPB>(p, a, s);
  }
}

}  // namespace kia
