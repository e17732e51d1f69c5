// Internal interface between the C ABI (kia_api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kia {

enum Calib { MINMAX = 0, FWM = 1 };
// reconstruction and surrogate: LERP; Nearest with the Weight-STE point (P^N, W^N);
// Nearest with the Prob-STE point (P^L, W^L)
enum Mode { LERP = 0, NEAREST_W = 1, NEAREST_P = 2 };
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
  float* OL;  // [N, D], Nearest + Prob-STE only (else nullptr)
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
  double scale;  // score scale, applied in double to the fp64 dot products
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
  float* dst;    // key-major tiles of dS (extremum terms included), written by the dq kernel
  float* rowmean;  // P1: per row, the mean of the detached dS over the visible keys (dq writes it)
  int T, K, causal;
  float tau, scale;
  int keepM, keepm;  // GK_SUMS: inject the maximum's / minimum's term
  int p1;            // dkdv: subtract rowmean from the visible dS elements
};

struct BinsArgs {
  RowRec rec;
  uint8_t* bins;
  int T, K, causal;
  float tau;
};

hipError_t launch_forward(const Problem& p, const FwdArgs& a, hipStream_t s);
// stages: bit 0 = dq kernel (dQ and the P, dS tiles), bit 1 = dkdv kernel (dK, dV)
hipError_t launch_backward(const Problem& p, const BwdArgs& a, hipStream_t s, int stages);
hipError_t launch_bins(const Problem& p, const BinsArgs& a, hipStream_t s);

}  // namespace kia
