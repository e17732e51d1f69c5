/*
 * kia.h -- C ABI of the K-interval attention library (libkia.so) for AMD
 * Instinct MI355X (gfx950).
 *
 * The operator is the one defined in "Pretraining Transformers with Quantized
 * Softmax in Attention" (Zhu, Hu, Kozlowski), §3 and App. A-C.  For one causal
 * row of scores s_j = scale * Q_i . K_j (j <= i), a per-row calibration places
 * K+1 grid values e^{b_r}:
 *   MinMax (§3 "Objects and calibration"): h = (M-m)/K, b_r = (1-r/K)(m-M),
 *     with the row maximum M and minimum m; rows with M - m <= 1e-12 use the
 *     safe width h = 1 (App. A "Edge cases and conventions");
 *   FWM: h = tau/K, b_r = -tau + r h, the score shifted by M is clipped to
 *     [-tau, 0] and keys below the window get weight 0.  Two other tail
 *     policies (kia_tail_t): floor (App. C.3 selection stages, App. D.4: z is
 *     clipped up to -tau, so such a key weighs e^{-tau} and has no score
 *     gradient) and resolved (App. D.4: the grid b_q = -tau + q h continues
 *     below -tau with negative indices q, so no key is truncated).
 * Each key's weight is rebuilt from the grid (§3 "Reconstruction"): LERP
 * interpolates between e^{b_r} and e^{b_{r+1}} at the key's local position t;
 * Nearest takes the grid value of index r + 1[t >= 1/2].  Weights are
 * normalized, P = w / sum(w), and O = P V.  The forward returns the hard value
 * P^N exactly for Nearest (App. C.2 (iii), strict forward).
 * The backward (App. B) applies the normalization Jacobian at the Weight-STE
 * point (P^N, W^N) or the Prob-STE point (P^L, W^L), the LERP secant slope
 * Delta_j = (e^{b_{r+1}} - e^{b_r})/h, and, in full mode, the calibration
 * gradient through the row extrema (split evenly among tied keys) that makes
 * every row's score gradient sum to zero.  Detached mode drops the extremum
 * terms (the legacy ablation of §5.1).  The range_grad ablations of §5.1 and
 * App. I: max_only / min_only keep only the maximum's / the minimum's term
 * (FWM has no minimum term: its max_only is full, its min_only detached); P1
 * (App. B "Detach") subtracts from each row of the detached score gradient its
 * mean over the row's visible keys.
 *
 * Conventions shared by every entry point:
 *  - Tensors Q, K, V, dO are [B, H, T, D], C-contiguous, in device memory, of
 *    the dtype given by params->dtype (KIA_F32 or KIA_BF16).  O, dQ, dK, dV are
 *    float32 [B, H, T, D] for every input dtype.
 *  - All buffers are owned and allocated by the caller; the library never
 *    allocates or frees device memory and keeps no state between calls.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *    the call returns after the launch, without synchronizing.
 *  - Arguments are checked before any launch; on failure nothing is enqueued,
 *    a negative status is returned and kia_last_error() describes it.
 *  - NaN and Inf inputs are not checked; they propagate.
 *  - Calls that share output or record buffers and overlap on different
 *    streams race; order them on one stream.
 */
#ifndef KIA_H
#define KIA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KIA_OK = 0,
  KIA_ERR_INVALID_ARG = -1, /* null pointer, bad size or enum value, tau <= 0 under FWM,
                               a tail policy other than zero under MinMax or an
                               exponential baseline */
  KIA_ERR_UNSUPPORTED = -2, /* valid but not built: D not in {64, 128}, K > 8 for bin mean */
  KIA_ERR_WORKSPACE = -3,   /* reserved: a buffer smaller than kia_workspace_size asks */
  KIA_ERR_HIP = -4          /* a HIP launch or runtime call failed */
} kia_status_t;

typedef enum { KIA_CALIB_MINMAX = 0, KIA_CALIB_FWM = 1 } kia_calib_t;
/* LERP and Nearest rebuild weights from the grid; SOFTMAX, EXP_BF16 and EXP_FP8 are the
   exponential baselines (App. B "Softmax", App. D.5): no grid, so calib, K, tau and ste are
   ignored (they are still checked) and tail must be ZERO:
     SOFTMAX   w = e^z, z = s - M;
     EXP_BF16  z rounded to bfloat16, e^(that) rounded to bfloat16; the backward carries the
               gradient through the bfloat16 weight in bfloat16 (dL/dw rounded to bfloat16,
               times the weight, rounded to bfloat16);
     EXP_FP8   e^z rounded to E4M3 (float8_e4m3fn), derivative e^z (the unrounded exponential);
   roundings to nearest, ties to even, of the exact values.  The row maximum's term
   -sum_j dL/dz_j goes to the arg-max key(s) in the full and max_only modes. */
/* BINMEAN (§5, App. I): each Nearest bin l = 0..K of the row's calibration weighs the mean of
   e^z over its members (bin mass conserved; keys below an FWM window belong to no bin); its
   backward is the exact derivative with the bins fixed: dL/ds_k = e^{z_k}/W^C (gbar_b(k) -
   sum_j P_j g_j), gbar_b the mean of dL/dP over bin b; the extrema add nothing.
   NEAREST_BINMEAN (App. I.3): the strict Nearest forward (P^N) with BINMEAN's backward.
   Both ignore ste, take the zero tail only and are built for K <= 8 (KIA_ERR_UNSUPPORTED
   above); full, detached, max_only and min_only give the same gradient, P1 projects it. */
typedef enum {
  KIA_RECON_LERP = 0,
  KIA_RECON_NEAREST = 1,
  KIA_RECON_SOFTMAX = 2,
  KIA_RECON_EXP_BF16 = 3,
  KIA_RECON_EXP_FP8 = 4,
  KIA_RECON_BINMEAN = 5,
  KIA_RECON_NEAREST_BINMEAN = 6
} kia_recon_t;
/* surrogate placement; ignored under LERP (both give the LERP Jacobian) */
typedef enum { KIA_STE_WEIGHT = 0, KIA_STE_PROB = 1 } kia_ste_t;
/* full calibration gradient, or one of the range_grad ablations */
typedef enum {
  KIA_GRAD_FULL = 0,
  KIA_GRAD_DETACHED = 1,
  KIA_GRAD_MAX_ONLY = 2, /* only the row maximum's calibration term */
  KIA_GRAD_MIN_ONLY = 3, /* only the row minimum's calibration term */
  KIA_GRAD_P1 = 4        /* detached, each row projected onto zero sum over its visible keys */
} kia_grad_t;
typedef enum { KIA_F32 = 0, KIA_BF16 = 1 } kia_dtype_t;
/* FWM treatment of keys below the window (z = s - M < -tau); MinMax takes ZERO */
typedef enum {
  KIA_TAIL_ZERO = 0,     /* weight 0 (the FWM operator of §3) */
  KIA_TAIL_FLOOR = 1,    /* z clipped to -tau: weight e^{-tau}, no score gradient */
  KIA_TAIL_RESOLVED = 2  /* grid continued below -tau: every key weighed on it */
} kia_tail_t;

typedef struct {
  int64_t B, H, T, D;   /* batch, heads, sequence length, head dim; T >= 1, D in {64, 128} */
  int32_t causal;       /* 1: query i sees keys j <= i; 0: every key */
  int32_t K;            /* number of intervals, 1..64 */
  float tau;            /* FWM window width in nats (> 0); ignored under MinMax */
  float scale;          /* score scale; 0 selects 1/sqrt(D) */
  int32_t calib;        /* kia_calib_t */
  int32_t recon;        /* kia_recon_t */
  int32_t ste;          /* kia_ste_t */
  int32_t grad;         /* kia_grad_t */
  int32_t dtype;        /* kia_dtype_t of Q, K, V and dO */
  int32_t tail;         /* kia_tail_t; must be KIA_TAIL_ZERO under MinMax */
} kia_params_t;

/*
 * Sizes of the two caller-owned buffers for `p` (host-only, no GPU needed).
 *  rowrec_bytes: the record written by kia_forward and read by kia_backward:
 *    per row the extrema, their first index and tie counts, W^N, W^L, for
 *    Nearest with Prob-STE the LERP output O^L, and the scores themselves.
 *    Layout (offsets are multiples of 256 bytes), N = B*H*T, nt = ceil(T/32):
 *      float M[N], m[N]; int32 amax[N], amin[N], nA[N], nC[N]; float WN[N], WL[N], E[N];
 *      (m, amin and nC belong to MinMax; under FWM m = M and amin = nC = 0; E: the
 *      rigorous bound on the error of each stored score of the row, below)
 *      float OL[N*D] (Nearest + Prob-STE: the output O^L; BF16-exp: the residual
 *        O - o of the double output whose float o is the kernel's output, and then WN
 *        holds W's residual, W = WL + WN; other modes: absent);
 *      float S[B*H][tiles][1024]: the scores s_ij = scale * Q_i . K_j as floats, in
 *        32 x 32 tiles (query tile, key tile); tiles = nt(nt+1)/2 when causal
 *        (key tile <= query tile), nt^2 otherwise.  About 2 T^2 bytes per head
 *        when causal.  Each is within a rigorous per-row bound of the exactly
 *        rounded score (exact products, double sum, one rounding), and equal to it
 *        wherever that bound could change an extremum or a bin decision, so every
 *        decision taken on S is the one the exactly rounded scores give.
 *  bwd_ws_bytes: scratch for kia_backward: two arrays of float tiles numbered
 *    like S, P[B*H][tiles][1024] (the forward's normalized weights: P^L for LERP,
 *    the hard P^N for Nearest) and dS[B*H][tiles][1024] (the unscaled score
 *    gradients, extremum terms included; under P1 the detached ones, before the
 *    projection), then float rowmean[N] (P1: each row's mean of dS over its
 *    visible keys), then float ptab[N][K+2].  Within a tile of S, P or dS, element
 *    (query row a, key column b of the tile) sits at float offset v*64 + a + 32*g,
 *    where b = 8*(v/4) + 4*g + v%4.
 *    Where every P of a row is one of K+1 table values times 1/W (recon Nearest,
 *    bin mean or the hybrid, with MinMax or with FWM and the zero or floored
 *    tail), the P array holds instead one byte per element, at byte offset
 *    (tile * 1024 + the element's offset above): the index j of its value
 *    ptab[row][j] (j = K+1, whose value is 0, for keys the query does not see
 *    and for FWM tail keys); the rest of the P array is unused.
 * Either output pointer may be NULL.  Returns KIA_ERR_INVALID_ARG or
 * KIA_ERR_UNSUPPORTED for parameters kia_forward would reject.
 */
kia_status_t kia_workspace_size(const kia_params_t* p, size_t* rowrec_bytes, size_t* bwd_ws_bytes);

/*
 * Forward pass (§3; strict hard forward of App. C.2 (iii) for Nearest).
 *  q, k, v: device, [B,H,T,D] of params->dtype.
 *  o:       device float32 [B,H,T,D], written.
 *  rowrec:  device, rowrec_bytes (kia_workspace_size), written; it must be
 *           passed unchanged to kia_backward with identical params.
 * Forwards under every kia_grad_t are bit-identical.
 */
kia_status_t kia_forward(const kia_params_t* p, const void* q, const void* k, const void* v,
                         float* o, void* rowrec, void* stream);

/*
 * The two halves of kia_forward as separate launches, for callers that time,
 * profile or schedule them apart (kia_forward runs both in one launch and writes
 * the same bits):
 *  kia_forward_scores  (first): the scores (stored in rowrec), the exact row
 *                      extrema, their first indices and tie counts, and the score
 *                      bounds E; o is not touched.
 *  kia_forward_weights (second): calibration, grid tables, reconstruction,
 *                      normalization and P V from what the first left in rowrec;
 *                      writes o and the rest of the record.
 * Same stream, same params, same rowrec, weights after scores.  Arguments as for
 * kia_forward.
 */
kia_status_t kia_forward_scores(const kia_params_t* p, const void* q, const void* k, const void* v, void* rowrec,
                                void* stream);
kia_status_t kia_forward_weights(const kia_params_t* p, const void* q, const void* k, const void* v, float* o,
                                 void* rowrec, void* stream);

/*
 * Backward pass (App. B): gradients of L = sum(dO * O) for the operator and
 * surrogate selected by params.
 *  q, k, v, d_o: device, [B,H,T,D] of params->dtype; d_o = dL/dO.
 *  o:       device float32, the output of kia_forward.
 *  rowrec:  the record written by kia_forward with the same params.
 *  dq, dk, dv: device float32 [B,H,T,D], written (not accumulated).
 *  workspace: device, bwd_ws_bytes (kia_workspace_size); contents on entry are ignored.
 * The backward reads the scores stored in rowrec; it does not recompute them.
 */
kia_status_t kia_backward(const kia_params_t* p, const void* q, const void* k, const void* v,
                          const float* o, const void* d_o, const void* rowrec,
                          float* dq, float* dk, float* dv, void* workspace, void* stream);

/*
 * The two stages of kia_backward, for callers that schedule or time them
 * separately; kia_backward runs exactly these two in this order.
 *  kia_backward_dq   (first): writes dq, and the P and dS tiles described under
 *                    kia_workspace_size into `workspace`.
 *  kia_backward_dkdv (second): reads `workspace` as kia_backward_dq left it and
 *                    writes dk, dv.  Both on the same stream, dkdv after dq.
 * Arguments as for kia_backward.
 */
kia_status_t kia_backward_dq(const kia_params_t* p, const void* q, const void* k, const void* v,
                             const float* o, const void* d_o, const void* rowrec, float* dq,
                             void* workspace, void* stream);
kia_status_t kia_backward_dkdv(const kia_params_t* p, const void* q, const void* k, const void* v,
                               const void* d_o, const void* rowrec, float* dk, float* dv,
                               void* workspace, void* stream);

/*
 * kia_backward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It allocates nothing: its workspace is a built-in
 * device array of KIA_NOALLOC_WS_BYTES per GPU, which each GPU the library runs
 * on holds until the process ends.
 *  Arguments as for kia_backward, without `workspace`.
 *  Returns KIA_ERR_WORKSPACE, launching nothing, when these params need more
 *  workspace (bwd_ws_bytes of kia_workspace_size) than the built-in array holds:
 *  call kia_backward with a workspace of your own instead.
 * Every call on one GPU uses that GPU's one array, which keeps what the last call
 * left there (nothing in it needs to start cleared: every element a call reads,
 * it wrote first).  Calls that overlap on one GPU (on different streams, or from
 * different host threads without ordering) race on it: serialize them.
 */
#define KIA_NOALLOC_WS_BYTES ((size_t)64 << 20)
kia_status_t kia_backward_noalloc(const kia_params_t* p, const void* q, const void* k, const void* v,
                                  const float* o, const void* d_o, const void* rowrec,
                                  float* dq, float* dk, float* dv, void* stream);

/*
 * One-pass exact softmax attention (App. B "Softmax"), FlashAttention-style: the
 * same-hardware speed reference for the K-interval operator.  The forward sweeps
 * the keys once with a running row maximum, rescaling the running weight sum and
 * output when it grows (the exponential is shift-invariant, so the probabilities
 * are those of the row maximum's shift); the backward recomputes the scores tile
 * by tile.  Memory beyond the inputs and outputs is O(T): nothing T x T is stored.
 *  p: params->recon must be KIA_RECON_SOFTMAX (KIA_ERR_UNSUPPORTED otherwise);
 *     calib, K, tau, ste, grad and tail are checked as for kia_forward and do not
 *     change the result (softmax's row-maximum term is zero).
 *  q, k, v, d_o: device, [B,H,T,D] of params->dtype.  o: device float32 [B,H,T,D].
 *  rowstats: device float[3*B*H*T], caller-owned: per row the shift M and weight
 *     sum W the forward ends with (written by kia_flash_forward, read by
 *     kia_flash_backward), then D_i = dO_i . O_i (written and read by
 *     kia_flash_backward).
 *  dq, dk, dv: device float32 [B,H,T,D], written.
 * The forward's o and rowstats must be passed unchanged to the backward.
 */
kia_status_t kia_flash_forward(const kia_params_t* p, const void* q, const void* k, const void* v, float* o,
                               float* rowstats, void* stream);
kia_status_t kia_flash_backward(const kia_params_t* p, const void* q, const void* k, const void* v,
                                const float* o, const void* d_o, float* rowstats, float* dq, float* dk,
                                float* dv, void* stream);

/*
 * Test hook: the reconstruction decision of every (query, key) pair as the
 * kernels take it, for bit-exact comparison of bin decisions.
 *  rowrec: the record written by kia_forward with the same params (its stored
 *        scores and row extrema decide the bins).
 *  bins: device uint8 [B,H,T,T]: for visible keys the Nearest index l in 0..K
 *        (recon = Nearest and the bin-mean modes) or the interval index r in 0..K-1
 *        (recon = LERP);
 *        on the resolved FWM grid (indices may be negative) the index + 64,
 *        with indices below -64 all given 0; 254 for FWM tail keys (zero and
 *        floor policies); 255 for keys the query does not see.  The exponential
 *        baselines give the E4M3 byte of the weight (EXP_FP8), the low byte of
 *        the bfloat16 weight (EXP_BF16) or 0 (SOFTMAX) for visible keys.
 * Costs O(B*H*T*T) bytes; meant for small T.
 */
kia_status_t kia_debug_bins(const kia_params_t* p, const void* rowrec, uint8_t* bins, void* stream);

/* Static string naming a status code: a kia_status_t value, or any other int
 * ("KIA_ERR_UNKNOWN"). */
const char* kia_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* kia_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KIA_H */
