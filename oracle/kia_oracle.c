/*
 * kia_oracle.c -- the oracle for K-interval attention: a plain, slow,
 * double-precision CPU implementation of the forward and backward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this code; the product path
 * (the HIP library and its Python binding) never does, and shares no code,
 * header, table or helper with it.
 *
 * Source of every step: "Pretraining Transformers with Quantized Softmax in
 * Attention" (Zhu, Hu, Kozlowski), §3 "Objects and calibration" and
 * "Reconstruction", App. A "Edge cases and conventions", App. B (normalization
 * Jacobian, LERP own-score slope, full calibration gradient (MinMax) = eq. (1),
 * detach (legacy) and its P1 projection, Weight-STE, Prob-STE, FWM, Softmax),
 * App. C.2 (iii) (strict hard forward), App. C.3 and D.4 (FWM tail policies),
 * App. D.5 (reduced-precision exponentials), §5 and App. I (bin mean; the
 * single-channel ablations max_only / min_only).
 *
 * Layout of this file:
 *  1. the method, one function per step in the pages' order and notation:
 *       ko_extrema     row extrema and the keys attaining them      (App. A)
 *       ko_calibrate   interval width and grid values e^{b_q}        (§3)
 *       ko_decide      interval index r, local position t, Nearest
 *                      index l, FWM tail flag of one key             (§3)
 *       ko_finish_grid reconstruction -> normalization -> P; backward:
 *                      gamma -> Delta -> dS -> calibration terms    (§3, App. B, C.2)
 *       ko_exp_*       the exponential baselines                     (App. B, D.5)
 *  2. the checking apparatus, used only by tests and never by the method
 *     functions: flags (positions whose decision the fp32 representation of
 *     the scores, or the guard, leaves open), flips (the other valid decision
 *     at a flagged position), bins (a map of the decisions);
 *  3. the drivers: ko_row (one row) and ko_head (one head: scores, P V, dQ,
 *     dK, dV), which call the method steps in order and the apparatus hooks
 *     between them.
 *
 * Readings taken where the pages are silent or lost in extraction:
 *  - eq. (1) (lost): differentiating w^L = (1-t)e^{b_r} + t e^{b_{r+1}} through
 *    t, b_r, b_{r+1} and h gives dw/dM = X - w - rho*Delta and
 *    dw/dm = w - X - (1-rho)*Delta, with rho and X as App. B defines them; these
 *    satisfy the stated identity Delta + dw/dM + dw/dm = 0.
 *  - Weight-STE body (lost): w = w^L + sg(w^N - w^L), P = w / sum(w); the
 *    normalization Jacobian is taken at the forward point (P^N, W^N) and the
 *    weight Jacobian is that of w^L (calibration terms included).
 *  - degenerate MinMax rows (M - m <= 1e-12): h is the constant 1 (no gradient
 *    through h); b_r = (1 - r/K)(m - M) keeps its dependence on M and m.
 *  - the clamp of t passes the gradient at its bounds (so the argmax / argmin
 *    keys keep their own-score term, as the zero-sum identity requires).
 *  - interval index r = clamp(floor(u), 0, K-1); Nearest rounds t = 1/2 up.
 *  - FWM: z = -tau is inside the window; only z < -tau is tail (weight 0).
 *  - tied extrema: the extremum's gradient is split evenly among tied keys.
 *  - max_only / min_only: the full score gradient with the other extremum's term
 *    dropped (g_self + g_M, g_self + g_m); FWM has no minimum term, so its
 *    max_only is the full gradient and its min_only the detached one.
 *  - P1: the detached score gradient minus its mean over the row's visible
 *    (causal) keys, tail keys included, so every row sums to zero.
 *  - FWM tail policies: zero (the paper's FWM: w = 0 below the window); floor
 *    (z <- -tau: a key below the window weighs e^{b_0} and, its score clamped,
 *    has no gradient); resolved (the grid b_q = -tau + q h continued below -tau,
 *    q unbounded below, so no key is truncated and every key has the LERP slope).
 *  - exponential baselines: roundings to nearest, ties to even, of the exact
 *    value; BF16-exp rounds z, then e^(rounded z), to bfloat16, and its backward
 *    rounds dL/dw to bfloat16 where it enters the bfloat16 weight, then the
 *    product with the weight; FP8 rounds e^z to E4M3 with e^z as derivative.
 *
 * Scores.  The pages run the attention operator in fp32 (App. C.1 "Numerics
 * and hardware"): a score is an fp32 number.  With cfg.score_fp32 the oracle
 * takes it as the product sum Q_i . K_j formed in double (exact products of the
 * fp32 or bf16 inputs), scaled, and rounded once to fp32; every later step works
 * in double on those values, so row extrema, ties and every decision are those
 * of correctly rounded fp32 scores.  Without it the double sum is used as is
 * (the method in exact arithmetic, for checks against derivatives).
 *
 * Flags and flips (apparatus).  A decision of the method (an interval, a
 * Nearest rounding, the FWM tail edge, a rounding to bfloat16 / E4M3) within
 * `guard` of its boundary (in the decision's own units), and a score whose
 * double product sum lies within its own rounding bound of an fp32 midpoint
 * (so that another correct summation order rounds it the other way), can go
 * either way: the flag list names those positions, and a flip asks the oracle
 * to take the other decision (the other fp32 neighbour of the score) there.
 * This is how a test checks that a result is one of the answers that are
 * correct at that precision.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { KO_MINMAX = 0, KO_FWM = 1 };
/* reconstructions; SOFTMAX, EXP_BF16 and EXP_FP8 are the exponential baselines (no grid);
   BINMEAN weighs each Nearest bin by the mean of e^z over its members, NEAREST_BINMEAN is the
   strict Nearest forward with the bin-mean backward */
enum { KO_LERP = 0, KO_NEAREST = 1, KO_SOFTMAX = 2, KO_EXP_BF16 = 3, KO_EXP_FP8 = 4, KO_BINMEAN = 5,
       KO_NEAREST_BINMEAN = 6 };
enum { KO_WEIGHT_STE = 0, KO_PROB_STE = 1 };
enum { KO_FULL = 0, KO_DETACHED = 1, KO_MAX_ONLY = 2, KO_MIN_ONLY = 3, KO_P1 = 4 };
enum { KO_TAIL_ZERO = 0, KO_TAIL_FLOOR = 1, KO_TAIL_RESOLVED = 2 };

/* flip kinds (bits of a per-key byte) */
enum {
  FLIP_INTERVAL = 1,   /* the other interval at an integer u */
  FLIP_NEAREST = 2,    /* the other rounding at u = k + 1/2 */
  FLIP_TAIL = 4,       /* the other side of the FWM window edge */
  FLIP_ROUND = 8,      /* FP8: the other E4M3 neighbour of e^z; BF16: of z */
  FLIP_ROUND2 = 16,    /* BF16: the other bfloat16 neighbour of e^(rounded z) */
  FLIP_GRAD = 32,      /* BF16: the other bfloat16 neighbour of dL/dw */
  FLIP_SCORE = 64      /* the other fp32 neighbour of the score */
};

typedef struct {
  int32_t calib, recon, ste, grad, K;
  double tau;
  int32_t tail;        /* FWM tail policy (KO_TAIL_*); zero for MinMax */
  int32_t score_fp32;  /* ko_head: 1 rounds each score to fp32 (the operator's precision), 0 keeps
                          the double product sum (the method in exact arithmetic) */
} ko_cfg_t;

#define DEGENERATE_EPS 1e-12

/* ================================================================ 1. the method */

/* Row extrema over the visible keys (App. A): M, m, the first keys attaining them and the
   sets A, C of keys attaining them (membership bytes inA, inC). */
typedef struct {
  double M, m;
  int amax, amin, nA, nC;
} ko_ext_t;

static void ko_extrema(int n, const double *s, ko_ext_t *x, uint8_t *inA, uint8_t *inC) {
  x->M = -INFINITY;
  x->m = INFINITY;
  for (int j = 0; j < n; ++j) {
    if (s[j] > x->M) x->M = s[j];
    if (s[j] < x->m) x->m = s[j];
  }
  x->amax = x->amin = -1;
  x->nA = x->nC = 0;
  for (int j = 0; j < n; ++j) {
    inA[j] = s[j] == x->M;
    inC[j] = s[j] == x->m;
    if (inA[j]) { if (x->amax < 0) x->amax = j; x->nA++; }
    if (inC[j]) { if (x->amin < 0) x->amin = j; x->nC++; }
  }
}

/* Calibration (§3 "Objects and calibration", App. A degenerate branch). */
typedef struct {
  double h;        /* interval width */
  int degenerate;  /* MinMax with M - m <= 1e-12: safe width 1 */
  double *E;       /* grid values E[q] = e^{b_q}, q = 0..K */
} ko_cal_t;

static void ko_calibrate(const ko_cfg_t *cfg, const ko_ext_t *x, ko_cal_t *c) {
  const int K = cfg->K;
  if (cfg->calib == KO_MINMAX) {
    /* MinMax: grid on the observed range, h = (M - m)/K, b_r = (1 - r/K)(m - M) */
    const double span = x->M - x->m;
    c->degenerate = !(span > DEGENERATE_EPS);
    c->h = c->degenerate ? 1.0 : span / K;
    for (int q = 0; q <= K; ++q) c->E[q] = exp((1.0 - (double)q / K) * (x->m - x->M));
  } else {
    /* FWM: fixed window [M - tau, M], h = tau/K, b_r = -tau + r h */
    c->degenerate = 0;
    c->h = cfg->tau / K;
    for (int q = 0; q <= K; ++q) c->E[q] = exp(-cfg->tau + q * c->h);
  }
}

/* Grid value e^{b_q} at any integer q: the table for 0 <= q <= K, else (the resolved FWM grid
   below the window) b_q = -tau + q h computed directly. */
static double ko_grid(const ko_cfg_t *cfg, const ko_cal_t *c, int q) {
  if (q >= 0 && q <= cfg->K) return c->E[q];
  return exp(-cfg->tau + q * c->h);
}

/* Decision of one key (§3): position u in interval widths, interval index r, local position t,
   Nearest index l = r + 1[t >= 1/2], FWM tail flag. */
typedef struct {
  double u, t;
  int r, ell, tail;
} ko_dec_t;

static void ko_decide(const ko_cfg_t *cfg, const ko_ext_t *x, const ko_cal_t *c, double s, ko_dec_t *d) {
  const int K = cfg->K;
  const int resolved = cfg->calib == KO_FWM && cfg->tail == KO_TAIL_RESOLVED;
  d->tail = 0;
  if (cfg->calib == KO_MINMAX) {
    d->u = (s - x->m) / c->h;
  } else if (resolved) {
    const double z = s - x->M;                                /* the grid continues below -tau */
    d->u = ((z > 0.0 ? 0.0 : z) + cfg->tau) / c->h;
  } else {
    const double z = s - x->M;
    d->tail = z < -cfg->tau;                                  /* w = 0 (or floored) below the window */
    const double zc = z < -cfg->tau ? -cfg->tau : (z > 0.0 ? 0.0 : z);   /* clip(z, -tau, 0) */
    d->u = (zc + cfg->tau) / c->h;
  }
  int r = (int)floor(d->u);
  if (r < 0 && !resolved) r = 0;
  if (r > K - 1) r = K - 1;
  double t = d->u - r;
  if (t < 0.0) t = 0.0;
  if (t > 1.0) t = 1.0;
  d->r = r;
  d->t = t;
  d->ell = r + (t >= 0.5);
}

/* Row sums and calibration terms reported by the finishing steps. */
typedef struct {
  double WL, WN, a, b, D;
} ko_sums_t;

/* Reconstruction (§3), normalization and the strict hard forward (App. C.2 (iii)); with g, the
   backward of App. B.  P: the forward's probabilities; Pv: the probabilities dV is taken with
   (the forward's value); dS: the score gradient. */
static void ko_finish_grid(const ko_cfg_t *cfg, int n, const double *s, const double *g,
                           const ko_ext_t *x, const ko_cal_t *c, const ko_dec_t *d,
                           const uint8_t *inA, const uint8_t *inC, double *P, double *Pv, double *dS,
                           ko_sums_t *sum) {
  const int K = cfg->K;
  const int tailp = cfg->calib == KO_FWM ? cfg->tail : KO_TAIL_ZERO;
  const int binmean = cfg->recon == KO_BINMEAN || cfg->recon == KO_NEAREST_BINMEAN;
  double *wL = (double *)malloc(sizeof(double) * n);
  double *wN = (double *)malloc(sizeof(double) * n);
  double *Delta = (double *)malloc(sizeof(double) * n);
  double *gam = (double *)malloc(sizeof(double) * n);

  /* --- reconstruction: LERP between adjacent grid values, Nearest grid centre; a zero-tail key
     weighs 0, a floored tail key sits on the window edge (u = 0) --- */
  for (int j = 0; j < n; ++j) {
    if (d[j].tail && tailp == KO_TAIL_ZERO) { wL[j] = 0.0; wN[j] = 0.0; continue; }
    const double Er = ko_grid(cfg, c, d[j].r), Er1 = ko_grid(cfg, c, d[j].r + 1);
    wL[j] = (1.0 - d[j].t) * Er + d[j].t * Er1;
    wN[j] = ko_grid(cfg, c, d[j].ell);
  }

  /* --- normalization (§3) and the strict hard forward P^N = w^N / W^N (App. C.2 (iii)) --- */
  double WL = 0.0, WN = 0.0;
  for (int j = 0; j < n; ++j) { WL += wL[j]; WN += wN[j]; }
  const int nearest_fwd = cfg->recon == KO_NEAREST || cfg->recon == KO_NEAREST_BINMEAN;
  for (int j = 0; j < n; ++j) {
    P[j] = nearest_fwd ? wN[j] / WN : wL[j] / WL;
    Pv[j] = P[j];                                          /* dV takes the forward value */
  }

  double a = 0.0, b = 0.0, Dsum = 0.0;
  if (binmean) {
    /* --- bin mean (§5, App. I): each bin's weight is the mean of exp over its members, so bin
       mass is conserved; its backward is the exact derivative with the bins held fixed.  Bins are
       the Nearest bins l = 0..K of the row's calibration; keys below an FWM window belong to none
       and weigh 0.  Under NEAREST_BINMEAN (App. I.3) the forward stays the strict Nearest one and
       only the backward is the bin mean's. --- */
    double *Sb = (double *)calloc(K + 1, sizeof(double)), *Gb = (double *)calloc(K + 1, sizeof(double));
    int *nb = (int *)calloc(K + 1, sizeof(int));
    double *ez = (double *)malloc(sizeof(double) * n);
    for (int j = 0; j < n; ++j) {
      ez[j] = d[j].tail ? 0.0 : exp(s[j] - x->M);
      if (d[j].tail) continue;
      Sb[d[j].ell] += ez[j];
      nb[d[j].ell] += 1;
      if (g) Gb[d[j].ell] += g[j];
    }
    double WC = 0.0;
    for (int j = 0; j < n; ++j) {
      wL[j] = d[j].tail ? 0.0 : Sb[d[j].ell] / nb[d[j].ell];   /* the bin's mean of e^z */
      WC += wL[j];
    }
    WL = WC;                                   /* the bin-mean normalizer, recorded as W^L */
    for (int j = 0; j < n; ++j) {
      if (cfg->recon == KO_BINMEAN) P[j] = wL[j] / WC;
      Pv[j] = P[j];
    }
    if (g) {
      /* dL/ds_k = P^E_k (gbar_{B(k)} - sum_j P^C_j g_j), P^E_k = e^{z_k} / W^C, gbar_B the mean of
         g over bin B: the upstream gradient replaced by its bin average */
      for (int j = 0; j < n; ++j) Dsum += wL[j] / WC * g[j];
      for (int j = 0; j < n; ++j) {
        if (d[j].tail) { dS[j] = 0.0; continue; }
        const double gbar = Gb[d[j].ell] / nb[d[j].ell];
        dS[j] = ez[j] / WC * (gbar - Dsum);
      }
      if (cfg->grad == KO_P1) {               /* the rows already sum to zero; kept for form */
        double tot = 0.0;
        for (int j = 0; j < n; ++j) tot += dS[j];
        for (int j = 0; j < n; ++j) dS[j] -= tot / n;
      }
    }
    free(Sb); free(Gb); free(nb); free(ez);
  } else if (g) {
    /* --- normalization Jacobian (App. B): gamma_j = (g_j - sum_i P_i g_i)/W, at (P^L, W^L) for
       LERP and Prob-STE, at (P^N, W^N) for Weight-STE --- */
    const int lerp_point = cfg->recon == KO_LERP || cfg->ste == KO_PROB_STE;
    const double Wg = lerp_point ? WL : WN;
    for (int j = 0; j < n; ++j) Dsum += (lerp_point ? wL[j] / WL : wN[j] / WN) * g[j];
    for (int j = 0; j < n; ++j) gam[j] = (g[j] - Dsum) / Wg;

    /* --- LERP own-score slope (App. B): Delta_j = (e^{b_{r+1}} - e^{b_r})/h; a zero-tail key has
       no weight and a floored one a constant weight: no slope --- */
    for (int j = 0; j < n; ++j) {
      if (d[j].tail) { Delta[j] = 0.0; dS[j] = 0.0; continue; }
      const double dE = ko_grid(cfg, c, d[j].r + 1) - ko_grid(cfg, c, d[j].r);
      Delta[j] = dE / c->h;
      dS[j] = gam[j] * Delta[j];
    }

    /* --- calibration gradient through the row extrema (App. B); max_only / min_only keep one
       of its two channels --- */
    const int keepM = cfg->grad == KO_FULL || cfg->grad == KO_MAX_ONLY;
    const int keepm = cfg->grad == KO_FULL || cfg->grad == KO_MIN_ONLY;
    if (keepM || keepm) {
      if (cfg->calib == KO_MINMAX) {
        for (int j = 0; j < n; ++j) {
          const int r = d[j].r;
          const double t = d[j].t;
          const double rho = (r + t) / K;
          const double X = ((1.0 - t) * r * c->E[r] + t * (r + 1) * c->E[r + 1]) / K;
          double dM, dm;
          if (!c->degenerate) {           /* eq. (1), regular branch */
            dM = X - wL[j] - rho * Delta[j];
            dm = wL[j] - X - (1.0 - rho) * Delta[j];
          } else {                        /* degenerate branch: h is a constant */
            dM = X - wL[j];
            dm = wL[j] - X - Delta[j];
          }
          a += gam[j] * dM;
          b += gam[j] * dm;
        }
      } else {
        /* FWM: in-window keys have dw/dM = -Delta, tail keys contribute nothing */
        for (int j = 0; j < n; ++j) if (!d[j].tail) a += -gam[j] * Delta[j];
      }
      if (!keepM) a = 0.0;
      if (!keepm) b = 0.0;
      /* the extremum gradient is split evenly among tied keys */
      for (int j = 0; j < n; ++j) {
        if (inA[j]) dS[j] += a / x->nA;
        if (cfg->calib == KO_MINMAX && inC[j]) dS[j] += b / x->nC;
      }
    }
    /* --- P1 (App. B "Detach"): the detached row projected onto the zero-sum subspace by
       subtracting its mean over the row's visible keys --- */
    if (cfg->grad == KO_P1) {
      double tot = 0.0;
      for (int j = 0; j < n; ++j) tot += dS[j];
      const double mean = tot / n;
      for (int j = 0; j < n; ++j) dS[j] -= mean;
    }
  }
  sum->WL = WL; sum->WN = WN; sum->a = a; sum->b = b; sum->D = Dsum;
  free(wL); free(wN); free(Delta); free(gam);
}

/* ---------------------------------------------------------------- exponential baselines
 * App. B "Softmax" and App. D.5 "Definitions".  Every weight is an exponential of the
 * row-max-shifted score z = s - M; no grid, no K, no tau:
 *  - SOFTMAX: w = e^z, the exact derivative dw/dz = w.
 *  - EXP_BF16: z rounded to bfloat16, the exponential of that value rounded to bfloat16
 *    (the input rounded before exponentiation, the output after), returned to full
 *    precision for the normalization.  The backward is the chain rule through the casts
 *    (a cast passes the gradient, converted to the tensor's format), with the tensors in
 *    their formats: dL/dw rounded to bfloat16 where it enters the bfloat16 output, times
 *    the bfloat16 weight (the exponential's derivative is its value), rounded to bfloat16.
 *  - EXP_FP8: w = e^z rounded to E4M3 (4 exponent bits, bias 7, 3 significand bits,
 *    subnormals, no infinities), with the identity as the rounding step's derivative, so
 *    dw/dz = e^z (the unrounded exponential), and the normalization Jacobian at the
 *    rounded weights.
 * The row maximum stays on the gradient path in all three: its term -sum_j dL/dz_j goes
 * to the arg-max key(s), split evenly among ties (it vanishes for SOFTMAX in exact
 * arithmetic).  There is no minimum term, so max_only is full and min_only detached, as
 * for FWM.
 */

/* Round x >= 0 to a binary format with mb stored significand bits and smallest normal
   exponent emin (subnormals below it): nearest, ties to even.  *pos is x in units of the
   format's spacing at x (rounding midpoints at pos = k + 1/2); *lo, *hi its two neighbours. */
static double round_fmt(double x, int mb, int emin, double *pos, double *lo, double *hi) {
  if (x == 0.0) { *pos = 0.0; *lo = *hi = 0.0; return 0.0; }
  int e;
  (void)frexp(x, &e);               /* x in [2^(e-1), 2^e) */
  const int E = e - 1 < emin ? emin : e - 1;
  const double ulp = ldexp(1.0, E - mb);
  const double q = x / ulp;         /* exact: a power-of-two scaling */
  const double fl = floor(q);
  *pos = q; *lo = fl * ulp; *hi = (fl + 1.0) * ulp;
  return rint(q) * ulp;             /* rint: nearest, ties to even */
}
/* the same for a signed value; *alt is the other neighbour */
static double round_signed(double x, int mb, int emin, double *pos, double *alt) {
  double lo, hi, pq;
  const double r = round_fmt(fabs(x), mb, emin, &pq, &lo, &hi);
  if (pos) *pos = pq;
  if (alt) *alt = copysign(r == lo ? hi : lo, x);
  return copysign(r, x);
}
#define BF16_MB 7
#define BF16_EMIN (-126)
#define E4M3_MB 3
#define E4M3_EMIN (-6)

/* E4M3 byte of a value in [0, 1] that the format represents */
static int e4m3_code(double w) {
  if (w <= 0.0) return 0;
  if (w < ldexp(1.0, E4M3_EMIN)) return (int)(w / ldexp(1.0, E4M3_EMIN - E4M3_MB));   /* subnormal */
  int e;
  double f = frexp(w, &e);          /* w = f 2^e, f in [0.5, 1) */
  const int E = e - 1;              /* w = (1 + m/8) 2^E */
  const int mant = (int)((2.0 * f - 1.0) * 8.0);
  return ((E + 7) << 3) | mant;
}
/* low byte of the bfloat16 encoding of a value the format represents */
static int bf16_low_byte(double w) {
  const float f = (float)w;         /* exact: bfloat16 values are floats */
  uint32_t bits;
  memcpy(&bits, &f, 4);
  return (int)((bits >> 16) & 0xFF);
}

/* One key's weight under an exponential baseline. */
typedef struct {
  double z;    /* s - M */
  double w;    /* the weight */
  double de;   /* dw/dz */
  int code;    /* a byte naming the weight (for the bins map) */
} ko_xdec_t;

static void ko_exp_decide(const ko_cfg_t *cfg, double z, ko_xdec_t *d) {
  d->z = z;
  d->code = 0;
  if (cfg->recon == KO_SOFTMAX) {
    d->w = exp(z);
    d->de = d->w;
  } else if (cfg->recon == KO_EXP_FP8) {
    double pos, lo, hi;
    const double we = exp(z);
    d->w = round_fmt(we, E4M3_MB, E4M3_EMIN, &pos, &lo, &hi);
    d->de = we;
    d->code = e4m3_code(d->w);
  } else {                          /* EXP_BF16 */
    const double zb = round_signed(z, BF16_MB, BF16_EMIN, NULL, NULL);
    d->w = round_signed(exp(zb), BF16_MB, BF16_EMIN, NULL, NULL);
    d->de = d->w;
    d->code = bf16_low_byte(d->w);
  }
}

/* gamma_j = dL/dw_j = (g_j - sum_i P_i g_i)/W (App. B normalization Jacobian at the weights). */
static double ko_exp_gamma(int n, const double *g, const double *P, double W, double *gam) {
  double D = 0.0;
  for (int j = 0; j < n; ++j) D += P[j] * g[j];
  for (int j = 0; j < n; ++j) gam[j] = (g[j] - D) / W;
  return D;
}

/* dL/dz_j from gamma; BF16: gb is gamma rounded to bfloat16 where it enters the bfloat16 weight,
   and the product with the weight is rounded to bfloat16 again.  Then the row maximum's term
   (z = s - M) on the arg-max keys, and P1. */
static double ko_exp_backward(const ko_cfg_t *cfg, int n, const ko_xdec_t *d, const double *gam,
                              const double *gb, const uint8_t *inA, int nA, double *dS) {
  for (int j = 0; j < n; ++j) {
    if (cfg->recon == KO_EXP_BF16) dS[j] = round_signed(gb[j] * d[j].w, BF16_MB, BF16_EMIN, NULL, NULL);
    else dS[j] = gam[j] * d[j].de;
  }
  double a = 0.0;
  if (cfg->grad == KO_FULL || cfg->grad == KO_MAX_ONLY) {
    for (int j = 0; j < n; ++j) a -= dS[j];
    for (int j = 0; j < n; ++j)
      if (inA[j]) dS[j] += a / nA;
  }
  if (cfg->grad == KO_P1) {
    double tot = 0.0;
    for (int j = 0; j < n; ++j) tot += dS[j];
    for (int j = 0; j < n; ++j) dS[j] -= tot / n;
  }
  return a;
}

/* ================================================================ 2. checking apparatus */

typedef struct {
  double guard;
  int64_t cap;
  int64_t count;      /* may exceed cap; only the first cap entries are stored */
  int32_t *pos;       /* cap x 3: row, key, kind */
  double *dist;       /* cap */
} ko_flags_t;

static void flag_push(ko_flags_t *f, int row, int key, int kind, double dist) {
  int64_t idx;
#ifdef _OPENMP
#pragma omp atomic capture
#endif
  idx = f->count++;
  if (idx < f->cap) {
    f->pos[3 * idx] = row; f->pos[3 * idx + 1] = key; f->pos[3 * idx + 2] = kind;
    f->dist[idx] = dist;
  }
}

/* Decisions within the guard (in interval widths) of a boundary. */
static void ko_flag_decision(const ko_cfg_t *cfg, const ko_ext_t *x, const ko_cal_t *c, double s,
                             const ko_dec_t *d, int row_id, int key, ko_flags_t *f) {
  const int K = cfg->K;
  const int resolved = cfg->calib == KO_FWM && cfg->tail == KO_TAIL_RESOLVED;
  const int nearest_bins = cfg->recon == KO_NEAREST || cfg->recon == KO_BINMEAN || cfg->recon == KO_NEAREST_BINMEAN;
  const double gj = f->guard;
  if (cfg->calib == KO_FWM && !resolved && fabs(s - x->M + cfg->tau) / c->h < gj)
    flag_push(f, row_id, key, FLIP_TAIL, fabs(s - x->M + cfg->tau) / c->h);
  const double kint = floor(d->u + 0.5);
  /* interval boundaries: the integers 1..K-1, and every integer below K on the resolved grid */
  if ((resolved || (K >= 2 && kint >= 1)) && kint <= K - 1 && fabs(d->u - kint) < gj)
    flag_push(f, row_id, key, FLIP_INTERVAL, fabs(d->u - kint));
  const double khalf = floor(d->u) + 0.5;
  if (nearest_bins && khalf < K && fabs(d->u - khalf) < gj)
    flag_push(f, row_id, key, FLIP_NEAREST, fabs(d->u - khalf));
}

/* The other decision at a flagged position: the other side of the window edge, the other
   interval at an integer u, the other rounding at u = k + 1/2. */
static void ko_flip_decision(const ko_cfg_t *cfg, uint8_t bits, ko_dec_t *d) {
  const int K = cfg->K;
  const int resolved = cfg->calib == KO_FWM && cfg->tail == KO_TAIL_RESOLVED;
  if (bits & FLIP_TAIL) {
    d->tail = !d->tail;
    /* a key leaving the tail sits on the window edge; one entering a floored tail too */
    if (!d->tail || cfg->tail == KO_TAIL_FLOOR) { d->u = 0.0; d->r = 0; d->t = 0.0; }
  }
  if (bits & FLIP_INTERVAL) {
    const int kint = (int)floor(d->u + 0.5);
    if ((kint >= 1 || resolved) && kint <= K - 1) {
      d->r = (d->r == kint) ? kint - 1 : kint;
      double t = d->u - d->r;
      d->t = t < 0.0 ? 0.0 : (t > 1.0 ? 1.0 : t);
    }
  }
  d->ell = d->r + (d->t >= 0.5);
  if (bits & FLIP_NEAREST) {
    int k2 = (int)floor(d->u);
    if (k2 > K - 1) k2 = K - 1;
    d->ell = (d->ell == k2 + 1) ? k2 : k2 + 1;
  }
}

/* Exponential baselines: roundings within the guard (in spacings of the target format) of a
   midpoint (z = s - M is exact in double for fp32 scores). */
static void ko_flag_exp(const ko_cfg_t *cfg, const ko_xdec_t *d, int row_id, int key, ko_flags_t *f) {
  double pos, lo, hi, alt;
  if (cfg->recon == KO_EXP_FP8) {
    (void)round_fmt(exp(d->z), E4M3_MB, E4M3_EMIN, &pos, &lo, &hi);
    const double dist = fabs(pos - floor(pos) - 0.5);
    if (dist < f->guard) flag_push(f, row_id, key, FLIP_ROUND, dist);
  } else if (cfg->recon == KO_EXP_BF16) {
    const double zb = round_signed(d->z, BF16_MB, BF16_EMIN, &pos, &alt);
    double dist = fabs(pos - floor(pos) - 0.5);
    if (d->z != 0.0 && dist < f->guard) flag_push(f, row_id, key, FLIP_ROUND, dist);
    (void)round_fmt(exp(zb), BF16_MB, BF16_EMIN, &pos, &lo, &hi);
    dist = fabs(pos - floor(pos) - 0.5);
    if (dist < f->guard) flag_push(f, row_id, key, FLIP_ROUND2, dist);
  }
}

/* The other rounding(s) at a flagged position of an exponential baseline. */
static void ko_flip_exp(const ko_cfg_t *cfg, uint8_t bits, ko_xdec_t *d) {
  double pos, lo, hi, alt;
  if (cfg->recon == KO_EXP_FP8 && (bits & FLIP_ROUND)) {
    const double r = round_fmt(exp(d->z), E4M3_MB, E4M3_EMIN, &pos, &lo, &hi);
    d->w = r == lo ? hi : lo;
    d->code = e4m3_code(d->w);
  } else if (cfg->recon == KO_EXP_BF16 && (bits & (FLIP_ROUND | FLIP_ROUND2))) {
    double zb = round_signed(d->z, BF16_MB, BF16_EMIN, NULL, &alt);
    if (bits & FLIP_ROUND) zb = alt;
    double wb = round_signed(exp(zb), BF16_MB, BF16_EMIN, NULL, &alt);
    if (bits & FLIP_ROUND2) wb = alt;
    d->w = wb;
    d->de = wb;
    d->code = bf16_low_byte(wb);
  }
}

/* BF16-exp backward: dL/dw within the guard (in bfloat16 spacings) of a rounding midpoint. */
static void ko_flag_grad(int n, const double *gam, int row_id, const int32_t *key_id, ko_flags_t *f) {
  for (int j = 0; j < n; ++j) {
    double pos;
    (void)round_signed(gam[j], BF16_MB, BF16_EMIN, &pos, NULL);
    const double dist = fabs(pos - floor(pos) - 0.5);
    if (gam[j] != 0.0 && dist < f->guard) flag_push(f, row_id, key_id[j], FLIP_GRAD, dist);
  }
}

/* ================================================================ 3. drivers */

/* per-row record: doubles and ints */
enum { RD_M = 0, RD_m, RD_h, RD_WL, RD_WN, RD_a, RD_b, RD_D, RD_N };
enum { RI_amax = 0, RI_amin, RI_nA, RI_nC, RI_degenerate, RI_N };

int ko_rowd_n(void) { return RD_N; }
int ko_rowi_n(void) { return RI_N; }

/* Per-key decision outputs a caller may ask for (any pointer may be NULL). */
typedef struct {
  double *u, *t;
  int32_t *r, *ell, *code;
  uint8_t *tail;
} ko_keyout_t;

/*
 * One attention row: the method's steps in order, with the apparatus between them.
 *  s[0..n): the scaled scores of the row's visible keys; g: dL/dP_j (NULL: forward only);
 *  flip: per-key flip bits (NULL: none); flags: the flag list (NULL: no flags).  Outputs P, Pv
 *  (probabilities for dV), dS (if g), key decisions, the row record.
 */
static void ko_row_run(const ko_cfg_t *cfg, int n, const double *s, const double *g, const uint8_t *flip,
                       ko_flags_t *flags, int row_id, const int32_t *key_id,
                       double *P, double *Pv, double *dS, const ko_keyout_t *ko, double *rowd, int32_t *rowi) {
  uint8_t *inA = (uint8_t *)malloc(n), *inC = (uint8_t *)malloc(n);
  ko_ext_t x;
  ko_extrema(n, s, &x, inA, inC);
  ko_sums_t sum = {0.0, 0.0, 0.0, 0.0, 0.0};
  double h = 0.0;
  int degenerate = 0;

  if (cfg->recon >= KO_SOFTMAX && cfg->recon <= KO_EXP_FP8) {
    ko_xdec_t *d = (ko_xdec_t *)malloc(sizeof(ko_xdec_t) * n);
    for (int j = 0; j < n; ++j) {
      ko_exp_decide(cfg, s[j] - x.M, &d[j]);
      if (flags) ko_flag_exp(cfg, &d[j], row_id, key_id[j], flags);
      if (flip && flip[j]) ko_flip_exp(cfg, flip[j], &d[j]);
    }
    double W = 0.0;
    for (int j = 0; j < n; ++j) W += d[j].w;
    for (int j = 0; j < n; ++j) { P[j] = d[j].w / W; Pv[j] = P[j]; }
    sum.WL = sum.WN = W;
    if (g) {
      double *gam = (double *)malloc(sizeof(double) * n), *gb = (double *)malloc(sizeof(double) * n);
      sum.D = ko_exp_gamma(n, g, P, W, gam);
      for (int j = 0; j < n; ++j) {
        double alt;
        gb[j] = round_signed(gam[j], BF16_MB, BF16_EMIN, NULL, &alt);   /* BF16-exp: into the bf16 weight */
        if (flip && (flip[j] & FLIP_GRAD)) gb[j] = alt;
      }
      if (flags && cfg->recon == KO_EXP_BF16) ko_flag_grad(n, gam, row_id, key_id, flags);
      sum.a = ko_exp_backward(cfg, n, d, gam, gb, inA, x.nA, dS);
      free(gam); free(gb);
    }
    if (ko->u) for (int j = 0; j < n; ++j) {
      ko->u[j] = d[j].z; ko->r[j] = 0; ko->t[j] = 0.0; ko->ell[j] = d[j].code; ko->tail[j] = 0;
    }
    if (ko->code) for (int j = 0; j < n; ++j) ko->code[j] = d[j].code;
    free(d);
  } else {
    double *E = (double *)malloc(sizeof(double) * (cfg->K + 1));
    ko_cal_t c;
    c.E = E;
    ko_calibrate(cfg, &x, &c);
    ko_dec_t *d = (ko_dec_t *)malloc(sizeof(ko_dec_t) * n);
    for (int j = 0; j < n; ++j) {
      ko_decide(cfg, &x, &c, s[j], &d[j]);
      if (flags) ko_flag_decision(cfg, &x, &c, s[j], &d[j], row_id, key_id[j], flags);
      if (flip && flip[j]) ko_flip_decision(cfg, flip[j], &d[j]);
    }
    ko_finish_grid(cfg, n, s, g, &x, &c, d, inA, inC, P, Pv, dS, &sum);
    if (ko->u) for (int j = 0; j < n; ++j) {
      ko->u[j] = d[j].u; ko->r[j] = d[j].r; ko->t[j] = d[j].t; ko->ell[j] = d[j].ell; ko->tail[j] = (uint8_t)d[j].tail;
    }
    if (ko->code) {
      /* bins map: the interval index (LERP) or Nearest index; on the resolved FWM grid the index
         + 64, clamped below at 0; 254 for FWM tail keys */
      const int resolved = cfg->calib == KO_FWM && cfg->tail == KO_TAIL_RESOLVED;
      for (int j = 0; j < n; ++j) {
        int idx = cfg->recon == KO_LERP ? d[j].r : d[j].ell;
        if (resolved) idx = idx < -64 ? 0 : idx + 64;
        ko->code[j] = d[j].tail ? 254 : idx;
      }
    }
    h = c.h;
    degenerate = c.degenerate;
    free(d); free(E);
  }
  if (rowd) {
    rowd[RD_M] = x.M; rowd[RD_m] = x.m; rowd[RD_h] = h; rowd[RD_WL] = sum.WL; rowd[RD_WN] = sum.WN;
    rowd[RD_a] = sum.a; rowd[RD_b] = sum.b; rowd[RD_D] = sum.D;
  }
  if (rowi) {
    rowi[RI_amax] = x.amax; rowi[RI_amin] = x.amin; rowi[RI_nA] = x.nA; rowi[RI_nC] = x.nC;
    rowi[RI_degenerate] = degenerate;
  }
  free(inA); free(inC);
}

static int ko_cfg_ok(const ko_cfg_t *cfg) {
  if (!cfg || cfg->K < 1) return 0;
  if (cfg->calib != KO_MINMAX && cfg->calib != KO_FWM) return 0;
  if (cfg->calib == KO_FWM && !(cfg->tau > 0.0)) return 0;
  if (cfg->tail < KO_TAIL_ZERO || cfg->tail > KO_TAIL_RESOLVED || (cfg->calib == KO_MINMAX && cfg->tail != 0)) return 0;
  if (cfg->recon < KO_LERP || cfg->recon > KO_NEAREST_BINMEAN) return 0;
  if (cfg->recon >= KO_BINMEAN && cfg->tail != KO_TAIL_ZERO) return 0;   /* bin mean: zero tail only */
  return 1;
}

/* Row-level entry point (no flags).  g may be NULL for forward only. */
int ko_row(const ko_cfg_t *cfg, int n, const double *s, const double *g, const uint8_t *flip,
           double *P, double *dS, double *u, int32_t *r, double *t, int32_t *ell, uint8_t *tail,
           double *rowd, int32_t *rowi) {
  if (!ko_cfg_ok(cfg) || n < 1 || !s || !P || (g && !dS)) return -1;
  if (u && !(r && t && ell && tail)) return -1;
  double *Pv = (double *)malloc(sizeof(double) * n);
  ko_keyout_t ko = {u, t, r, ell, NULL, tail};
  ko_row_run(cfg, n, s, g, flip, NULL, 0, NULL, P, Pv, dS, &ko, rowd, rowi);
  free(Pv);
  return 0;
}

/*
 * One attention head: Q, K, V, dO are [T, D] row-major doubles.  Scores are
 * s_ij = scale * Q_i . K_j over the visible keys (j <= i when causal).
 * O = P V; dQ_i = scale * sum_j dS_ij K_j; dK_j = scale * sum_i dS_ij Q_i;
 * dV_j = sum_i P_ij dO_i.  dO may be NULL (forward only; dQ/dK/dV untouched).
 * flips: nflip triples (row, key, bits).  flags: optional near-boundary report (flag_cap > 0).
 * bins: optional [T, T] decision map: Nearest index l (Nearest, bin mean) or interval index r
 * (LERP) for visible keys, 254 for FWM tail keys, 255 for keys the query does not see; the
 * exponential baselines give the E4M3 byte of the weight (EXP_FP8), the low byte of the
 * bfloat16 weight (EXP_BF16) or 0 (SOFTMAX).
 * row_mask: optional [T]; rows with 0 are skipped (their O, dQ rows stay 0 and they add nothing
 * to dK, dV), so a caller can get the contributions of chosen rows alone.
 * scores: optional [T, T]: the fp32 scores of the visible keys (0 elsewhere).
 */
int ko_head(const ko_cfg_t *cfg, int T, int D, int causal, double scale,
            const double *Q, const double *Kt, const double *V, const double *dO,
            double *O, double *dQ, double *dK, double *dV, double *rowd, int32_t *rowi,
            int64_t nflip, const int32_t *flips,
            double guard, int64_t flag_cap, int32_t *flag_pos, double *flag_dist, int64_t *nflags,
            uint8_t *bins, const uint8_t *row_mask, double *scores, int nthreads) {
  if (!ko_cfg_ok(cfg) || T < 1 || D < 1 || !Q || !Kt || !V || !O) return -1;
  if (dO && !(dQ && dK && dV)) return -1;
  ko_flags_t fl_store, *fl = NULL;
  if (flag_cap > 0 && flag_pos && flag_dist) {
    fl_store.guard = guard; fl_store.cap = flag_cap; fl_store.count = 0;
    fl_store.pos = flag_pos; fl_store.dist = flag_dist;
    fl = &fl_store;
  }
  if (nthreads < 1) nthreads = 1;
  memset(O, 0, sizeof(double) * (size_t)T * D);
  if (dO) {
    memset(dQ, 0, sizeof(double) * (size_t)T * D);
    memset(dK, 0, sizeof(double) * (size_t)T * D);
    memset(dV, 0, sizeof(double) * (size_t)T * D);
  }
  /* thread-private dK, dV accumulators, summed in thread order at the end */
  double *accK = NULL, *accV = NULL;
  if (dO) {
    accK = (double *)calloc((size_t)nthreads * T * D, sizeof(double));
    accV = (double *)calloc((size_t)nthreads * T * D, sizeof(double));
    if (!accK || !accV) { free(accK); free(accV); return -2; }
  }

#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
#endif
  for (int i = 0; i < T; ++i) {
    if (row_mask && !row_mask[i]) continue;
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    const int n = causal ? i + 1 : T;                     /* the visible keys j <= i (causal) */
    double *s = (double *)malloc(sizeof(double) * n);
    double *g = dO ? (double *)malloc(sizeof(double) * n) : NULL;
    double *P = (double *)malloc(sizeof(double) * n);
    double *Pv = (double *)malloc(sizeof(double) * n);
    double *dS = dO ? (double *)malloc(sizeof(double) * n) : NULL;
    int32_t *kid = (int32_t *)malloc(sizeof(int32_t) * n);
    int32_t *code = bins ? (int32_t *)malloc(sizeof(int32_t) * n) : NULL;
    uint8_t *flip = NULL;
    for (int64_t f = 0; f < nflip; ++f) {
      if (flips[3 * f] == i && flips[3 * f + 1] >= 0 && flips[3 * f + 1] < n) {
        if (!flip) flip = (uint8_t *)calloc(n, 1);
        flip[flips[3 * f + 1]] |= (uint8_t)flips[3 * f + 2];
      }
    }
    for (int j = 0; j < n; ++j) {
      kid[j] = j;
      double acc = 0.0, aabs = 0.0;
      for (int k = 0; k < D; ++k) {
        acc += Q[(size_t)i * D + k] * Kt[(size_t)j * D + k];
        aabs += fabs(Q[(size_t)i * D + k] * Kt[(size_t)j * D + k]);
      }
      s[j] = cfg->score_fp32 ? (double)(float)(scale * acc) : scale * acc;   /* fp32 score (App. C.1) */
      if (cfg->score_fp32 && (fl || (flip && (flip[j] & FLIP_SCORE)))) {
        /* the double sum errs by at most 2 D 2^-53 sum|q k| and the scaling by 2^-53 |s|; a
           summation in another order (the same bound) may round to the other fp32 neighbour
           when the exact value is that close to a midpoint */
        const double x = scale * acc;
        const double bound = (4.0 * D + 4.0) * 0x1p-53 * fabs(scale) * aabs;
        const float lo = (float)x <= x ? (float)x : nextafterf((float)x, -INFINITY);
        const float hi = nextafterf(lo, INFINITY);
        const double mid = 0.5 * ((double)lo + (double)hi);
        if (fl && fabs(x - mid) <= bound) flag_push(fl, i, j, FLIP_SCORE, fabs(x - mid));
        if (flip && (flip[j] & FLIP_SCORE)) s[j] = s[j] == (double)lo ? (double)hi : (double)lo;
      }
      if (dO) {
        double ga = 0.0;
        for (int k = 0; k < D; ++k) ga += dO[(size_t)i * D + k] * V[(size_t)j * D + k];
        g[j] = ga;                                          /* g_j = dL/dP_j = dO_i . V_j */
      }
    }
    if (scores) {
      for (int j = 0; j < T; ++j) scores[(size_t)i * T + j] = 0.0;
      for (int j = 0; j < n; ++j) scores[(size_t)i * T + j] = s[j];
    }
    ko_keyout_t ko = {NULL, NULL, NULL, NULL, code, NULL};
    ko_row_run(cfg, n, s, g, flip, fl, i, kid, P, Pv, dS, &ko,
               rowd ? rowd + (size_t)i * RD_N : NULL, rowi ? rowi + (size_t)i * RI_N : NULL);
    if (bins) {
      for (int j = 0; j < T; ++j) bins[(size_t)i * T + j] = 255;
      for (int j = 0; j < n; ++j) bins[(size_t)i * T + j] = (uint8_t)code[j];
    }
    /* O_i = sum_j P_ij V_j */
    for (int j = 0; j < n; ++j)
      for (int k = 0; k < D; ++k) O[(size_t)i * D + k] += P[j] * V[(size_t)j * D + k];
    if (dO) {
      double *aK = accK + (size_t)tid * T * D, *aV = accV + (size_t)tid * T * D;
      for (int j = 0; j < n; ++j) {
        for (int k = 0; k < D; ++k) {
          dQ[(size_t)i * D + k] += scale * dS[j] * Kt[(size_t)j * D + k];
          aK[(size_t)j * D + k] += scale * dS[j] * Q[(size_t)i * D + k];
          aV[(size_t)j * D + k] += Pv[j] * dO[(size_t)i * D + k];
        }
      }
    }
    free(s); free(g); free(P); free(Pv); free(dS); free(kid); free(flip); free(code);
  }
  if (dO) {
    for (int th = 0; th < nthreads; ++th)
      for (size_t x = 0; x < (size_t)T * D; ++x) {
        dK[x] += accK[(size_t)th * T * D + x];
        dV[x] += accV[(size_t)th * T * D + x];
      }
    free(accK); free(accV);
  }
  if (nflags) *nflags = fl ? fl->count : 0;
  return 0;
}
