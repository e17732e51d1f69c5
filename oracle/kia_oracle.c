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
 * detach (legacy) and its P1 projection, Weight-STE, Prob-STE, FWM), App. C.2
 * (iii) (strict hard forward), §5.1 and the single-channel ablation paragraph of
 * App. I (max_only / min_only keep one extremum's calibration term).  Steps follow the pages' order and notation: calibration ->
 * interval index r_j and local position t_j -> LERP / Nearest weights ->
 * normalization -> P V; backward: gamma (normalization Jacobian) -> Delta
 * (secant slope) -> calibration terms through the row extrema -> dS -> dQ, dK, dV.
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
 *  - FWM tail policies (App. C.3 tau-selection stages, App. D.4 tail policy):
 *    zero (the paper's FWM: w = 0 below the window); floor (z <- -tau: a key
 *    below the window weighs e^{b_0} and, its score clamped, has no gradient);
 *    resolved (the grid b_r = -tau + r h continued below -tau, r unbounded
 *    below, so no key is truncated and every key has the LERP slope).
 *
 * Flip list: a test may ask the oracle to take, at named (row, key) positions,
 * the other valid decision at a bin boundary (the other interval at an integer
 * u, the other rounding at u = k + 1/2, the other side of the FWM tail edge).
 * The positions come from the oracle's own list of near-boundary positions;
 * this is how a test checks that a result computed in fp32 is one of the
 * answers that are correct within the boundary guard.
 *
 * Near-boundary positions are those within `guard` (in units of the interval
 * width) of a boundary, or within the distance that representing the scores in
 * fp32 (the operator's precision) can move u: a score rounded to fp32 moves by
 * at most one unit in its last place, 2^-23 |s|, and u inherits that change in s
 * and in the row extrema it is measured from.
 *
 * Mutations: cfg.mutation != 0 plants one known mistake; tests use this to
 * show that the pins catch such mistakes.  Zero in every other use.
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

enum { FLIP_INTERVAL = 1, FLIP_NEAREST = 2, FLIP_TAIL = 4, FLIP_ROUND = 8, FLIP_ROUND2 = 16 };

enum {
  MUT_NONE = 0,
  MUT_DROP_RHO_DELTA = 1,   /* dw/dM without the -rho*Delta term */
  MUT_SIGN_DM = 2,          /* dw/dm with the wrong sign */
  MUT_DELTA_TIMES_H = 3,    /* secant slope multiplied by h instead of divided */
  MUT_NEAREST_STRICT = 4,   /* Nearest rounds t = 1/2 down */
  MUT_WSTE_USES_LERP = 5,   /* Weight-STE gamma taken at (P^L, W^L) */
  MUT_DK_WITH_DO = 6,       /* dK accumulates dO instead of Q */
  MUT_TAIL_INCLUSIVE = 7,   /* FWM tail includes z = -tau */
  MUT_NO_TIE_SPLIT = 8,     /* extremum gradient given whole to the first tied key */
  MUT_NEAREST_FWD_LERP = 9, /* Nearest forward returns P^L */
  MUT_EXTREMA_ALL_KEYS = 10,/* row extrema over all keys, ignoring the causal set */
  MUT_DQ_NO_SCALE = 11,     /* dQ without the score scale */
  MUT_NO_HSAFE = 12,        /* degenerate rows divide by span/K */
  MUT_INTERVAL_ROUND = 13,  /* interval index by rounding instead of floor */
  MUT_GAMMA_SIGN = 14,      /* gamma = (D - g)/W */
  MUT_DV_WITH_PL = 15,      /* Nearest dV uses P^L instead of the forward P^N */
  MUT_FWM_GRID_SHIFT = 16,  /* FWM grid b_r = -tau + (r+1)h */
  MUT_X_INDEX = 17,         /* X uses r instead of r+1 in its second term */
  MUT_DETACH_KEEPS_M = 18,  /* detached mode keeps the M channel */
  MUT_ONLY_SWAPPED = 19,    /* max_only keeps the m channel, min_only the M channel */
  MUT_P1_SKIP_TAIL = 20,    /* P1 shifts only the keys inside the FWM window */
  MUT_FLOOR_TAIL_SLOPE = 21, /* floored tail keys keep the slope of the first interval */
  MUT_RESOLVED_GRID_CLAMP = 22, /* the resolved grid reads the table's end values below the window */
  MUT_FP8_TRUNCATES = 23,   /* FP8-rounded exp rounds toward zero */
  MUT_BF16_GRAD_UNROUNDED = 24, /* BF16-exp backward keeps the fp32 gradient (no bf16 casts) */
  MUT_FP8_DELTA_ROUNDED = 25, /* FP8-rounded exp backward uses the rounded weight as derivative */
  MUT_BINMEAN_SUM = 26,     /* a bin weighs the sum of e^z over its members, not the mean */
  MUT_BINMEAN_OWN_G = 27    /* the bin-mean backward keeps each key's own upstream gradient */
};

typedef struct {
  int32_t calib, recon, ste, grad, K, mutation;
  double tau;
  int32_t tail;   /* FWM tail policy (KO_TAIL_*); zero for MinMax */
} ko_cfg_t;

/* Grid value e^{b_q} at any integer q: the table for 0 <= q <= K, else (the resolved FWM grid
   below the window) b_q = -tau + q h computed directly. */
static double grid_at(const double *E, int K, double tau, double h, int q, int mut) {
  if (q >= 0 && q <= K) return E[q];
  if (mut == MUT_RESOLVED_GRID_CLAMP) return E[q < 0 ? 0 : K];
  return exp(-tau + q * h);
}

/* per-row record: doubles */
enum { RD_M = 0, RD_m, RD_h, RD_WL, RD_WN, RD_a, RD_b, RD_gapM, RD_gapm, RD_D, RD_tolM, RD_tolm, RD_N };
/* per-row record: ints */
enum { RI_amax = 0, RI_amin, RI_nA, RI_nC, RI_degenerate, RI_amax2, RI_amin2, RI_N };

#define DEGENERATE_EPS 1e-12

int ko_rowd_n(void) { return RD_N; }
int ko_rowi_n(void) { return RI_N; }

typedef struct {
  double guard;
  int64_t cap;
  int64_t count;      /* may exceed cap; only the first cap entries are stored */
  int32_t *pos;       /* cap x 3: row, key, kind */
  double *dist;       /* cap */
} ko_flags_t;

static void flag_push(ko_flags_t *f, int row, int key, int kind, double dist) {
  if (!f) return;
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
 * Readings: roundings are to nearest, ties to even, on the exact value (the exponential
 * of the rounded bfloat16 input, correctly rounded to bfloat16; e^z correctly rounded to
 * E4M3).
 */

/* Round x >= 0 to a binary format with mb stored significand bits and smallest normal
   exponent emin (subnormals below it): nearest, ties to even.  *pos is x in units of the
   format's spacing at x (rounding midpoints at pos = k + 1/2); *lo, *hi its two neighbours. */
static double round_fmt(double x, int mb, int emin, int truncate, double *pos, double *lo, double *hi) {
  if (x == 0.0) { *pos = 0.0; *lo = *hi = 0.0; return 0.0; }
  int e;
  (void)frexp(x, &e);               /* x in [2^(e-1), 2^e) */
  int E = e - 1 < emin ? emin : e - 1;
  const double ulp = ldexp(1.0, E - mb);
  const double q = x / ulp;         /* exact: a power-of-two scaling */
  const double fl = floor(q);
  *pos = q; *lo = fl * ulp; *hi = (fl + 1.0) * ulp;
  return (truncate ? fl : rint(q)) * ulp;   /* rint: nearest, ties to even */
}
static double round_signed(double x, int mb, int emin, double *pos, double *alt) {
  double lo, hi, pq;
  const double r = round_fmt(fabs(x), mb, emin, 0, &pq, &lo, &hi);
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
  uint32_t b;
  memcpy(&b, &f, 4);
  return (int)((b >> 16) & 0xFF);
}

static void ko_row_exp(const ko_cfg_t *cfg, int n, const double *s, const double *g, const double *gabs,
                       const uint8_t *flip, double *P, double *dS, double *PL_out,
                       double *z_out, int32_t *r_out, double *t_out, int32_t *code_out, uint8_t *tail_out,
                       double *rowd, int32_t *rowi, int row_id, const int32_t *key_id, ko_flags_t *flags,
                       const double *eb, double *amb) {
  const int mode = cfg->recon, mut = cfg->mutation;
  double *w = (double *)malloc(sizeof(double) * n);
  double *de = (double *)malloc(sizeof(double) * n);   /* dw/dz (SOFTMAX, EXP_FP8) */
  int32_t *code = (int32_t *)malloc(sizeof(int32_t) * n);
  double M = -INFINITY, m = INFINITY;
  for (int j = 0; j < n; ++j) {
    if (s[j] > M) M = s[j];
    if (s[j] < m) m = s[j];
  }
  int amax = -1, amin = -1, nA = 0, nC = 0, ibelowM = -1, iabovem = -1;
  double belowM = -INFINITY, abovem = INFINITY;
  for (int j = 0; j < n; ++j) {
    if (s[j] == M) { if (amax < 0) amax = j; nA++; } else if (s[j] > belowM) { belowM = s[j]; ibelowM = j; }
    if (s[j] == m) { if (amin < 0) amin = j; nC++; } else if (s[j] < abovem) { abovem = s[j]; iabovem = j; }
  }
  const double ebM = eb ? eb[amax] : 0.0, ebm = eb ? eb[amin] : 0.0;

  /* --- forward: the weights --- */
  for (int j = 0; j < n; ++j) {
    const double z = s[j] - M;
    const int kid = key_id ? key_id[j] : j;
    const uint8_t fl = flip ? flip[j] : 0;
    const double ez = eb ? eb[j] + ebM : 0.0;      /* how far fp32 scores can move z */
    code[j] = 0;
    if (mode == KO_SOFTMAX) {
      w[j] = exp(z);
      de[j] = w[j];
    } else if (mode == KO_EXP_FP8) {
      double pos, lo, hi;
      const double we = exp(z);
      double r = round_fmt(we, E4M3_MB, E4M3_EMIN, mut == MUT_FP8_TRUNCATES, &pos, &lo, &hi);
      const double dist = fabs(pos - floor(pos) - 0.5);
      if (flags && dist < fmax(flags->guard, pos * ez)) flag_push(flags, row_id, kid, FLIP_ROUND, dist);
      if (fl & FLIP_ROUND) r = (r == lo) ? hi : lo;
      w[j] = r;
      de[j] = mut == MUT_FP8_DELTA_ROUNDED ? r : we;
      code[j] = e4m3_code(r);
    } else {                                      /* EXP_BF16 */
      double pos, alt;
      double zb = round_signed(z, BF16_MB, BF16_EMIN, &pos, &alt);
      double dist = fabs(pos - floor(pos) - 0.5);
      if (flags && z != 0.0 && dist < fmax(flags->guard, pos * ez / fabs(z)))
        flag_push(flags, row_id, kid, FLIP_ROUND, dist);
      if (fl & FLIP_ROUND) zb = alt;
      double wb = round_signed(exp(zb), BF16_MB, BF16_EMIN, &pos, &alt);
      dist = fabs(pos - floor(pos) - 0.5);
      if (flags && dist < flags->guard) flag_push(flags, row_id, kid, FLIP_ROUND2, dist);
      if (fl & FLIP_ROUND2) wb = alt;
      w[j] = wb;
      de[j] = wb;
      code[j] = bf16_low_byte(wb);
    }
  }
  double W = 0.0;
  for (int j = 0; j < n; ++j) W += w[j];
  for (int j = 0; j < n; ++j) {
    P[j] = w[j] / W;
    if (PL_out) PL_out[j] = P[j];
  }

  /* --- backward --- */
  double a = 0.0, Dsum = 0.0;
  if (g) {
    for (int j = 0; j < n; ++j) Dsum += P[j] * g[j];
    double gmax = 0.0;
    for (int j = 0; j < n; ++j) gmax = fmax(gmax, gabs ? gabs[j] : fabs(g[j]));
    double amb_sum = 0.0;
    for (int j = 0; j < n; ++j) {
      const double gam = (g[j] - Dsum) / W;     /* dL/dw_j (App. B normalization Jacobian) */
      if (amb) amb[j] = 0.0;
      if (mode != KO_EXP_BF16 || mut == MUT_BF16_GRAD_UNROUNDED) {
        dS[j] = gam * de[j];
        continue;
      }
      double pos, alt;
      const double gb = round_signed(gam, BF16_MB, BF16_EMIN, &pos, &alt);   /* into the bf16 output */
      dS[j] = round_signed(gb * w[j], BF16_MB, BF16_EMIN, NULL, NULL);       /* exp's backward, in bf16 */
      if (amb) {
        /* a gradient computed in fp32 rounds the other way when it lies within its own error of a
           rounding midpoint: the change that would make, for the tolerance of a comparison */
        double lo, hi, pq;
        (void)round_fmt(fabs(gam), BF16_MB, BF16_EMIN, 0, &pq, &lo, &hi);
        const double ulp = hi - lo;
        const double band = 1e-5 * ((gabs ? gabs[j] : fabs(g[j])) + gmax) / W;
        if (fabs(pq - floor(pq) - 0.5) * ulp < band)
          amb[j] = fabs(round_signed(alt * w[j], BF16_MB, BF16_EMIN, NULL, NULL) - dS[j]);
        amb_sum += amb[j];
      }
    }
    const int keepM = cfg->grad == KO_FULL || cfg->grad == KO_MAX_ONLY;
    if (keepM) {
      for (int j = 0; j < n; ++j) a -= dS[j];   /* the row maximum's term: z = s - M */
      for (int j = 0; j < n; ++j)
        if (s[j] == M) {
          dS[j] += a / nA;
          if (amb) amb[j] += amb_sum / nA;
        }
    }
    if (cfg->grad == KO_P1) {
      double sum = 0.0;
      for (int j = 0; j < n; ++j) sum += dS[j];
      for (int j = 0; j < n; ++j) {
        dS[j] -= sum / n;
        if (amb) amb[j] += amb_sum / n;
      }
    }
  }
  if (z_out) for (int j = 0; j < n; ++j) {
    z_out[j] = s[j] - M; r_out[j] = 0; t_out[j] = 0.0; code_out[j] = code[j]; tail_out[j] = 0;
  }
  if (rowd) {
    rowd[RD_M] = M; rowd[RD_m] = m; rowd[RD_h] = 0.0; rowd[RD_WL] = W; rowd[RD_WN] = W;
    rowd[RD_a] = a; rowd[RD_b] = 0.0; rowd[RD_gapM] = M - belowM; rowd[RD_gapm] = abovem - m; rowd[RD_D] = Dsum;
    rowd[RD_tolM] = eb ? ebM + (ibelowM >= 0 ? eb[ibelowM] : 0.0) : 0.0;
    rowd[RD_tolm] = eb ? ebm + (iabovem >= 0 ? eb[iabovem] : 0.0) : 0.0;
  }
  if (rowi) {
    rowi[RI_amax] = amax; rowi[RI_amin] = amin; rowi[RI_nA] = nA; rowi[RI_nC] = nC; rowi[RI_degenerate] = 0;
    rowi[RI_amax2] = ibelowM; rowi[RI_amin2] = iabovem;
  }
  free(w); free(de); free(code);
}

/*
 * One attention row.  s[0..n) are the scaled scores of the row's visible keys,
 * g[0..n) the upstream gradient dL/dP_j (may be NULL: forward only).
 * Outputs P (forward probabilities), dS (score gradient, if g != NULL), and
 * optional per-key diagnostics.  row_id is used only for flag reporting.
 */
static void ko_row_impl(const ko_cfg_t *cfg, int n, const double *s, const double *g,
                        const uint8_t *flip, double *P, double *dS, double *PL_out,
                        double *u_out, int32_t *r_out, double *t_out, int32_t *ell_out, uint8_t *tail_out,
                        double *rowd, int32_t *rowi, int row_id, const int32_t *key_id, ko_flags_t *flags,
                        const double *eb, const double *gabs, double *amb) {
  if (cfg->recon >= KO_SOFTMAX && cfg->recon <= KO_EXP_FP8) {
    ko_row_exp(cfg, n, s, g, gabs, flip, P, dS, PL_out, u_out, r_out, t_out, ell_out, tail_out, rowd, rowi,
               row_id, key_id, flags, eb, amb);
    return;
  }
  const int K = cfg->K;
  const int mut = cfg->mutation;
  const int tailp = cfg->calib == KO_FWM ? cfg->tail : KO_TAIL_ZERO;
  const int binmean = cfg->recon == KO_BINMEAN || cfg->recon == KO_NEAREST_BINMEAN;
  const int nearest_bins = cfg->recon == KO_NEAREST || binmean;
  double *E = (double *)malloc(sizeof(double) * (K + 1));
  double *bgrid = (double *)malloc(sizeof(double) * (K + 1));
  double *u = (double *)malloc(sizeof(double) * n);
  double *t = (double *)malloc(sizeof(double) * n);
  double *wL = (double *)malloc(sizeof(double) * n);
  double *wN = (double *)malloc(sizeof(double) * n);
  double *Delta = (double *)malloc(sizeof(double) * n);
  double *gam = (double *)malloc(sizeof(double) * n);
  int *r = (int *)malloc(sizeof(int) * n);
  int *ell = (int *)malloc(sizeof(int) * n);
  uint8_t *tail = (uint8_t *)malloc(n);

  /* --- calibration (§3 Objects and calibration; App. A) --- */
  /* row extrema over the visible keys, and the sets of keys attaining them */
  double M = -INFINITY, m = INFINITY;
  for (int j = 0; j < n; ++j) {
    if (s[j] > M) M = s[j];
    if (s[j] < m) m = s[j];
  }
  int amax = -1, amin = -1, nA = 0, nC = 0;
  double belowM = -INFINITY, abovem = INFINITY;
  int ibelowM = -1, iabovem = -1;
  for (int j = 0; j < n; ++j) {
    if (s[j] == M) { if (amax < 0) amax = j; nA++; } else if (s[j] > belowM) { belowM = s[j]; ibelowM = j; }
    if (s[j] == m) { if (amin < 0) amin = j; nC++; } else if (s[j] < abovem) { abovem = s[j]; iabovem = j; }
  }
  /* rounding-error bounds of the extrema (0 without eb) */
  const double ebM = eb ? eb[amax] : 0.0, ebm = eb ? eb[amin] : 0.0;
  double h;
  int degenerate = 0;
  if (cfg->calib == KO_MINMAX) {
    /* MinMax: grid on the observed range, h = (M - m)/K, b_r = (1 - r/K)(m - M).
       Degenerate rows (M - m <= eps) use the safe width 1 before any division. */
    double span = M - m;
    degenerate = !(span > DEGENERATE_EPS);
    h = (degenerate && mut != MUT_NO_HSAFE) ? 1.0 : span / K;
    for (int q = 0; q <= K; ++q) bgrid[q] = (1.0 - (double)q / K) * (m - M);
  } else {
    /* FWM: fixed window [M - tau, M], h = tau/K, b_r = -tau + r h. */
    h = cfg->tau / K;
    for (int q = 0; q <= K; ++q)
      bgrid[q] = -cfg->tau + (mut == MUT_FWM_GRID_SHIFT ? q + 1 : q) * h;
  }
  for (int q = 0; q <= K; ++q) E[q] = exp(bgrid[q]);

  /* --- interval index and local position (§3) --- */
  for (int j = 0; j < n; ++j) {
    double uj;
    int tj = 0;
    if (cfg->calib == KO_MINMAX) {
      uj = (s[j] - m) / h;
    } else if (tailp == KO_TAIL_RESOLVED) {
      double z = s[j] - M;                                 /* the grid continues below -tau */
      uj = ((z > 0.0 ? 0.0 : z) + cfg->tau) / h;
    } else {
      double z = s[j] - M;
      tj = (mut == MUT_TAIL_INCLUSIVE) ? (z <= -cfg->tau) : (z < -cfg->tau);
      double zc = z < -cfg->tau ? -cfg->tau : (z > 0.0 ? 0.0 : z);   /* clip(z, -tau, 0) */
      uj = (zc + cfg->tau) / h;
    }
    if (flags) {
      /* guard in u units: the stated guard, or the rounding bound of u if larger */
      double gj = flags->guard;
      if (eb) {
        double eu = (cfg->calib == KO_MINMAX) ? (eb[j] + 2.0 * ebm + ebM) / h : (eb[j] + ebM) / h;
        if (eu > gj) gj = eu;
      }
      if (cfg->calib == KO_FWM && tailp != KO_TAIL_RESOLVED && fabs(s[j] - M + cfg->tau) / h < gj)
        flag_push(flags, row_id, key_id ? key_id[j] : j, FLIP_TAIL, fabs(s[j] - M + cfg->tau) / h);
      double kint = floor(uj + 0.5);
      /* interval boundaries: the integers 1..K-1, and every integer below K on the resolved grid */
      if ((tailp == KO_TAIL_RESOLVED || (K >= 2 && kint >= 1)) && kint <= K - 1 && fabs(uj - kint) < gj)
        flag_push(flags, row_id, key_id ? key_id[j] : j, FLIP_INTERVAL, fabs(uj - kint));
      double khalf = floor(uj) + 0.5;
      if (nearest_bins && khalf < K && fabs(uj - khalf) < gj)
        flag_push(flags, row_id, key_id ? key_id[j] : j, FLIP_NEAREST, fabs(uj - khalf));
    }
    int rj = (mut == MUT_INTERVAL_ROUND) ? (int)floor(uj + 0.5) : (int)floor(uj);
    if (rj < 0 && tailp != KO_TAIL_RESOLVED) rj = 0;
    if (rj > K - 1) rj = K - 1;
    double tt = uj - rj;
    if (tt < 0.0) tt = 0.0;
    if (tt > 1.0) tt = 1.0;
    uint8_t fl = flip ? flip[j] : 0;
    if (fl & FLIP_TAIL) {
      tj = !tj;
      if (!tj && uj > 0.0 && (s[j] - M) < -cfg->tau + 0.5 * h) { /* leaving the tail: onto the edge */
        uj = 0.0; rj = 0; tt = 0.0;
      }
      if (!tj && uj == 0.0) { rj = 0; tt = 0.0; }
      if (tj && tailp == KO_TAIL_FLOOR) { uj = 0.0; rj = 0; tt = 0.0; }   /* into the tail: floored */
    }
    if (fl & FLIP_INTERVAL) {
      int kint = (int)floor(uj + 0.5);
      if ((kint >= 1 || tailp == KO_TAIL_RESOLVED) && kint <= K - 1) {
        rj = (rj == kint) ? kint - 1 : kint;
        tt = uj - rj;
        if (tt < 0.0) tt = 0.0;
        if (tt > 1.0) tt = 1.0;
      }
    }
    int lj = rj + ((mut == MUT_NEAREST_STRICT) ? (tt > 0.5) : (tt >= 0.5));
    if (fl & FLIP_NEAREST) {
      int k2 = (int)floor(uj);
      if (k2 > K - 1) k2 = K - 1;
      lj = (lj == k2 + 1) ? k2 : k2 + 1;
    }
    u[j] = uj; r[j] = rj; t[j] = tt; ell[j] = lj; tail[j] = (uint8_t)tj;
  }

  /* --- reconstruction (§3 Reconstruction); a floored tail key sits on the window edge (u = 0) --- */
  for (int j = 0; j < n; ++j) {
    if (tail[j] && tailp == KO_TAIL_ZERO) { wL[j] = 0.0; wN[j] = 0.0; continue; }
    const double Er = grid_at(E, K, cfg->tau, h, r[j], mut), Er1 = grid_at(E, K, cfg->tau, h, r[j] + 1, mut);
    wL[j] = (1.0 - t[j]) * Er + t[j] * Er1;                 /* LERP between adjacent grid values */
    wN[j] = grid_at(E, K, cfg->tau, h, ell[j], mut);              /* Nearest grid centre */
  }

  /* --- normalization (§3) and strict hard forward (App. C.2 (iii)) --- */
  double WL = 0.0, WN = 0.0;
  for (int j = 0; j < n; ++j) { WL += wL[j]; WN += wN[j]; }
  int nearest_fwd = (cfg->recon == KO_NEAREST || cfg->recon == KO_NEAREST_BINMEAN) && (mut != MUT_NEAREST_FWD_LERP);
  for (int j = 0; j < n; ++j) {
    P[j] = nearest_fwd ? wN[j] / WN : wL[j] / WL;
    if (PL_out) PL_out[j] = (mut == MUT_DV_WITH_PL) ? wL[j] / WL : P[j];
  }

  double a = 0.0, b = 0.0, Dsum = 0.0;
  if (binmean) {
    /* --- bin-mean reconstruction (§5 and App. I: each bin's weight is the mean of exp over its
       members, so bin mass is conserved; its backward is the exact derivative, the bins held
       fixed).  Bins are the Nearest bins l = 0..K of the row's calibration; keys below an FWM
       window belong to none and weigh 0.  Under NEAREST_BINMEAN (App. I.3) the forward stays
       the strict Nearest one and only the backward is the bin mean's. --- */
    double *Sb = (double *)calloc(K + 1, sizeof(double)), *Gb = (double *)calloc(K + 1, sizeof(double));
    int *nb = (int *)calloc(K + 1, sizeof(int));
    double *ez = (double *)malloc(sizeof(double) * n);
    for (int j = 0; j < n; ++j) {
      ez[j] = tail[j] ? 0.0 : exp(s[j] - M);
      if (tail[j]) continue;
      Sb[ell[j]] += ez[j];
      nb[ell[j]] += 1;
      if (g) Gb[ell[j]] += g[j];
    }
    double WC = 0.0;
    for (int j = 0; j < n; ++j) {
      wL[j] = tail[j] ? 0.0 : (mut == MUT_BINMEAN_SUM ? Sb[ell[j]] : Sb[ell[j]] / nb[ell[j]]);
      WC += wL[j];
    }
    WL = WC;                                   /* the bin-mean normalizer, recorded as W^L */
    for (int j = 0; j < n; ++j) {
      if (cfg->recon == KO_BINMEAN) P[j] = wL[j] / WC;
      if (PL_out) PL_out[j] = P[j];            /* dV takes the forward's value */
    }
    if (g) {
      /* dL/ds_k = P^E_k (gbar_{B(k)} - sum_j P^C_j g_j) with P^E_k = e^{z_k} / W^C and gbar_B
         the mean of g over bin B: the upstream gradient replaced by its bin average */
      for (int j = 0; j < n; ++j) Dsum += wL[j] / WC * g[j];
      for (int j = 0; j < n; ++j) {
        if (tail[j]) { dS[j] = 0.0; continue; }
        const double gbar = mut == MUT_BINMEAN_OWN_G ? g[j] : Gb[ell[j]] / nb[ell[j]];
        dS[j] = ez[j] / WC * (gbar - Dsum);
        gam[j] = (g[j] - Dsum) / WC;
        Delta[j] = 0.0;
      }
      if (cfg->grad == KO_P1) {               /* the rows already sum to zero; kept for form */
        double sum = 0.0;
        for (int j = 0; j < n; ++j) sum += dS[j];
        for (int j = 0; j < n; ++j) dS[j] -= sum / n;
      }
    }
    free(Sb); free(Gb); free(nb); free(ez);
  } else if (g) {
    /* --- normalization Jacobian (App. B): gamma_j = (g_j - sum_i P_i g_i)/W,
       at (P^L, W^L) for LERP and Prob-STE, at (P^N, W^N) for Weight-STE --- */
    int use_lerp_point = (cfg->recon == KO_LERP) || (cfg->ste == KO_PROB_STE) || (mut == MUT_WSTE_USES_LERP);
    double Wg = use_lerp_point ? WL : WN;
    for (int j = 0; j < n; ++j) Dsum += (use_lerp_point ? wL[j] / WL : wN[j] / WN) * g[j];
    for (int j = 0; j < n; ++j) gam[j] = (mut == MUT_GAMMA_SIGN) ? (Dsum - g[j]) / Wg : (g[j] - Dsum) / Wg;

    /* --- LERP own-score slope (App. B): Delta_j = (e^{b_{r+1}} - e^{b_r})/h --- */
    for (int j = 0; j < n; ++j) {
      if (tail[j] && !(mut == MUT_FLOOR_TAIL_SLOPE && tailp == KO_TAIL_FLOOR)) {
        Delta[j] = 0.0;   /* zero tail: no weight; floor: a constant weight */
        continue;
      }
      const double dE = grid_at(E, K, cfg->tau, h, r[j] + 1, mut) - grid_at(E, K, cfg->tau, h, r[j], mut);
      Delta[j] = (mut == MUT_DELTA_TIMES_H) ? dE * h : dE / h;
      dS[j] = gam[j] * Delta[j];
    }
    for (int j = 0; j < n; ++j)
      if (tail[j] && !(mut == MUT_FLOOR_TAIL_SLOPE && tailp == KO_TAIL_FLOOR)) dS[j] = 0.0;

    /* --- calibration gradient through the row extrema (App. B); max_only / min_only keep
       one of its two channels --- */
    int keepM = cfg->grad == KO_FULL || cfg->grad == KO_MAX_ONLY || (cfg->grad == KO_DETACHED && mut == MUT_DETACH_KEEPS_M);
    int keepm = cfg->grad == KO_FULL || cfg->grad == KO_MIN_ONLY;
    if (mut == MUT_ONLY_SWAPPED && (cfg->grad == KO_MAX_ONLY || cfg->grad == KO_MIN_ONLY)) {
      int tmp = keepM; keepM = keepm; keepm = tmp;
    }
    if (keepM || keepm) {
      if (cfg->calib == KO_MINMAX) {
        for (int j = 0; j < n; ++j) {
          double rho = (r[j] + t[j]) / K;
          double X = mut == MUT_X_INDEX
                         ? ((1.0 - t[j]) * r[j] * E[r[j]] + t[j] * r[j] * E[r[j] + 1]) / K
                         : ((1.0 - t[j]) * r[j] * E[r[j]] + t[j] * (r[j] + 1) * E[r[j] + 1]) / K;
          double dM, dm;
          if (!degenerate) {              /* eq. (1), regular branch */
            dM = X - wL[j] - (mut == MUT_DROP_RHO_DELTA ? 0.0 : rho * Delta[j]);
            dm = wL[j] - X - (1.0 - rho) * Delta[j];
          } else {                        /* degenerate branch: h is a constant */
            dM = X - wL[j];
            dm = wL[j] - X - Delta[j];
          }
          if (mut == MUT_SIGN_DM) dm = -dm;
          a += gam[j] * dM;
          b += gam[j] * dm;
        }
      } else {
        /* FWM: in-window keys have dw/dM = -Delta, tail keys contribute nothing */
        for (int j = 0; j < n; ++j) if (!tail[j]) a += -gam[j] * Delta[j];
      }
      if (!keepM) a = 0.0;
      if (!keepm) b = 0.0;
      /* the extremum gradient is split evenly among tied keys */
      for (int j = 0; j < n; ++j) {
        if (s[j] == M) {
          if (mut == MUT_NO_TIE_SPLIT) { if (j == amax) dS[j] += a; }
          else dS[j] += a / nA;
        }
        if (cfg->calib == KO_MINMAX && s[j] == m) {
          if (mut == MUT_NO_TIE_SPLIT) { if (j == amin) dS[j] += b; }
          else dS[j] += b / nC;
        }
      }
    }
    /* --- P1 (App. B "Detach"): the detached row projected onto the zero-sum subspace by
       subtracting its mean over the row's visible keys --- */
    if (cfg->grad == KO_P1) {
      double sum = 0.0;
      for (int j = 0; j < n; ++j) sum += dS[j];
      const double mean = sum / n;
      for (int j = 0; j < n; ++j)
        if (!(mut == MUT_P1_SKIP_TAIL && tail[j])) dS[j] -= mean;
    }
  }

  if (u_out) for (int j = 0; j < n; ++j) {
    u_out[j] = u[j]; r_out[j] = r[j]; t_out[j] = t[j]; ell_out[j] = ell[j]; tail_out[j] = tail[j];
  }
  if (rowd) {
    rowd[RD_M] = M; rowd[RD_m] = m; rowd[RD_h] = h; rowd[RD_WL] = WL; rowd[RD_WN] = WN;
    rowd[RD_a] = a; rowd[RD_b] = b; rowd[RD_gapM] = M - belowM; rowd[RD_gapm] = abovem - m; rowd[RD_D] = Dsum;
    rowd[RD_tolM] = eb ? ebM + (ibelowM >= 0 ? eb[ibelowM] : 0.0) : 0.0;
    rowd[RD_tolm] = eb ? ebm + (iabovem >= 0 ? eb[iabovem] : 0.0) : 0.0;
  }
  if (rowi) {
    rowi[RI_amax] = amax; rowi[RI_amin] = amin; rowi[RI_nA] = nA; rowi[RI_nC] = nC; rowi[RI_degenerate] = degenerate;
    rowi[RI_amax2] = ibelowM; rowi[RI_amin2] = iabovem;   /* runner-up keys (-1 if none) */
  }
  free(E); free(bgrid); free(u); free(t); free(wL); free(wN); free(Delta); free(gam); free(r); free(ell); free(tail);
}

/* Row-level entry point (no flags).  g may be NULL for forward only. */
int ko_row(const ko_cfg_t *cfg, int n, const double *s, const double *g, const uint8_t *flip,
           double *P, double *dS, double *u, int32_t *r, double *t, int32_t *ell, uint8_t *tail,
           double *rowd, int32_t *rowi) {
  if (!cfg || n < 1 || cfg->K < 1 || !s || !P || (g && !dS)) return -1;
  if (cfg->calib == KO_FWM && !(cfg->tau > 0.0)) return -1;
  if (cfg->tail < KO_TAIL_ZERO || cfg->tail > KO_TAIL_RESOLVED || (cfg->calib == KO_MINMAX && cfg->tail != 0)) return -1;
  if (cfg->recon < KO_LERP || cfg->recon > KO_NEAREST_BINMEAN) return -1;
  if (cfg->recon >= KO_BINMEAN && cfg->tail != KO_TAIL_ZERO) return -1;   /* bin mean: zero tail only */
  if (u && !(r && t && ell && tail)) return -1;
  ko_row_impl(cfg, n, s, g, flip, P, dS, NULL, u, r, t, ell, tail, rowd, rowi, 0, NULL, NULL, NULL, NULL, NULL);
  return 0;
}

/*
 * One attention head: Q, K, V, dO are [T, D] row-major doubles.  Scores are
 * s_ij = scale * Q_i . K_j over the visible keys (j <= i when causal).
 * O = P V; dQ_i = scale * sum_j dS_ij K_j; dK_j = scale * sum_i dS_ij Q_i;
 * dV_j = sum_i P_ij dO_i.  dO may be NULL (forward only; dQ/dK/dV untouched).
 * flips: nflip triples (row, key, bits).  flags: optional near-boundary report.
 * bins: optional [T, T] decision map: Nearest index l (Nearest) or interval index r
 * (LERP) for visible keys, 254 for FWM tail keys, 255 for keys the query does not see.
 * row_mask: optional [T]; rows with 0 are skipped (their O, dQ rows stay 0 and they
 * add nothing to dK, dV), so a caller can get the contributions of chosen rows alone.
 * absout: optional [4, T, D]: the same sums with every term replaced by its absolute
 * value (sum_j P|V|, scale sum_j |dS||K|, scale sum_i |dS||Q|, sum_i P|dO|), the
 * scale against which cancellation in an output element is judged.
 * ambout: optional [2, T, D] (EXP_BF16 only, else zeros): scale sum_j A_ij |K_j| and
 * scale sum_i A_ij |Q_i|, where A_ij is how much dS_ij changes if its bfloat16 gradient
 * rounding goes the other way at a position where a gradient computed in fp32 may do so.
 * Exponential baselines: bins holds the E4M3 byte of the weight (EXP_FP8), the low byte
 * of the bfloat16 weight (EXP_BF16) or 0 (SOFTMAX) for visible keys.
 */
int ko_head(const ko_cfg_t *cfg, int T, int D, int causal, double scale,
            const double *Q, const double *Kt, const double *V, const double *dO,
            double *O, double *dQ, double *dK, double *dV, double *rowd, int32_t *rowi,
            int64_t nflip, const int32_t *flips,
            double guard, int64_t flag_cap, int32_t *flag_pos, double *flag_dist, int64_t *nflags,
            uint8_t *bins, const uint8_t *row_mask, double *absout, double *ambout, int nthreads) {
  if (!cfg || T < 1 || D < 1 || !Q || !Kt || !V || !O) return -1;
  if (dO && !(dQ && dK && dV)) return -1;
  if (cfg->K < 1 || (cfg->calib == KO_FWM && !(cfg->tau > 0.0))) return -1;
  if (cfg->tail < KO_TAIL_ZERO || cfg->tail > KO_TAIL_RESOLVED || (cfg->calib == KO_MINMAX && cfg->tail != 0)) return -1;
  if (cfg->recon < KO_LERP || cfg->recon > KO_NEAREST_BINMEAN) return -1;
  if (cfg->recon >= KO_BINMEAN && cfg->tail != KO_TAIL_ZERO) return -1;   /* bin mean: zero tail only */
  const int mut = cfg->mutation;
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
  double *absK = NULL, *absV = NULL;
  if (dO) {
    accK = (double *)calloc((size_t)nthreads * T * D, sizeof(double));
    accV = (double *)calloc((size_t)nthreads * T * D, sizeof(double));
    if (!accK || !accV) { free(accK); free(accV); return -2; }
    if (absout) {
      absK = (double *)calloc((size_t)nthreads * T * D, sizeof(double));
      absV = (double *)calloc((size_t)nthreads * T * D, sizeof(double));
      if (!absK || !absV) { free(accK); free(accV); free(absK); free(absV); return -2; }
    }
  }
  if (absout) memset(absout, 0, sizeof(double) * 4 * (size_t)T * D);
  double *ambK = NULL;
  if (ambout) memset(ambout, 0, sizeof(double) * 2 * (size_t)T * D);
  if (ambout && dO) {
    ambK = (double *)calloc((size_t)nthreads * T * D, sizeof(double));
    if (!ambK) { free(accK); free(accV); free(absK); free(absV); return -2; }
  }
  const double dq_scale = (mut == MUT_DQ_NO_SCALE) ? 1.0 : scale;

#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
#endif
  for (int i = 0; i < T; ++i) {
    if (row_mask && !row_mask[i]) continue;
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    int n = (causal && mut != MUT_EXTREMA_ALL_KEYS) ? i + 1 : T;
    double *s = (double *)malloc(sizeof(double) * n);
    double *g = dO ? (double *)malloc(sizeof(double) * n) : NULL;
    double *P = (double *)malloc(sizeof(double) * n);
    double *Pv = (double *)malloc(sizeof(double) * n);
    double *dS = dO ? (double *)malloc(sizeof(double) * n) : NULL;
    int32_t *kid = (int32_t *)malloc(sizeof(int32_t) * n);
    double *eb = (double *)malloc(sizeof(double) * n);
    double *gabs = dO ? (double *)malloc(sizeof(double) * n) : NULL;
    double *amb = (dO && ambout) ? (double *)calloc(n, sizeof(double)) : NULL;
    uint8_t *flip = NULL;
    for (int j = 0; j < n; ++j) {
      kid[j] = j;
      double acc = 0.0, aabs = 0.0;
      for (int k = 0; k < D; ++k) {
        acc += Q[(size_t)i * D + k] * Kt[(size_t)j * D + k];
        aabs += fabs(Q[(size_t)i * D + k] * Kt[(size_t)j * D + k]);
      }
      s[j] = scale * acc;
      /* one fp32 ulp of the score, 2^-23 |s|, plus the double accumulation's own bound */
      eb[j] = 1.1920928955078125e-07 * fabs(s[j]) + 1e-15 * fabs(scale) * aabs;
      if (dO) {
        double ga = 0.0, gb = 0.0;
        for (int k = 0; k < D; ++k) {
          ga += dO[(size_t)i * D + k] * V[(size_t)j * D + k];
          gb += fabs(dO[(size_t)i * D + k] * V[(size_t)j * D + k]);
        }
        g[j] = ga;
        gabs[j] = gb;
      }
    }
    for (int64_t f = 0; f < nflip; ++f) {
      if (flips[3 * f] == i && flips[3 * f + 1] >= 0 && flips[3 * f + 1] < n) {
        if (!flip) flip = (uint8_t *)calloc(n, 1);
        flip[flips[3 * f + 1]] |= (uint8_t)flips[3 * f + 2];
      }
    }
    double *du = NULL, *dt = NULL;
    int32_t *dr = NULL, *dl = NULL;
    uint8_t *dtail = NULL;
    if (bins) {
      du = (double *)malloc(sizeof(double) * n); dt = (double *)malloc(sizeof(double) * n);
      dr = (int32_t *)malloc(sizeof(int32_t) * n); dl = (int32_t *)malloc(sizeof(int32_t) * n);
      dtail = (uint8_t *)malloc(n);
    }
    ko_row_impl(cfg, n, s, g, flip, P, dS, Pv, du, dr, dt, dl, dtail,
                rowd ? rowd + (size_t)i * RD_N : NULL, rowi ? rowi + (size_t)i * RI_N : NULL, i, kid, fl, eb,
                gabs, amb);
    if (bins) {
      for (int j = 0; j < T; ++j) bins[(size_t)i * T + j] = 255;
      /* bin value: the index (interval r, or Nearest l); on the resolved FWM grid the index + 64,
         clamped below at 0 (indices below -64 share the value 0); 254 tail, 255 not visible */
      for (int j = 0; j < n && j < T; ++j) {
        int idx = (cfg->recon == KO_NEAREST || cfg->recon >= KO_SOFTMAX) ? dl[j] : dr[j];
        if (cfg->calib == KO_FWM && cfg->tail == KO_TAIL_RESOLVED) idx = idx < -64 ? 0 : idx + 64;
        bins[(size_t)i * T + j] = dtail[j] ? 254 : (uint8_t)idx;
      }
      free(du); free(dt); free(dr); free(dl); free(dtail);
    }
    if (mut == MUT_EXTREMA_ALL_KEYS && causal) {
      /* the planted mistake computed the extrema over all keys; keep the causal output shape */
      double Wsum = 0.0;
      for (int j = 0; j <= i; ++j) Wsum += P[j];
      for (int j = 0; j <= i; ++j) { P[j] /= Wsum; Pv[j] = P[j]; }
      n = i + 1;
    }
    /* O_i = sum_j P_ij V_j */
    for (int j = 0; j < n; ++j)
      for (int k = 0; k < D; ++k) O[(size_t)i * D + k] += P[j] * V[(size_t)j * D + k];
    if (absout)
      for (int j = 0; j < n; ++j)
        for (int k = 0; k < D; ++k) absout[(size_t)i * D + k] += P[j] * fabs(V[(size_t)j * D + k]);
    if (dO) {
      double *aK = accK + (size_t)tid * T * D, *aV = accV + (size_t)tid * T * D;
      for (int j = 0; j < n; ++j) {
        for (int k = 0; k < D; ++k) {
          dQ[(size_t)i * D + k] += dq_scale * dS[j] * Kt[(size_t)j * D + k];
          double src = (mut == MUT_DK_WITH_DO) ? dO[(size_t)i * D + k] : Q[(size_t)i * D + k];
          aK[(size_t)j * D + k] += scale * dS[j] * src;
          aV[(size_t)j * D + k] += Pv[j] * dO[(size_t)i * D + k];
        }
      }
      if (amb) {
        double *cK = ambK + (size_t)tid * T * D;
        for (int j = 0; j < n; ++j)
          for (int k = 0; k < D; ++k) {
            ambout[(size_t)i * D + k] += fabs(scale) * amb[j] * fabs(Kt[(size_t)j * D + k]);
            cK[(size_t)j * D + k] += fabs(scale) * amb[j] * fabs(Q[(size_t)i * D + k]);
          }
      }
      if (absout) {
        double *bK = absK + (size_t)tid * T * D, *bV = absV + (size_t)tid * T * D;
        double *bQ = absout + (size_t)T * D;
        for (int j = 0; j < n; ++j)
          for (int k = 0; k < D; ++k) {
            bQ[(size_t)i * D + k] += fabs(scale * dS[j] * Kt[(size_t)j * D + k]);
            bK[(size_t)j * D + k] += fabs(scale * dS[j] * Q[(size_t)i * D + k]);
            bV[(size_t)j * D + k] += fabs(Pv[j] * dO[(size_t)i * D + k]);
          }
      }
    }
    free(s); free(g); free(P); free(Pv); free(dS); free(kid); free(flip); free(eb); free(gabs); free(amb);
  }
  if (dO) {
    for (int th = 0; th < nthreads; ++th)
      for (size_t x = 0; x < (size_t)T * D; ++x) {
        dK[x] += accK[(size_t)th * T * D + x];
        dV[x] += accV[(size_t)th * T * D + x];
      }
    if (absout) {
      for (int th = 0; th < nthreads; ++th)
        for (size_t x = 0; x < (size_t)T * D; ++x) {
          absout[2 * (size_t)T * D + x] += absK[(size_t)th * T * D + x];
          absout[3 * (size_t)T * D + x] += absV[(size_t)th * T * D + x];
        }
    }
    if (ambout)
      for (int th = 0; th < nthreads; ++th)
        for (size_t x = 0; x < (size_t)T * D; ++x) ambout[(size_t)T * D + x] += ambK[(size_t)th * T * D + x];
    free(accK); free(accV); free(absK); free(absV); free(ambK);
  }
  if (nflags) *nflags = fl ? fl->count : 0;
  return 0;
}
