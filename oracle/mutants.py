"""Planted mistakes in the oracle, built as separate mutant libraries (test infrastructure).

Each entry names a plausible mistake and gives the exact source lines of kia_oracle.c it
replaces.  build_mutant(name) copies the source, applies the replacements (each original
line must occur exactly once, so the mutant changes the code the method really runs) and
compiles it to its own shared library.  The oracle's method functions carry no trace of
these mistakes; the tests load a mutant only to show that some pin catches it.
"""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kia_oracle.c")
_DIR = os.path.join(_HERE, "_mutants")

# name -> [(original, replacement), ...]
MUTANTS = {
    # dw/dM without the -rho*Delta term (eq. (1))
    "drop_rho_delta": [("dM = X - wL[j] - rho * Delta[j];", "dM = X - wL[j];")],
    # dw/dm with the wrong sign
    "sign_dm": [("dm = wL[j] - X - (1.0 - rho) * Delta[j];", "dm = -(wL[j] - X - (1.0 - rho) * Delta[j]);")],
    # secant slope multiplied by h instead of divided
    "delta_times_h": [("Delta[j] = dE / c->h;", "Delta[j] = dE * c->h;")],
    # Nearest rounds t = 1/2 down
    "nearest_strict": [("d->ell = r + (t >= 0.5);", "d->ell = r + (t > 0.5);")],
    # Weight-STE gamma taken at (P^L, W^L)
    "wste_uses_lerp": [("const int lerp_point = cfg->recon == KO_LERP || cfg->ste == KO_PROB_STE;",
                        "const int lerp_point = 1;")],
    # dK accumulates dO instead of Q
    "dk_with_do": [("aK[(size_t)j * D + k] += scale * dS[j] * Q[(size_t)i * D + k];",
                    "aK[(size_t)j * D + k] += scale * dS[j] * dO[(size_t)i * D + k];")],
    # FWM tail includes z = -tau
    "tail_inclusive": [("d->tail = z < -cfg->tau;", "d->tail = z <= -cfg->tau;")],
    # extremum gradient given whole to the first tied key
    "no_tie_split": [("if (inA[j]) dS[j] += a / x->nA;", "if (inA[j] && j == x->amax) dS[j] += a;")],
    # Nearest forward returns P^L
    "nearest_fwd_lerp": [("const int nearest_fwd = cfg->recon == KO_NEAREST || cfg->recon == KO_NEAREST_BINMEAN;",
                          "const int nearest_fwd = 0;")],
    # the causal set takes one key too many (j <= i + 1)
    "causal_off_by_one": [("const int n = causal ? i + 1 : T;", "const int n = causal ? (i + 2 < T ? i + 2 : T) : T;")],
    # dQ without the score scale
    "dq_no_scale": [("dQ[(size_t)i * D + k] += scale * dS[j] * Kt[(size_t)j * D + k];",
                     "dQ[(size_t)i * D + k] += dS[j] * Kt[(size_t)j * D + k];")],
    # degenerate rows divide by span/K
    "no_hsafe": [("c->h = c->degenerate ? 1.0 : span / K;", "c->h = span / K;")],
    # interval index by rounding instead of floor
    "interval_round": [("int r = (int)floor(d->u);", "int r = (int)floor(d->u + 0.5);")],
    # gamma = (D - g)/W
    "gamma_sign": [("for (int j = 0; j < n; ++j) gam[j] = (g[j] - Dsum) / Wg;",
                    "for (int j = 0; j < n; ++j) gam[j] = (Dsum - g[j]) / Wg;")],
    # Nearest dV uses P^L instead of the forward P^N
    "dv_with_pl": [("Pv[j] = P[j];                                          /* dV takes the forward value */",
                    "Pv[j] = wL[j] / WL;")],
    # FWM grid b_r = -tau + (r+1)h
    "fwm_grid_shift": [("for (int q = 0; q <= K; ++q) c->E[q] = exp(-cfg->tau + q * c->h);",
                        "for (int q = 0; q <= K; ++q) c->E[q] = exp(-cfg->tau + (q + 1) * c->h);")],
    # X uses r instead of r+1 in its second term
    "x_index": [("const double X = ((1.0 - t) * r * c->E[r] + t * (r + 1) * c->E[r + 1]) / K;",
                 "const double X = ((1.0 - t) * r * c->E[r] + t * r * c->E[r + 1]) / K;")],
    # detached mode keeps the M channel
    "detach_keeps_m": [("const int keepM = cfg->grad == KO_FULL || cfg->grad == KO_MAX_ONLY;",
                        "const int keepM = cfg->grad == KO_FULL || cfg->grad == KO_MAX_ONLY || cfg->grad == KO_DETACHED;")],
    # max_only keeps the m channel, min_only the M channel
    "only_swapped": [("const int keepM = cfg->grad == KO_FULL || cfg->grad == KO_MAX_ONLY;",
                      "const int keepM = cfg->grad == KO_FULL || cfg->grad == KO_MIN_ONLY;"),
                     ("const int keepm = cfg->grad == KO_FULL || cfg->grad == KO_MIN_ONLY;",
                      "const int keepm = cfg->grad == KO_FULL || cfg->grad == KO_MAX_ONLY;")],
    # P1 shifts only the keys inside the FWM window
    "p1_skip_tail": [("for (int j = 0; j < n; ++j) dS[j] -= mean;",
                      "for (int j = 0; j < n; ++j) if (!d[j].tail) dS[j] -= mean;")],
    # floored tail keys keep the slope of the first interval
    "floor_tail_slope": [("if (d[j].tail) { Delta[j] = 0.0; dS[j] = 0.0; continue; }",
                          "if (d[j].tail && tailp != KO_TAIL_FLOOR) { Delta[j] = 0.0; dS[j] = 0.0; continue; }")],
    # the resolved grid reads the table's end values below the window
    "resolved_grid_clamp": [("return exp(-cfg->tau + q * c->h);", "return c->E[q < 0 ? 0 : cfg->K];")],
    # FP8-rounded exp rounds toward zero
    "fp8_truncates": [("d->w = round_fmt(we, E4M3_MB, E4M3_EMIN, &pos, &lo, &hi);",
                       "(void)round_fmt(we, E4M3_MB, E4M3_EMIN, &pos, &lo, &hi); d->w = lo;")],
    # BF16-exp backward keeps the fp32 gradient (no bf16 casts)
    "bf16_grad_unrounded": [("if (cfg->recon == KO_EXP_BF16) dS[j] = round_signed(gb[j] * d[j].w, BF16_MB, BF16_EMIN, NULL, NULL);",
                             "if (cfg->recon == KO_EXP_BF16) dS[j] = gam[j] * d[j].w;")],
    # FP8-rounded exp backward uses the rounded weight as derivative
    "fp8_delta_rounded": [("d->de = we;", "d->de = d->w;")],
    # a bin weighs the sum of e^z over its members, not the mean
    "binmean_sum": [("wL[j] = d[j].tail ? 0.0 : Sb[d[j].ell] / nb[d[j].ell];   /* the bin's mean of e^z */",
                     "wL[j] = d[j].tail ? 0.0 : Sb[d[j].ell];")],
    # the bin-mean backward keeps each key's own upstream gradient
    "binmean_own_g": [("const double gbar = Gb[d[j].ell] / nb[d[j].ell];", "const double gbar = g[j];")],
}


def mutant_source(name: str, src: str | None = None) -> str:
    """The oracle's source with the named mistake planted; each original line must occur once."""
    text = open(_SRC).read() if src is None else src
    for old, new in MUTANTS[name]:
        count = text.count(old)
        if count != 1:
            raise ValueError(f"mutant {name!r}: the original line occurs {count} times in kia_oracle.c: {old!r}")
        text = text.replace(old, new)
    return text


def build_mutant(name: str) -> str:
    """Compile the mutant library (cached until kia_oracle.c changes); returns its path."""
    os.makedirs(_DIR, exist_ok=True)
    lib = os.path.join(_DIR, f"libkia_oracle_{name}.so")
    if os.path.exists(lib) and os.path.getmtime(lib) >= os.path.getmtime(_SRC) \
            and os.path.getmtime(lib) >= os.path.getmtime(__file__):
        return lib
    src = os.path.join(_DIR, f"kia_oracle_{name}.{os.getpid()}.c")
    with open(src, "w") as fh:
        fh.write(mutant_source(name))
    tmp = f"{lib}.{os.getpid()}.tmp"
    try:
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, lib)
    finally:
        if os.path.exists(src):
            os.remove(src)
    return lib
