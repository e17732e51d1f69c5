"""Pins of the oracle against what the pages and the mathematics fix.

Each pin takes an oracle configuration (possibly carrying a planted mutation)
and raises AssertionError when the oracle disagrees with:
  * float64 torch autograd of the literal forward definitions (independent
    derivation route for every backward term, including ties);
  * central finite differences of the oracle's own double forward (LERP, and
    dV for Nearest);
  * the zero-sum identity of the full calibration gradient and of the P1
    projection, and its violation under detached extrema (App. B, §5.1);
  * the channel decomposition g_full = g_self + g_M + g_m of the single-channel
    ablations (App. I);
  * the two-key softmax identity (App. B, Verification);
  * the interpolation bounds of a chord of exp and the K -> infinity limit;
  * brute-force nearest grid centre in score coordinates;
  * shift invariance of the output (and of dQ for the full gradient);
  * degenerate rows, causal row 0, V = 1, tied extrema, K = 1 affine LERP;
  * the hand-derived fixtures in tests/golden/;
  * for the FWM tail policies (App. C.3, App. D.4): floored tail keys weigh e^{-tau}
    and carry no gradient, moving them deeper changes nothing; the resolved grid
    keeps every key within the chord and nearest-centre bounds of e^z and
    converges to softmax as h -> 0 even with a narrow window;
  * for the exponential baselines (App. B "Softmax", App. D.5): torch's native
    autograd through its own bfloat16 / float8_e4m3fn casts, the textbook softmax
    gradient, the E4M3 value set (56 nonzero values in (0, 1], underflow below
    2^-10) and the rounding of each weight to its format.
Source: "Pretraining Transformers with Quantized Softmax in Attention", §3,
§5.1, App. A, App. B, App. C.2, App. C.3, App. D.4, App. D.5.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

import autograd_ref as AR
import golden_io
from oracle import oracle as ORC

VARIANTS = [(c, r, s, g) for c in ("minmax", "fwm") for r in ("lerp", "nearest")
            for s in ("weight", "prob") for g in ("full", "detached")]
# the range_grad ablations (App. I single-channel modes, App. B P1 projection)
VARIANTS += [(c, r, s, g) for c in ("minmax", "fwm") for (r, s) in (("lerp", "prob"), ("nearest", "weight"),
             ("nearest", "prob")) for g in ("max_only", "min_only", "p1")]
# the FWM tail policies (App. D.4: the tau-floor variant, also the floor tail of the App. C.3
# tau-selection stages, and the resolved grid)
VARIANTS += [("fwm", r, s, g, tp) for tp in ("floor", "resolved") for (r, s) in (("lerp", "prob"),
             ("nearest", "weight"), ("nearest", "prob")) for g in ("full", "detached")]
# the exponential baselines (App. B "Softmax", App. D.5): no grid; calib, K, tau and ste are ignored
EXP_RECON = ("softmax", "exp_bf16", "exp_fp8")
VARIANTS += [("fwm", r, "prob", g) for r in EXP_RECON for g in ("full", "detached", "max_only", "min_only", "p1")]
# bin-mean reconstruction and the Nearest-forward / bin-mean-backward hybrid (§5, App. I)
BINMEAN = ("binmean", "nearest_binmean")
VARIANTS += [(c, r, "prob", g) for c in ("minmax", "fwm") for r in BINMEAN for g in ("full", "detached", "p1")]


def is_exp(cfg):
    return cfg.recon in EXP_RECON


def max_only_calib(cfg):
    """FWM and the exponential baselines calibrate on the row maximum alone."""
    return cfg.calib == "fwm" or is_exp(cfg)


def zero_sum_mode(cfg):
    """Modes whose row score gradients sum to zero: full, P1, and max_only where there is no
    minimum channel (FWM, the exponential baselines: max_only is their full gradient); every
    mode of softmax."""
    if cfg.recon in ("softmax",) + BINMEAN:
        return True   # no extremum term: shift invariant in every mode
    return cfg.grad in ("full", "p1") or (max_only_calib(cfg) and cfg.grad == "max_only")


def _fmt_pos(x, mb, emin):
    """|x| in units of the spacing of a binary format with mb significand bits (smallest normal
    exponent emin) at |x|, and its distance from a rounding midpoint, in those units."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(x)
    E = np.maximum(e - 1, emin)
    q = x / np.ldexp(1.0, E - mb)
    return q, np.abs(q - np.floor(q) - 0.5)


def _exp_near(s, g, res, cfg, guard=1e-4):
    """True when a rounding of an exponential baseline lies within guard (in units of the target
    format's spacing) of a midpoint: there the fp32 steps of torch's casts may round the other way."""
    z = s - s.max()
    if cfg.recon == "exp_fp8":
        return bool((_fmt_pos(np.exp(z), 3, -6)[1] < guard).any())
    if cfg.recon != "exp_bf16":
        return False
    q, d = _fmt_pos(z, 7, -126)
    zb = np.copysign(np.rint(q) * np.ldexp(1.0, np.maximum(np.frexp(np.abs(z))[1] - 1, -126) - 7), z)
    bad = (d < guard) & (z != 0)
    bad |= _fmt_pos(np.exp(zb), 7, -126)[1] < guard
    if g is not None:
        gam = (g - (res["P"] * g).sum()) / res["WL"]
        bad |= _fmt_pos(gam, 7, -126)[1] < guard
    return bool(bad.any())


def cfg_of(calib, recon, ste, grad, tail="zero", K=4, tau=8.0, mutation=None):
    # the pins check the method in exact arithmetic: double scores, not rounded to fp32
    return ORC.OracleConfig(calib, recon, ste, grad, K, tau, mutation, tail, score_fp32=False)


def _resolved(cfg):
    return cfg.calib == "fwm" and cfg.tail == "resolved"


def _tail_mask(cfg, z):
    """Keys the policy truncates or floors: z < -tau under the zero and floor FWM policies."""
    if cfg.calib != "fwm" or cfg.tail == "resolved":
        return np.zeros_like(z, dtype=bool)
    return z < -cfg.tau


def _ar(cfg):
    return (cfg.calib, cfg.recon, cfg.ste, cfg.grad, cfg.K, cfg.tau)


def _near_boundary(res, cfg, guard=1e-6):
    u = res["u"]
    near_int = np.abs(u - np.round(u)) < guard
    near_half = np.abs(u - (np.floor(u) + 0.5)) < guard
    interior = (np.round(u) <= cfg.K - 1) & ((np.round(u) >= 1) | _resolved(cfg))
    bad = (near_int & interior) | near_half
    return bool(bad.any())


def _random_rows(seed, cfg, count=24):
    """Random rows (n in 2..40) at several score scales, away from bin boundaries."""
    rng = np.random.default_rng(seed)
    rows = []
    scales = (0.7, 2.5, 6.0) if cfg.calib == "minmax" else (1.0, 3.0, 7.0)
    tries = 0
    while len(rows) < count and tries < 10 * count:
        tries += 1
        n = int(rng.integers(2, 41))
        s = rng.standard_normal(n) * scales[len(rows) % 3]
        g = rng.standard_normal(n)
        res = ORC.row(dataclasses.replace(cfg, mutation=None), s, g)
        if is_exp(cfg):
            if _exp_near(s, g, res, cfg):
                continue
        else:
            if _near_boundary(res, cfg):
                continue
            if cfg.calib == "fwm" and np.any(np.abs(s - s.max() + cfg.tau) < 1e-6):
                continue
        rows.append((s, g))
    return rows


def _close(a, b, rtol, atol, what):
    a = np.asarray(a, dtype=np.float64); b = np.asarray(b, dtype=np.float64)
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    if not np.all(err <= lim) or not np.all(np.isfinite(a)):
        i = int(np.argmax(err - lim))
        raise AssertionError(f"{what}: max excess at {i}: got {a.flat[i]!r}, want {b.flat[i]!r}")


# ----------------------------------------------------------------------------- pins

def pin_autograd_rows(cfg):
    for s, g in _random_rows(11, cfg):
        res = ORC.row(cfg, s, g)
        P, dS = AR.row_grad(s, g, *_ar(cfg), tail_policy=cfg.tail)
        _close(res["P"], P.numpy(), 1e-12, 1e-14, "row P vs autograd")
        _close(res["dS"], dS.numpy(), 1e-9, 1e-12, "row dS vs autograd")


def pin_autograd_ties(cfg):
    rng = np.random.default_rng(5)
    for n in (5, 9, 17):
        s = rng.standard_normal(n) * 2.0
        s[1] = s[3] = s.max() + 0.75        # tied maxima
        s[0] = s[2] = s.min() - 0.4         # tied minima
        if cfg.calib == "fwm":
            s[0] = s[2] = s.max() - 0.6 * cfg.tau   # keep both in the window
        g = rng.standard_normal(n)
        res = ORC.row(dataclasses.replace(cfg, mutation=None), s, g)
        if _exp_near(s, g, res, cfg) if is_exp(cfg) else _near_boundary(res, cfg):
            continue
        res = ORC.row(cfg, s, g)
        P, dS = AR.row_grad(s, g, *_ar(cfg), tail_policy=cfg.tail)
        _close(res["P"], P.numpy(), 1e-12, 1e-14, "tied row P vs autograd")
        _close(res["dS"], dS.numpy(), 1e-9, 1e-12, "tied row dS vs autograd")


def _head_inputs(seed, T, D, qscale=1.0):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((T, D)) * qscale
    K = rng.standard_normal((T, D))
    V = rng.standard_normal((T, D))
    dO = rng.standard_normal((T, D))
    return Q, K, V, dO


def pin_autograd_head(cfg):
    for seed, T, D, causal, qs in ((1, 24, 8, True, 1.5), (2, 10, 6, False, 3.0), (3, 33, 4, True, 4.0)):
        Q, K, V, dO = _head_inputs(seed, T, D, qs)
        if is_exp(cfg) and ORC.head(dataclasses.replace(cfg, mutation=None), Q, K, V, dO, causal=causal,
                                    guard=1e-4, flag_cap=64, nthreads=2)["nflags"]:
            continue
        res = ORC.head(cfg, Q, K, V, dO, causal=causal, nthreads=2)
        O, dQ, dK, dV = AR.head_grad(Q, K, V, dO, *_ar(cfg), causal=causal, tail_policy=cfg.tail)
        _close(res["O"], O.numpy(), 1e-11, 1e-13, "head O vs autograd")
        _close(res["dV"], dV.numpy(), 1e-10, 1e-12, "head dV vs autograd")
        _close(res["dQ"], dQ.numpy(), 1e-8, 1e-11, "head dQ vs autograd")
        _close(res["dK"], dK.numpy(), 1e-8, 1e-11, "head dK vs autograd")


def pin_zero_sum(cfg):
    """Full gradient and P1: every row's score gradient sums to zero; detached and the
    single-channel modes (other than FWM's max_only): it does not."""
    nonzero = 0
    rows = _random_rows(23, cfg)
    for s, g in rows:
        res = ORC.row(cfg, s, g)
        tot, mag = abs(res["dS"].sum()), np.abs(res["dS"]).sum()
        if zero_sum_mode(cfg):
            # rounding of O(1) terms: an absolute 1e-15 besides the relative bound (a row's
            # gradient can be tiny when its bins average the upstream gradient away)
            assert tot <= 1e-12 * mag + 1e-15, f"zero-sum violated: {tot} vs {mag}"
        elif tot > 1e-6 * mag:
            nonzero += 1
    if not zero_sum_mode(cfg):
        assert nonzero >= len(rows) // 2, f"{cfg.grad} gradient unexpectedly zero-sum"


def pin_channel_additivity(cfg):
    """App. I: g_full = g_self + g_M + g_m, g_max_only = g_self + g_M, g_min_only = g_self + g_m,
    so max_only + min_only - detached = full; FWM has no g_m: max_only = full, min_only = detached."""
    if cfg.grad not in ("max_only", "min_only"):
        return
    other = {"max_only": "min_only", "min_only": "max_only"}[cfg.grad]
    for s, g in _random_rows(29, cfg, count=12):
        got = ORC.row(cfg, s, g)["dS"]
        oth = ORC.row(dataclasses.replace(cfg, grad=other), s, g)["dS"]
        det = ORC.row(dataclasses.replace(cfg, grad="detached", mutation=None), s, g)["dS"]
        full = ORC.row(dataclasses.replace(cfg, grad="full", mutation=None), s, g)["dS"]
        if not max_only_calib(cfg):
            _close(got + oth - det, full, 1e-12, 1e-14, "max_only + min_only - detached vs full")
        else:
            _close(got, full if cfg.grad == "max_only" else det, 1e-14, 0.0, f"FWM {cfg.grad}")


def pin_two_key(cfg):
    """MinMax with two keys reproduces softmax and, with full gradients, its gradient."""
    if cfg.calib != "minmax":
        return
    rng = np.random.default_rng(7)
    for _ in range(12):
        s = rng.standard_normal(2) * 3.0
        g = rng.standard_normal(2)
        res = ORC.row(cfg, s, g)
        e = np.exp(s - s.max())
        Pe = e / e.sum()
        _close(res["P"], Pe, 1e-14, 1e-15, "two-key P vs softmax")
        if cfg.grad == "full":
            _close(res["dS"], Pe * (g - (Pe * g).sum()), 1e-12, 1e-15, "two-key dS vs softmax gradient")


def _weights(res, recon):
    return res["P"] * (res["WL"] if recon == "lerp" else res["WN"])


def pin_reconstruction_bounds(cfg):
    """LERP is a chord of the convex e^z: above it, by at most h^2/8 e^{z+h};
    Nearest picks a grid value within h/2 of z in score coordinates."""
    if is_exp(cfg) or cfg.recon == "binmean":   # bin means: pin_binmean
        return
    for s, g in _random_rows(31, cfg):
        res = ORC.row(cfg, s, g)
        if res["degenerate"]:
            continue
        z = s - res["M"]
        w = _weights(res, cfg.recon)
        h = res["h"]
        tail = _tail_mask(cfg, z)
        if cfg.tail == "floor":
            _close(w[tail], np.full(int(tail.sum()), math.exp(-cfg.tau)), 1e-14, 0.0, "floored tail weight")
        else:
            assert np.all(w[tail] == 0.0), "tail weight not zero"
        assert np.array_equal(res["tail"].astype(bool), tail), "tail flags"
        win = ~tail
        if cfg.recon == "lerp":
            ez = np.exp(z[win])
            assert np.all(w[win] >= ez * (1 - 1e-12)), "LERP below exp"
            assert np.all(w[win] - ez <= (h * h / 8.0) * np.exp(z[win] + h) * (1 + 1e-9) + 1e-300), \
                "LERP chord error above h^2/8 bound"
        else:
            assert np.all(np.abs(np.log(w[win]) - z[win]) <= 0.5 * h * (1 + 1e-9) + 1e-12), \
                "Nearest weight farther than h/2 from e^z"


def pin_nearest_brute_force(cfg):
    """The Nearest index is the grid point closest to z (ties upward), found by brute force."""
    if is_exp(cfg):
        return
    for s, g in _random_rows(41, cfg):
        res = ORC.row(cfg, s, g)
        if res["degenerate"]:
            continue
        M, m = s.max(), s.min()
        K = cfg.K
        if cfg.calib == "minmax":
            grid = m + np.arange(K + 1) * (M - m) / K
        else:
            lowest = -int(np.ceil((M - m) / (cfg.tau / K))) - 2 if _resolved(cfg) else 0
            q = np.arange(lowest, K + 1)
            grid = M - cfg.tau + q * (cfg.tau / K)
        for j in range(len(s)):
            if _tail_mask(cfg, np.array([s[j] - M]))[0]:
                assert cfg.tail != "floor" or res["ell"][j] == 0, "floored tail key not at grid point 0"
                continue
            d = np.abs(s[j] - grid)
            best = np.flatnonzero(d <= d.min() * (1 + 1e-12) + 1e-15)
            want = best.max() + (lowest if cfg.calib == "fwm" else 0)
            assert res["ell"][j] == want, f"nearest index {res['ell'][j]} vs brute force {want}"


def pin_finite_differences(cfg):
    """Central differences of the double forward: LERP full gradient in Q, K, V; dV for every variant."""
    Q, K, V, dO = _head_inputs(13, 12, 6, 2.0)
    base = ORC.head(cfg, Q, K, V, dO, nthreads=1)
    clean = ORC.head(dataclasses.replace(cfg, mutation=None), Q, K, V, dO, guard=1e-4, flag_cap=64, nthreads=1)
    if clean["nflags"]:
        return
    rng = np.random.default_rng(3)
    eps = 1e-6

    def loss(Qx, Kx, Vx):
        return float((ORC.head(cfg, Qx, Kx, Vx, None, nthreads=1)["O"] * dO).sum())

    targets = [("V", "dV")]
    if cfg.recon in ("lerp", "softmax", "binmean") and cfg.grad == "full":
        targets += [("Q", "dQ"), ("K", "dK")]
    for name, gname in targets:
        for _ in range(8):
            i, k = int(rng.integers(0, 12)), int(rng.integers(0, 6))
            arrs = {"Q": Q.copy(), "K": K.copy(), "V": V.copy()}
            arrs[name][i, k] += eps
            lp = loss(arrs["Q"], arrs["K"], arrs["V"])
            arrs[name][i, k] -= 2 * eps
            lm = loss(arrs["Q"], arrs["K"], arrs["V"])
            fd = (lp - lm) / (2 * eps)
            an = base[gname][i, k]
            assert abs(fd - an) <= 2e-7 * max(1.0, abs(an)), f"finite difference {name}[{i},{k}]: {fd} vs {an}"


def pin_shift_invariance(cfg):
    """K_j -> K_j + v adds a per-row constant to the scores: O, dK, dV unchanged;
    dQ unchanged exactly when the row gradients sum to zero (full mode)."""
    Q, K, V, dO = _head_inputs(17, 16, 8, 1.5)
    v = np.random.default_rng(4).standard_normal(8) * 0.5
    a = ORC.head(cfg, Q, K, V, dO, nthreads=1)
    b = ORC.head(cfg, Q, K + v, V, dO, nthreads=1)
    fl = ORC.head(dataclasses.replace(cfg, mutation=None), Q, K, V, dO, guard=1e-6, flag_cap=64, nthreads=1)
    if fl["nflags"]:
        return
    _close(b["O"], a["O"], 1e-10, 1e-12, "O under key shift")
    _close(b["dV"], a["dV"], 1e-10, 1e-12, "dV under key shift")
    _close(b["dK"], a["dK"], 1e-8, 1e-11, "dK under key shift")
    if zero_sum_mode(cfg):
        _close(b["dQ"], a["dQ"], 1e-8, 1e-11, "dQ under key shift (zero-sum rows)")
    else:
        assert np.max(np.abs(b["dQ"] - a["dQ"])) > 1e-8, f"{cfg.grad} dQ unexpectedly shift-invariant"


def pin_degenerate_and_causal_edges(cfg):
    """All-equal scores: uniform P; MinMax gradient exactly zero.  Causal row 0 (one
    key): O_0 = V_0 and dQ_0 = 0.  V = 1 gives O = 1."""
    for n in (1, 3, 8):
        s = np.full(n, 0.8125)
        g = np.random.default_rng(n).standard_normal(n)
        res = ORC.row(cfg, s, g)
        _close(res["P"], np.full(n, 1.0 / n), 1e-15, 0.0, "degenerate P")
        if cfg.calib == "minmax":
            assert np.all(np.abs(res["dS"]) <= 1e-15), "degenerate MinMax row has a gradient"
        assert abs(res["dS"].sum()) <= 1e-15 or not zero_sum_mode(cfg), "degenerate row not zero-sum"
    Q, K, V, dO = _head_inputs(19, 9, 5, 2.0)
    r = ORC.head(cfg, Q, K, V, dO, nthreads=1)
    assert np.array_equal(r["O"][0], V[0]), "causal row 0 must return V_0"
    assert np.all(r["dQ"][0] == 0.0), "causal row 0 has a query gradient"
    r1 = ORC.head(cfg, Q, K, np.ones_like(V), dO, nthreads=1)
    _close(r1["O"], np.ones_like(V), 1e-14, 0.0, "V = 1 must give O = 1")


def pin_special_cases(cfg):
    """w at the argmax is e^0 = 1; MinMax w at the argmin is e^{m-M}; sum P = 1;
    the STE flag does not change LERP; K = 1 LERP is affine in s."""
    for s, g in _random_rows(53, cfg, count=10):
        res = ORC.row(cfg, s, g)
        w = _weights(res, cfg.recon)
        assert abs(res["P"].sum() - 1.0) <= 1e-14, "probabilities do not sum to 1"
        if cfg.recon == "binmean":
            continue   # the arg-max key's bin is averaged; pin_binmean covers it
        assert abs(w[res["amax"]] - 1.0) <= 1e-14, "weight at the argmax is not 1"
        if cfg.calib == "minmax":
            assert abs(w[res["amin"]] - math.exp(res["m"] - res["M"])) <= 1e-14, "weight at the argmin"
        if cfg.recon == "lerp" or is_exp(cfg):
            other = dataclasses.replace(cfg, ste="weight" if cfg.ste == "prob" else "prob")
            assert np.array_equal(ORC.row(other, s, g)["dS"], res["dS"]), "STE flag changed LERP"
    if cfg.calib == "minmax" and cfg.recon == "lerp":
        c1 = dataclasses.replace(cfg, K=1)
        s = np.random.default_rng(2).standard_normal(15) * 2.0
        res = ORC.row(c1, s)
        M, m = s.max(), s.min()
        want = math.exp(m - M) + (s - m) / (M - m) * (1.0 - math.exp(m - M))
        _close(res["P"] * res["WL"], want, 1e-13, 1e-15, "K=1 LERP is affine in s")


def pin_k_limit(cfg):
    """LERP -> softmax as K grows: forward error O(h^2), gradient error O(h) (full)."""
    if is_exp(cfg):
        return
    if cfg.recon != "lerp":
        return
    rng = np.random.default_rng(61)
    s = rng.standard_normal(48) * 2.0
    g = rng.standard_normal(48)
    e = np.exp(s - s.max()); Pe = e / e.sum()
    dSe = Pe * (g - (Pe * g).sum())
    # the resolved grid is never truncated, so a narrow window converges too
    tau = 1.0 if _resolved(cfg) else float(s.max() - s.min() + 1.0)
    errs, gerrs = [], []
    for K in (16, 64, 256):
        res = ORC.row(dataclasses.replace(cfg, K=K, tau=tau), s, g)
        errs.append(np.max(np.abs(res["P"] - Pe)))
        gerrs.append(np.max(np.abs(res["dS"] - dSe)))
    assert errs[2] < errs[0] / 100.0 and errs[2] < 1e-4, f"LERP forward not converging: {errs}"
    if cfg.grad == "full":
        assert gerrs[2] < gerrs[0] / 6.0 and gerrs[2] < 5e-3, f"LERP gradient not converging: {gerrs}"


def pin_golden(cfg):
    """Hand-derived fixtures (tests/golden/hand_rows.txt)."""
    if is_exp(cfg):
        return
    for case in golden_io.load_cases():
        if case["calib"] != cfg.calib or case.get("tail_policy", "zero") != cfg.tail:
            continue
        if (case.get("recon") == "binmean") != (cfg.recon == "binmean"):
            continue
        c = dataclasses.replace(cfg, K=int(case["K"]), tau=float(case.get("tau", cfg.tau)))
        s = np.array(case["s"], dtype=np.float64)
        g = np.linspace(-1.0, 1.0, len(s))
        res = ORC.row(c, s, g)
        name = case["case"]
        _close(res["u"], case["u"], 0.0, 1e-15, f"{name}: u")
        assert list(res["r"]) == [int(x) for x in case["r"]], f"{name}: r"
        _close(res["t"], case["t"], 0.0, 1e-15, f"{name}: t")
        assert list(res["tail"].astype(int)) == [int(x) for x in case["tail"]], f"{name}: tail"
        if c.recon != "lerp":
            assert list(res["ell"]) == [int(x) for x in case["ell"]], f"{name}: ell"
        w = np.array(case["wC"] if c.recon == "binmean" else case["wL" if c.recon == "lerp" else "wN"])
        _close(res["P"], w / w.sum(), 1e-14, 1e-16, f"{name}: P")
        for key in ("M", "m", "h"):
            assert abs(res[key] - case[key]) <= 1e-15, f"{name}: {key}"
        for key in ("nA", "nC", "degenerate"):
            assert res[key] == int(case[key]), f"{name}: {key}"


def pin_tail_policy(cfg):
    """Floor: a tail key weighs e^{-tau}, has no score gradient, and lowering it further changes
    nothing.  Resolved: nothing is truncated, and a key's weight keeps following e^z below the
    window (LERP within the chord bound, so deeper keys weigh less).  Zero: tail keys weigh 0."""
    if is_exp(cfg):
        return
    if cfg.calib != "fwm":
        return
    rng = np.random.default_rng(71)
    for n in (6, 13, 29):
        s = rng.standard_normal(n) * 2.0
        h = cfg.tau / cfg.K
        s[1] = s.max() - cfg.tau - 1.3 * h    # one key below the window
        s[2] = s.max() - cfg.tau - 3.4 * h    # one further below
        g = rng.standard_normal(n)
        if _near_boundary(ORC.row(dataclasses.replace(cfg, mutation=None), s, g), cfg):
            continue
        res = ORC.row(cfg, s, g)
        w = _weights(res, cfg.recon)
        if cfg.tail == "floor":
            assert res["tail"][1] and res["tail"][2], "keys below the window not flagged"
            assert w[1] == w[2], "floored tail keys weigh differently"
            assert res["dS"][1] == 0.0 or cfg.grad == "p1", "floored tail key has a gradient"
            s2 = s.copy(); s2[1] -= 5.0
            res2 = ORC.row(cfg, s2, g)
            _close(res2["P"], res["P"], 1e-15, 0.0, "floor: P moved with a tail key")
            _close(res2["dS"], res["dS"], 1e-14, 1e-16, "floor: dS moved with a tail key")
        elif cfg.tail == "resolved":
            assert not res["tail"].any(), "the resolved grid flagged a tail key"
            assert w[2] < w[1] < math.exp(-cfg.tau), "resolved weights do not decrease below the window"
            assert res["r"][1] < 0 and res["r"][2] < res["r"][1], "resolved intervals below the window"
            if cfg.recon == "lerp":
                assert res["dS"][1] != 0.0 and res["dS"][2] != 0.0, "resolved key below the window lacks a slope"
        else:
            assert w[1] == 0.0 and w[2] == 0.0, "zero-policy tail keys weigh something"


def pin_exp_weights(cfg):
    """Exponential baselines: softmax is e^z / sum and its gradient P (g - sum P g) (App. B
    "Softmax"); the FP8 weight is the E4M3 value nearest e^z, one of the format's 56 nonzero values
    in (0, 1] (or 0 below 2^-10), with the unrounded e^z as derivative; the BF16 weight is the
    bfloat16 value nearest exp of the bfloat16 value nearest z (App. D.5 "Definitions")."""
    if not is_exp(cfg):
        return
    # the E4M3 values in (0, 1]: 7 subnormal multiples of 2^-9 and 8 normal values per binade 2^-6 .. 2^-1, plus 1
    e4m3 = sorted({m * 2.0 ** -9 for m in range(1, 8)} | {(1 + f / 8) * 2.0 ** e for e in range(-6, 0) for f in range(8)}
                  | {1.0})
    assert len(e4m3) == 56
    grid = np.array([0.0] + e4m3)
    for s, g in _random_rows(83, cfg):
        res = ORC.row(cfg, s, g)
        z = s - s.max()
        w = res["P"] * res["WL"]
        if cfg.recon == "softmax":
            e = np.exp(z)
            _close(res["P"], e / e.sum(), 1e-14, 1e-16, "softmax P")
            if cfg.grad in ("full", "max_only"):
                P = e / e.sum()
                _close(res["dS"], P * (g - (P * g).sum()), 1e-12, 1e-15, "softmax gradient")
        elif cfg.recon == "exp_fp8":
            e = np.exp(z)
            nearest = grid[np.argmin(np.abs(grid[None, :] - e[:, None]), axis=1)]
            _close(w, nearest, 1e-13, 0.0, "E4M3 weight is the nearest representable value")
            assert np.all((w == 0) == (e < 2.0 ** -10)), "E4M3 underflow threshold"
            if cfg.grad == "detached":
                gam = (g - (res["P"] * g).sum()) / res["WL"]
                _close(res["dS"], gam * e, 1e-12, 1e-15, "FP8 derivative is the unrounded e^z")
        else:
            zb = np.array([float(torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)) for x in z])
            assert np.all(np.abs(zb - z) <= np.abs(z) * 2.0 ** -8), "bfloat16 input rounding"
            wb = np.exp(zb)
            assert np.all(np.abs(w - wb) <= wb * 2.0 ** -8), "bfloat16 output rounding"
            bits = np.array([np.float32(x).view(np.uint32) for x in w])
            assert np.all(bits & 0xFFFF == 0), "weights are bfloat16 values"


def pin_binmean(cfg):
    """Bin mean (§5, App. I): every in-window key of a bin weighs the mean of e^z over the bin,
    so bin mass is conserved (sum_j w^C_j = sum_j e^{z_j}); with every bin a singleton it is
    softmax; its score gradient divided by e^{z_k}/W^C is constant within a bin (the upstream
    gradient replaced by its bin average).  The hybrid (App. I.3) has the strict Nearest forward
    bit for bit and the bin mean's backward bit for bit."""
    if cfg.recon not in BINMEAN:
        return
    for s, g in _random_rows(97, cfg, count=12):
        res = ORC.row(cfg, s, g)
        bm = ORC.row(dataclasses.replace(cfg, recon="binmean"), s, g)
        if cfg.recon == "nearest_binmean":
            near = ORC.row(dataclasses.replace(cfg, recon="nearest", mutation=None), s, g)
            assert np.array_equal(res["P"], near["P"]), "hybrid forward differs from Nearest"
            assert np.array_equal(res["dS"], bm["dS"]), "hybrid backward differs from the bin mean's"
            continue
        z = s - s.max()
        keep = ~res["tail"]
        w = res["P"] * res["WL"]
        _close(w.sum(), np.exp(z[keep]).sum(), 1e-13, 0.0, "bin mass conservation")
        ratio = np.zeros_like(z)
        ratio[keep] = res["dS"][keep] / (np.exp(z[keep]) / res["WL"])
        for b in np.unique(res["ell"][keep]):
            mem = keep & (res["ell"] == b)
            e = np.exp(z[mem])
            _close(w[mem], np.full(mem.sum(), e.mean()), 1e-13, 0.0, f"bin {b} weight is the mean of e^z")
            if cfg.grad in ("full", "detached"):
                _close(ratio[mem], np.full(mem.sum(), ratio[mem][0]), 1e-9, 1e-12, f"bin {b} gradient contrast")
    # singleton bins: softmax (MinMax with K far above the number of keys)
    if cfg.calib == "minmax":
        s = np.random.default_rng(5).standard_normal(6) * 2.0
        g = np.random.default_rng(6).standard_normal(6)
        res = ORC.row(dataclasses.replace(cfg, K=4096), s, g)
        if len(set(res["ell"].tolist())) == 6:
            e = np.exp(s - s.max()); P = e / e.sum()
            if cfg.recon == "binmean":   # the hybrid's forward is Nearest's
                _close(res["P"], P, 1e-13, 1e-16, "singleton bins give softmax")
            if cfg.grad == "full":
                _close(res["dS"], P * (g - (P * g).sum()), 1e-10, 1e-14, "singleton bins give the softmax gradient")


PINS = [pin_golden, pin_exp_weights, pin_binmean, pin_autograd_rows, pin_autograd_ties, pin_autograd_head, pin_zero_sum, pin_channel_additivity,
        pin_two_key,
        pin_reconstruction_bounds, pin_nearest_brute_force, pin_finite_differences, pin_shift_invariance,
        pin_degenerate_and_causal_edges, pin_special_cases, pin_k_limit, pin_tail_policy]
