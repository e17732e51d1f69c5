"""Parity harness: HIP results against the oracle, element by element.

Tolerance (stated by the target): |x - x_ref| <= 1e-5 + 2e-4 |x_ref| on every element of O,
dQ, dK, dV.  Nothing is excluded and no element gets a wider tolerance.

Decisions.  The method takes discrete decisions: the interval and Nearest index of a key,
the side of the FWM window edge, a rounding to bfloat16 / E4M3 (the exponential baselines,
BF16-exp's gradient), which keys attain a row extremum.  Both sides take them on fp32 scores
(the operator's precision): the kernels on the correctly rounded score wherever their own
faster score cannot settle a decision, the oracle on its double product sum rounded once.  At
a position within GUARD = 1e-5 of a decision's boundary (in the decision's own units: interval
widths, format spacings), and at a score whose double sum lies within its rounding bound of
an fp32 midpoint, either decision is correct; the oracle lists those positions (its flags).
When the kernel's output differs from the oracle's, the harness asks the oracle to take the
other decision at listed positions (greedily, one at a time, each time the flip that most
reduces the total excess over the tolerance, recomputing only the affected row) and accepts
only if every element then agrees.
"""
from __future__ import annotations

import numpy as np

from oracle import oracle as ORC

ATOL, RTOL = 1e-5, 2e-4
GUARD = 1e-5
KEYS = ("O", "dQ", "dK", "dV")
EXP_RECON = ("softmax", "exp_bf16", "exp_fp8")


def bad_mask(got, ref):
    return ~(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref))


def _count(gpu, ref):
    masks = {k: bad_mask(gpu[k], ref[k]) for k in KEYS if gpu.get(k) is not None}
    return masks, int(sum(int(m.sum()) for m in masks.values()))


def _excess(gpu, ref):
    """How far the elements outside tolerance are outside it, summed: the flip search's objective
    (a flip can move an element toward agreement without yet bringing it inside, e.g. one of the
    many rows whose tied maximum shares a key's extremum term)."""
    return float(sum(np.maximum(np.abs(gpu[k] - ref[k]) - (ATOL + RTOL * np.abs(ref[k])), 0.0).sum()
                     for k in KEYS if gpu.get(k) is not None))


def relevant_kinds(cfg):
    """Flag kinds that can change the variant's results."""
    if cfg.recon in EXP_RECON:
        kinds = {ORC.FLIP_ROUND, ORC.FLIP_ROUND2, ORC.FLIP_SCORE}
        if cfg.recon == "exp_bf16":
            kinds.add(ORC.FLIP_GRAD)
        return kinds
    kinds = {ORC.FLIP_INTERVAL, ORC.FLIP_SCORE}
    if cfg.recon in ("nearest", "binmean", "nearest_binmean"):
        kinds.add(ORC.FLIP_NEAREST)
    if cfg.calib == "fwm" and getattr(cfg, "tail", "zero") != "resolved":
        kinds.add(ORC.FLIP_TAIL)
    return kinds


def relevant_flags(ref, cfg):
    f = ref["flags"]
    if f.shape[0] == 0:
        return f, ref["flag_dist"]
    keep = np.isin(f[:, 2], sorted(relevant_kinds(cfg)))
    return f[keep], ref["flag_dist"][keep]


def check_head(cfg, q, k, v, do, gpu, *, causal=True, scale=None, max_flips=128, nthreads=None, guard=GUARD):
    """Compare one head.  gpu: dict with O, dQ, dK, dV arrays [T, D].

    Returns a report dict; raises AssertionError when the mismatch cannot be explained by
    alternative decisions at flagged positions.  A flip in row i changes only row i's
    contributions (O_i, dQ_i and its terms of dK, dV), so candidates are scored by recomputing
    that row alone.
    """
    ref = ORC.head(cfg, q, k, v, do, causal=causal, scale=scale, guard=guard, flag_cap=1 << 22,
                   nthreads=nthreads)
    assert ref["nflags"] <= 1 << 22, "flag list overflowed"
    cur = {key: ref[key] for key in KEYS if gpu.get(key) is not None}
    masks, nbad = _count(gpu, cur)
    flags, dist = relevant_flags(ref, cfg)
    report = dict(nflags=int(flags.shape[0]), bad0=nbad, flips=[], elements=int(sum(cur[x].size for x in cur)),
                  ties=int((ref["rowi"]["nA"] > 1).sum() + (ref["rowi"]["nC"] > 1).sum()))
    if nbad == 0:
        return report
    order = np.argsort(dist, kind="stable")
    flags = flags[order]
    by_row: dict[int, list] = {}
    cache: dict[tuple, dict] = {}

    def row_part(i, fl):
        key = (i, tuple(sorted(fl)))
        if key not in cache:
            r = ORC.head(cfg, q, k, v, do, causal=causal, scale=scale, rows=[i],
                         flips=np.array(fl, dtype=np.int32).reshape(-1, 3) if fl else None, nthreads=1)
            cache[key] = {kk: r[kk] for kk in cur}
        return cache[key]

    chosen = []
    amax, amin = ref["rowi"]["amax"], ref["rowi"]["amin"]
    excess = _excess(gpu, cur)
    for _ in range(max_flips):
        bad_rows = set()
        for key in ("O", "dQ"):
            if key in masks:
                bad_rows |= set(np.flatnonzero(masks[key].any(1)).tolist())
        bad_cols = set()
        for key in ("dK", "dV"):
            if key in masks:
                bad_cols |= set(np.flatnonzero(masks[key].any(1)).tolist())
        cand = [tuple(int(y) for y in x) for x in flags
                if (x[0] in bad_rows or x[1] in bad_cols or amax[x[0]] in bad_cols or amin[x[0]] in bad_cols)]
        cand = [c for c in cand if c not in chosen][:256]
        best = None
        for c in cand:
            i = c[0]
            old = row_part(i, by_row.get(i, []))
            new = row_part(i, by_row.get(i, []) + [c])
            trial = {kk: cur[kk] + (new[kk] - old[kk]) for kk in cur}
            e = _excess(gpu, trial)
            if best is None or e < best[0]:
                best = (e, c, trial)
        if best is None or best[0] >= excess:
            break
        excess, c, cur = best
        chosen.append(c)
        by_row.setdefault(c[0], []).append(c)
        masks, nbad = _count(gpu, cur)
        if nbad == 0:
            report["flips"] = chosen
            return report
    msg = []
    for key, m in masks.items():
        if m.any():
            i = np.argwhere(m)[0]
            msg.append(f"{key}{tuple(i)}: gpu={gpu[key][tuple(i)]!r} ref={cur[key][tuple(i)]!r} ({int(m.sum())} bad)")
    raise AssertionError(f"{cfg}: {nbad} elements outside tolerance after flips {chosen}; "
                         f"{report['nflags']} flagged positions; " + "; ".join(msg))


def check_bins(cfg, q, k, gpu_bins, *, causal=True, scale=None):
    """Bin decisions: bit-exact except at flagged positions (listed by the oracle)."""
    ref = ORC.head(cfg, q, k, k, None, causal=causal, scale=scale, guard=GUARD, flag_cap=1 << 22, bins=True)
    diff = np.argwhere(gpu_bins != ref["bins"])
    flags, _ = relevant_flags(ref, cfg)
    flagged = {(int(a), int(b)) for a, b, kind in flags}
    unexplained = [tuple(x) for x in diff if (int(x[0]), int(x[1])) not in flagged]
    assert not unexplained, (f"{len(unexplained)} bin decisions differ away from any boundary, e.g. "
                             f"{unexplained[:3]}: gpu={[int(gpu_bins[t]) for t in unexplained[:3]]} "
                             f"ref={[int(ref['bins'][t]) for t in unexplained[:3]]}")
    return dict(pairs=int((ref["bins"] != 255).sum()), flagged=len(flagged), differing=len(diff))


def all_heads(q):
    """Every (b, h) of a [B, H, T, D] array."""
    B, H = q.shape[:2]
    return [(b, h) for b in range(B) for h in range(H)]
