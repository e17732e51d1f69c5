"""Parity harness: HIP results against the oracle, element by element.

Tolerance (stated by the target): |x - x_ref| <= 1e-5 + 2e-4 |x_ref| on O, dQ,
dK, dV.  Bin decisions are taken in fp32 by the kernels and in double by the
oracle; at a position within GUARD = 1e-5 (in units of the interval width) of
a bin boundary, or within the change of u that representing the scores in
fp32 (one ulp of s and of the row extrema) can cause when that is larger,
either decision is correct.  The oracle lists those positions;
when the kernel's output differs from the oracle's, the harness asks the oracle
to take the other decision at listed positions (greedily, a few at a time) and
accepts only if that makes every element agree.

Cancellation: an output element that is a sum of terms of both signs much
larger than the result (a key that is the arg-max of several rows collects
extremum terms that cancel against the rest of its column) carries the fp32
rounding of those terms.  Such an element is also accepted when it is within
CANCEL = 1e-5 of the sum of the absolute values of its terms (the oracle
returns that sum); these elements are counted separately and must stay below
MAX_CANCEL_FRACTION of the head's elements.  Rows whose top-2 or bottom-2
scores are within GUARD (or the scores' rounding bound) of a tie may pick either
key as the extremum: their O and dQ rows, and the dK / dV rows of the competing
keys, are excluded and counted (tie_exclusions).

Exponential baselines: their roundings to bfloat16 / E4M3 are decisions like the
bin decisions (flagged within the guard of a rounding midpoint, flipped the same
way).  BF16-exp's backward rounds the fp32 gradient dL/dw to bfloat16; where that
gradient lies within its own fp32 error of a rounding midpoint either rounding is
correct, and there are too many such positions to flip one by one: the oracle
returns, per element of dQ and dK, how much those roundings can change it
(`amb`), and that amount is added to the element's tolerance.
"""
from __future__ import annotations

import numpy as np

from oracle import oracle as ORC

ATOL, RTOL = 1e-5, 2e-4
GUARD = 1e-5
# cancellation allowance: an element whose value is a sum of much larger terms of both
# signs is judged against the sum of |terms| (see check_head)
CANCEL = 1e-5
MAX_CANCEL_FRACTION = 1e-3
KEYS = ("O", "dQ", "dK", "dV")


def bad_mask(got, ref):
    return ~(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref))


def _count(gpu, ref, absref=None, excluded=None, amb=None):
    masks = {}
    for k in KEYS:
        if gpu.get(k) is None:
            continue
        m = bad_mask(gpu[k], ref[k])
        if amb is not None and amb.get(k) is not None:
            m &= ~(np.abs(gpu[k] - ref[k]) <= ATOL + RTOL * np.abs(ref[k]) + amb[k])
        if absref is not None:
            m &= ~(np.abs(gpu[k] - ref[k]) <= CANCEL * absref[k])
        if excluded is not None and excluded.get(k) is not None:
            m[excluded[k]] = False
        masks[k] = m
    return masks, int(sum(int(m.sum()) for m in masks.values()))


def tie_exclusions(ref, cfg):
    """Rows with near-tied extrema may pick either key: exclude those rows' O and dQ and the
    dK, dV rows of the competing keys (the extremum gradient lands on one of them)."""
    rows = near_tie_rows(ref, cfg)
    ri = ref["rowi"]
    keys = set()
    for i in rows:
        for name in (("amax", "amax2", "amin", "amin2") if cfg.calib == "minmax" else ("amax", "amax2")):
            j = int(ri[name][i])
            if j >= 0:
                keys.add(j)
    keys = np.array(sorted(keys), dtype=np.int64)
    return dict(O=rows, dQ=rows, dK=keys, dV=keys), len(rows)


def near_tie_rows(ref, cfg):
    rd = ref["rowd"]
    rows = rd["gapM"] < np.maximum(GUARD * np.maximum(1.0, np.abs(rd["M"])), rd["tolM"])
    if cfg.calib == "minmax":
        rows |= rd["gapm"] < np.maximum(GUARD * np.maximum(1.0, np.abs(rd["m"])), rd["tolm"])
    # a gap of exactly 0 cannot occur (ties are counted as ties); inf means no second value
    return np.flatnonzero(rows)


def relevant_flags(ref, cfg):
    f = ref["flags"]
    if f.shape[0] == 0:
        return f
    if cfg.recon in ("softmax", "exp_bf16", "exp_fp8"):
        kinds = {ORC.FLIP_ROUND, ORC.FLIP_ROUND2}
        return f[np.isin(f[:, 2], list(kinds))]
    kinds = {ORC.FLIP_INTERVAL}
    if cfg.recon == "nearest":
        kinds.add(ORC.FLIP_NEAREST)
    if cfg.calib == "fwm":
        kinds.add(ORC.FLIP_TAIL)
    keep = np.isin(f[:, 2], list(kinds))
    return f[keep]


def check_head(cfg, q, k, v, do, gpu, *, causal=True, scale=None, max_flips=8, nthreads=None, guard=GUARD):
    """Compare one head.  gpu: dict with O, dQ, dK, dV arrays [T, D].

    Returns a report dict; raises AssertionError when the mismatch cannot be
    explained by alternative decisions at near-boundary positions.  A flip in
    row i changes only row i's contributions (O_i, dQ_i and its terms of dK,
    dV), so candidates are scored by recomputing that row alone.
    """
    ref = ORC.head(cfg, q, k, v, do, causal=causal, scale=scale, guard=guard, flag_cap=1 << 20,
                   absolute=True, nthreads=nthreads)
    cur = {key: ref[key] for key in KEYS if gpu.get(key) is not None}
    absref = ref["abs"]
    amb = ref["amb"] if cfg.recon == "exp_bf16" else None
    excl, nties = tie_exclusions(ref, cfg)
    masks, nbad = _count(gpu, cur, absref, excl, amb)
    flags = relevant_flags(ref, cfg)
    dist = ref["flag_dist"][np.isin(ref["flags"][:, 2], np.unique(flags[:, 2]))] if flags.shape[0] else np.zeros(0)
    report = dict(nflags=int(flags.shape[0]), near_ties=nties, bad0=nbad, flips=[],
                  elements=int(sum(cur[k].size for k in cur)))

    def finish(rep, cur_now):
        _, ns = _count(gpu, cur_now, None, excl, amb)
        _, nb = _count(gpu, cur_now, absref, excl, amb)
        rep["cancel"] = ns - nb
        assert rep["cancel"] <= MAX_CANCEL_FRACTION * rep["elements"], \
            f"{rep['cancel']} of {rep['elements']} elements need the cancellation allowance"
        return rep

    if nbad == 0:
        return finish(report, cur)
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
            _, n = _count(gpu, trial, absref, excl, amb)
            if best is None or n < best[0]:
                best = (n, c, trial)
        if best is None or best[0] >= nbad:
            break
        nbad, c, cur = best
        chosen.append(c)
        by_row.setdefault(c[0], []).append(c)
        masks, _ = _count(gpu, cur, absref, excl, amb)
        if nbad == 0:
            report["flips"] = chosen
            return finish(report, cur)
    msg = []
    for key, m in masks.items():
        if m.any():
            i = np.argwhere(m)[0]
            msg.append(f"{key}{tuple(i)}: gpu={gpu[key][tuple(i)]!r} ref={cur[key][tuple(i)]!r} ({int(m.sum())} bad)")
    raise AssertionError(f"{cfg}: {nbad} elements outside tolerance after flips {chosen}; "
                         f"{report['nflags']} flagged positions; " + "; ".join(msg))


def check_bins(cfg, q, k, gpu_bins, *, causal=True, scale=None):
    """Bin decisions: bit-exact except at near-boundary positions (listed by the oracle)."""
    ref = ORC.head(cfg, q, k, k, None, causal=causal, scale=scale, guard=GUARD, flag_cap=1 << 20, bins=True)
    diff = np.argwhere(gpu_bins != ref["bins"])
    flags = relevant_flags(ref, cfg)
    flagged = {(int(a), int(b)) for a, b, _ in flags}
    ties = set(near_tie_rows(ref, cfg).tolist())
    unexplained = [tuple(x) for x in diff if (int(x[0]), int(x[1])) not in flagged and int(x[0]) not in ties]
    assert not unexplained, (f"{len(unexplained)} bin decisions differ away from any boundary, e.g. "
                             f"{unexplained[:3]}: gpu={[int(gpu_bins[t]) for t in unexplained[:3]]} "
                             f"ref={[int(ref['bins'][t]) for t in unexplained[:3]]}")
    return dict(pairs=int((ref["bins"] != 255).sum()), flagged=len(flagged), differing=len(diff))


def pick_heads(cfg, q, k, *, causal=True, scale=None, want=2, nthreads=None):
    """Deterministic choice of heads: the first, the last, then the middle one."""
    B, H = q.shape[:2]
    order = [(0, 0), (B - 1, H - 1), (B // 2, H // 2)]
    picked = []
    for bh in order:
        if bh not in picked:
            picked.append(bh)
    return picked[:want]
