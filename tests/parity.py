"""Parity harness: HIP results against the oracle, element by element.

Tolerance (stated by the target): |x - x_ref| <= 1e-5 + 2e-4 |x_ref| on O, dQ,
dK, dV.  Bin decisions are taken in fp32 by the kernels and in double by the
oracle; at a position within GUARD = 1e-5 (in units of the interval width) of
a bin boundary either decision is correct.  The oracle lists those positions;
when the kernel's output differs from the oracle's, the harness asks the oracle
to take the other decision at listed positions (greedily, a few at a time) and
accepts only if that makes every element agree.  Rows whose top-2 or bottom-2
scores are within GUARD of a tie are reported; heads containing them are not
used for element-wise parity (see pick_heads).
"""
from __future__ import annotations

import numpy as np

from oracle import oracle as ORC

ATOL, RTOL = 1e-5, 2e-4
GUARD = 1e-5
KEYS = ("O", "dQ", "dK", "dV")


def bad_mask(got, ref):
    return ~(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref))


def _count(gpu, ref):
    masks = {k: bad_mask(gpu[k], ref[k]) for k in KEYS if gpu.get(k) is not None}
    return masks, int(sum(int(m.sum()) for m in masks.values()))


def near_tie_rows(ref, cfg):
    M = ref["rowd"]["M"]
    tol = GUARD * np.maximum(1.0, np.abs(M))
    rows = ref["rowd"]["gapM"] < tol
    if cfg.calib == "minmax":
        rows |= ref["rowd"]["gapm"] < GUARD * np.maximum(1.0, np.abs(ref["rowd"]["m"]))
    # a gap of exactly 0 cannot occur (ties are counted as ties); inf means no second value
    return np.flatnonzero(rows)


def relevant_flags(ref, cfg):
    f = ref["flags"]
    if f.shape[0] == 0:
        return f
    kinds = {ORC.FLIP_INTERVAL}
    if cfg.recon == "nearest":
        kinds.add(ORC.FLIP_NEAREST)
    if cfg.calib == "fwm":
        kinds.add(ORC.FLIP_TAIL)
    keep = np.isin(f[:, 2], list(kinds))
    return f[keep]


def check_head(cfg, q, k, v, do, gpu, *, causal=True, scale=None, max_flips=6, nthreads=None):
    """Compare one head.  gpu: dict with O, dQ, dK, dV arrays [T, D].

    Returns a report dict; raises AssertionError when the mismatch cannot be
    explained by alternative decisions at near-boundary positions.
    """
    ref = ORC.head(cfg, q, k, v, do, causal=causal, scale=scale, guard=GUARD, flag_cap=1 << 20,
                   nthreads=nthreads)
    masks, nbad = _count(gpu, ref)
    flags = relevant_flags(ref, cfg)
    report = dict(nflags=int(flags.shape[0]), near_ties=len(near_tie_rows(ref, cfg)), bad0=nbad, flips=[])
    if nbad == 0:
        return report
    T = q.shape[0]
    chosen = []
    for _ in range(max_flips):
        bad_rows = set(np.flatnonzero(masks.get("O", np.zeros((T, 1), bool)).any(1)))
        if masks.get("dQ") is not None:
            bad_rows |= set(np.flatnonzero(masks["dQ"].any(1)))
        bad_cols = set()
        for key in ("dK", "dV"):
            if masks.get(key) is not None:
                bad_cols |= set(np.flatnonzero(masks[key].any(1)))
        amax, amin = ref["rowi"]["amax"], ref["rowi"]["amin"]
        cand = [tuple(x) for x in flags
                if (x[0] in bad_rows or x[1] in bad_cols or amax[x[0]] in bad_cols or amin[x[0]] in bad_cols)
                and tuple(x) not in chosen]
        if not cand:
            cand = [tuple(x) for x in flags if tuple(x) not in chosen][:24]
        best = None
        for c in cand[:48]:
            trial = ORC.head(cfg, q, k, v, do, causal=causal, scale=scale, flips=np.array(chosen + [c]),
                             nthreads=nthreads)
            _, n = _count(gpu, trial)
            if best is None or n < best[0]:
                best = (n, c, trial)
        if best is None or best[0] >= nbad:
            break
        nbad = best[0]
        chosen.append(best[1])
        masks, _ = _count(gpu, best[2])
        if nbad == 0:
            report["flips"] = chosen
            return report
    # describe the worst element for the failure message
    msg = []
    for key, m in masks.items():
        if m.any():
            i = np.argwhere(m)[0]
            msg.append(f"{key}{tuple(i)}: gpu={gpu[key][tuple(i)]!r} ref={ref[key][tuple(i)]!r} ({int(m.sum())} bad)")
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
    """Deterministic choice of heads (first, last, then middle ones) without near-tied extrema."""
    B, H = q.shape[:2]
    order = [(0, 0), (B - 1, H - 1)] + [(b, h) for b in range(B) for h in range(H)][1:-1]
    seen, picked = set(), []
    for bh in order:
        if bh in seen:
            continue
        seen.add(bh)
        r = ORC.head(cfg, q[bh], k[bh], k[bh], None, causal=causal, scale=scale, nthreads=nthreads)
        if len(near_tie_rows(r, cfg)) == 0:
            picked.append(bh)
        if len(picked) == want:
            break
    return picked
