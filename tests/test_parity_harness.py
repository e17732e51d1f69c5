"""CPU tests of the parity harness and of the oracle's flag list (the acceptance apparatus).

The harness must accept a result that differs from the oracle only by the other valid
decision at a flagged position (an interval or Nearest boundary, the FWM window edge, a
bfloat16 rounding, an fp32 score at a rounding midpoint), and reject results with a planted
arithmetic mistake, a tie the fp32 scores do not have, or a flipped decision at a position
the oracle did not flag.  The scores themselves are pinned by exact rational arithmetic."""
import numpy as np
import pytest

import parity
from oracle import oracle as ORC
from quantized_softmax_attention_kia_amd.inputs import make_inputs


def _setup(calib, recon, T=300, K=16, qs=4.0, seed=5):
    q, k, v, do = make_inputs(1, 1, T, 64, seed, q_scale=qs)
    cfg = ORC.OracleConfig(calib, recon, "prob", "full", K, 8.0)
    return cfg, q[0, 0], k[0, 0], v[0, 0], do[0, 0]


def _outputs(r):
    return {key: r[key] for key in parity.KEYS}


@pytest.mark.parametrize("calib,recon", [("fwm", "nearest"), ("minmax", "lerp"), ("minmax", "nearest")])
def test_accepts_alternative_decision(calib, recon):
    cfg, q, k, v, do = _setup(calib, recon)
    guard = 1e-3                      # wide, so that this small case has flagged positions
    ref = ORC.head(cfg, q, k, v, do, guard=guard, flag_cap=100000)
    flags, _ = parity.relevant_flags(ref, cfg)
    assert flags.shape[0] > 0
    tested = 0
    for f in flags[::-1]:
        flip = tuple(int(x) for x in f)
        alt = ORC.head(cfg, q, k, v, do, flips=np.array([flip]))
        got = _outputs(alt)
        if not any(parity.bad_mask(got[key], ref[key]).any() for key in parity.KEYS):
            continue                  # this flip stays within tolerance: nothing to explain
        rep = parity.check_head(cfg, q, k, v, do, got, guard=guard)
        assert rep["bad0"] > 0 and len(rep["flips"]) >= 1
        tested += 1
        if tested == 2:
            break
    assert tested >= 1


@pytest.mark.parametrize("mutation", ["drop_rho_delta", "x_index", "dv_with_pl", "no_tie_split"])
def test_rejects_planted_error(mutation):
    cfg, q, k, v, do = _setup("minmax", "nearest")
    k = k.copy()
    k[7] = k[3]                       # ties, so that the tie mutation shows
    wrong = ORC.head(ORC.OracleConfig(cfg.calib, cfg.recon, cfg.ste, cfg.grad, cfg.K, cfg.tau, mutation),
                     q, k, v, do)
    with pytest.raises(AssertionError):
        parity.check_head(cfg, q, k, v, do, _outputs(wrong))


@pytest.mark.parametrize("calib", ["minmax", "fwm"])
def test_ties_are_ties_of_fp32_scores(calib):
    """A key whose score rounds to the same fp32 value as the row maximum ties it (the extremum
    gradient is split between them); one an fp32 ulp below does not, and a result that splits the
    gradient there is rejected.  Every element is compared."""
    cfg, q, k, v, do = _setup(calib, "lerp", T=120, K=4, qs=2.0)
    i = 100
    sc = ORC.head(cfg, q, k, v, do, scores=True)["scores"][i, : i + 1]
    j0 = int(np.argmax(sc))
    j1 = int(np.argsort(sc)[-2])
    tie = k.astype(np.float64).copy()
    tie[j1] = tie[j0]                         # the same fp32 score: a tie
    assert ORC.head(cfg, q, tie, v, do)["rowi"]["nA"][i] == 2
    near = tie.copy()
    near[j1] = tie[j0] * (1.0 - 2.0 ** -20)   # a few fp32 ulps below: no tie
    ref = ORC.head(cfg, q, near, v, do, guard=parity.GUARD, flag_cap=100000, scores=True)
    assert ref["rowi"]["nA"][i] == 1 and ref["scores"][i, j1] < ref["scores"][i, j0]
    # a result whose row i splits the maximum's term between j0 and j1 as a tie would (row i's
    # contributions computed with the tie, every other row as the reference has it)
    tied_i = ORC.head(cfg, q, tie, v, do, rows=[i])
    ref_i = ORC.head(cfg, q, near, v, do, rows=[i])
    got = {key: ref[key] + (tied_i[key] - ref_i[key]) for key in parity.KEYS}
    assert parity.bad_mask(got["dK"], ref["dK"]).any(), "the split changes nothing"
    with pytest.raises(AssertionError):
        parity.check_head(cfg, q, near, v, do, got)


def test_bf16_gradient_rounding_at_unflagged_position_is_rejected():
    """BF16-exp: a gradient dL/dw rounded to the other bfloat16 neighbour at a position the oracle
    does not flag (one bfloat16 ulp of one score-gradient term) is rejected, on a GPT-2-sized head
    (T = 1024, D = 64); at a flagged position it would be accepted."""
    q, k, v, do = make_inputs(1, 1, 1024, 64, 1)
    q, k, v, do = q[0, 0], k[0, 0], v[0, 0], do[0, 0]
    cfg = ORC.OracleConfig("fwm", "exp_bf16", "prob", "full", 4, 8.0)
    ref = ORC.head(cfg, q, k, v, do, guard=parity.GUARD, flag_cap=1 << 20)
    flagged = {(int(a), int(b)) for a, b, kind in ref["flags"] if kind == ORC.FLIP_GRAD}
    rng = np.random.default_rng(3)
    tried = rejected = 0
    while tried < 40 and rejected < 3:
        i = int(rng.integers(200, 1024))
        j = int(rng.integers(0, i + 1))
        if (i, j) in flagged:
            continue
        tried += 1
        alt = ORC.head(cfg, q, k, v, do, flips=np.array([(i, j, ORC.FLIP_GRAD)]), rows=[i])
        base = ORC.head(cfg, q, k, v, do, rows=[i])
        got = {key: ref[key] + (alt[key] - base[key]) for key in parity.KEYS}
        if not any(parity.bad_mask(got[key], ref[key]).any() for key in parity.KEYS):
            continue                  # one ulp of a small term: within tolerance anyway
        with pytest.raises(AssertionError):
            parity.check_head(cfg, q, k, v, do, got)
        rejected += 1
    assert rejected >= 1, "no single-ulp gradient rounding was large enough to test"


def _exact_f32(x):
    """The fp32 value nearest the rational x, ties to even (no double rounding)."""
    from fractions import Fraction
    d = float(x)                              # correctly rounded double
    f = np.float32(d)
    lo = f if Fraction(float(f)) <= x else np.nextafter(f, np.float32(-np.inf))
    hi = np.nextafter(lo, np.float32(np.inf))
    mid = (Fraction(float(lo)) + Fraction(float(hi))) / 2
    if x < mid:
        return float(lo)
    if x > mid:
        return float(hi)
    return float(lo) if (lo.view(np.uint32) & 1) == 0 else float(hi)


def test_scores_are_correctly_rounded_fp32():
    """The scores the oracle runs on are the exact product sums, scaled and rounded once to fp32
    (checked with exact rational arithmetic), except where the oracle flags that its double sum
    lies within its own rounding bound of an fp32 midpoint; a value exactly at a midpoint is
    flagged, and the flip takes the other fp32 neighbour."""
    from fractions import Fraction
    rng = np.random.default_rng(2)
    T, D = 24, 16
    q = rng.standard_normal((T, D)).astype(np.float32).astype(np.float64)
    k = rng.standard_normal((T, D)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((T, D))
    scale = 0.3                               # not a power of two: the scaling rounds too
    cfg = ORC.OracleConfig("minmax", "lerp", "prob", "full", 4, 8.0)
    ref = ORC.head(cfg, q, k, v, None, scale=scale, guard=0.0, flag_cap=1000, scores=True)
    flagged = {(int(a), int(b)) for a, b, kind in ref["flags"] if kind == ORC.FLIP_SCORE}
    fs = Fraction(scale)
    for i in range(T):
        for j in range(i + 1):
            exact = fs * sum(Fraction(q[i, d]) * Fraction(k[j, d]) for d in range(D))
            if (i, j) not in flagged:
                assert ref["scores"][i, j] == _exact_f32(exact), (i, j)
    # an exact midpoint between 1 and 1 + 2^-23: 1 + 2^-24, rounded to even (1.0), is flagged
    q2 = np.zeros((2, 4)); k2 = np.zeros((2, 4))
    q2[1, :2] = [1.0, 2.0 ** -12]; k2[1, :2] = [1.0, 2.0 ** -12]; k2[0, 0] = 0.5
    r = ORC.head(cfg, q2, k2, np.ones((2, 4)), None, scale=1.0, guard=0.0, flag_cap=10, scores=True)
    assert r["scores"][1, 1] == 1.0
    assert (1, 1, ORC.FLIP_SCORE) in {tuple(int(x) for x in f) for f in r["flags"]}
    r2 = ORC.head(cfg, q2, k2, np.ones((2, 4)), None, scale=1.0, flips=np.array([(1, 1, ORC.FLIP_SCORE)]),
                  scores=True)
    assert r2["scores"][1, 1] == 1.0 + 2.0 ** -23


@pytest.mark.parametrize("calib,recon,tail,K", [("minmax", "lerp", "zero", 4), ("minmax", "nearest", "zero", 16),
                                               ("fwm", "nearest", "zero", 4), ("fwm", "lerp", "resolved", 8)])
def test_decision_flags_are_the_positions_within_the_guard(calib, recon, tail, K):
    """The flag list holds exactly the visible positions whose u lies within the guard of a
    decision boundary (§3: interior interval boundaries 1..K-1, every integer below K on the
    resolved grid; the Nearest midpoints k + 1/2; the FWM window edge z = -tau), found here by
    brute force over every pair from the fp32 scores and the row extrema.  A wider or narrower
    band, a missed boundary or a spurious one fails; positions within 1e-9 of the guard's edge are
    left out (either answer is the definition's)."""
    T, guard = 200, 2e-3
    q, k, v, do = make_inputs(1, 1, T, 64, 11, q_scale=3.0)
    q, k, v, do = q[0, 0], k[0, 0], v[0, 0], do[0, 0]
    cfg = ORC.OracleConfig(calib, recon, "prob", "full", K, 6.0, tail=tail)
    ref = ORC.head(cfg, q, k, v, do, guard=guard, flag_cap=1 << 20, scores=True)
    kinds = ORC.FLIP_INTERVAL | ORC.FLIP_NEAREST | ORC.FLIP_TAIL
    got = {(int(i), int(j), int(kd)) for i, j, kd in ref["flags"] if kd & kinds}
    S, M, m = ref["scores"], ref["rowd"]["M"], ref["rowd"]["m"]
    want, edge = set(), set()
    nearest = recon == "nearest"
    for i in range(T):
        for j in range(i + 1):
            s = S[i, j]
            if calib == "minmax":
                if M[i] - m[i] <= 1e-12:
                    continue                          # degenerate row: no boundary
                h = (M[i] - m[i]) / K
                u = (s - m[i]) / h
            else:
                h = 6.0 / K
                z = min(s - M[i], 0.0)
                u = ((z if tail == "resolved" else max(z, -6.0)) + 6.0) / h
                if tail != "resolved":
                    dt = abs(z + 6.0) / h             # distance from the window edge
                    if dt < guard:
                        want.add((i, j, ORC.FLIP_TAIL))
                    if abs(dt - guard) < 1e-9:
                        edge.add((i, j, ORC.FLIP_TAIL))
            ki = np.floor(u + 0.5)
            if (tail == "resolved" or ki >= 1) and ki <= K - 1:
                di = abs(u - ki)
                if di < guard:
                    want.add((i, j, ORC.FLIP_INTERVAL))
                if abs(di - guard) < 1e-9:
                    edge.add((i, j, ORC.FLIP_INTERVAL))
            kh = np.floor(u) + 0.5
            if nearest and kh < K:
                dh = abs(u - kh)
                if dh < guard:
                    want.add((i, j, ORC.FLIP_NEAREST))
                if abs(dh - guard) < 1e-9:
                    edge.add((i, j, ORC.FLIP_NEAREST))
    assert len(want) > 20, "the guard is wide enough that this head has flagged positions"
    assert got - edge == want - edge
