"""CPU tests of the parity harness and of the oracle's flag list (the acceptance apparatus).

The harness must accept a result that differs from the oracle only by the other valid
decision at a flagged position (an interval or Nearest boundary, the FWM window edge, a
near tie of a row extremum, a bfloat16 rounding), and reject results with a planted
arithmetic mistake or a flipped decision at a position the oracle did not flag.  The flag
list itself is pinned against a direct computation: every decision that rounding the
scores to fp32 changes is flagged, and nothing is flagged farther from its boundary than
the fp32 bound (or the guard) allows."""
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
def test_near_tie_is_a_flip_not_an_exclusion(calib):
    """A key within the fp32 bound of the row maximum may tie it in fp32: the harness accepts
    the split extremum gradient through a flip, with every element compared; a key farther away
    than the bound is not flagged, and a split there is rejected."""
    cfg, q, k, v, do = _setup(calib, "lerp", T=120, K=4, qs=2.0)
    i = 100
    s = (q[i].astype(np.float64) @ k[: i + 1].astype(np.float64).T) / 8.0
    j0 = int(np.argmax(s))
    j1 = int(np.argsort(s)[-2])
    # move key j1 so that its exact score is one part in 1e8 below the row maximum: inside the
    # fp32 bound (2 ulps), hence a legitimate fp32 tie
    kk = k.astype(np.float64).copy()
    kk[j1] = kk[j0] * (1.0 - 1e-8)
    ref = ORC.head(cfg, q, kk, v, do, guard=parity.GUARD, flag_cap=100000)
    flags, _ = parity.relevant_flags(ref, cfg)
    tie = [tuple(int(x) for x in f) for f in flags if f[0] == i and f[1] == j1 and f[2] == ORC.FLIP_TIE_MAX]
    assert tie, "near tie not flagged"
    alt = ORC.head(cfg, q, kk, v, do, flips=np.array(tie))
    got = _outputs(alt)
    assert any(parity.bad_mask(got[key], ref[key]).any() for key in ("dQ", "dK")), "tie flip changes nothing"
    rep = parity.check_head(cfg, q, kk, v, do, got)
    assert rep["flips"] == tie and rep["elements"] == 4 * q.size
    # 1e-5 below the maximum: far outside the fp32 bound, so no flag and the split is rejected
    kk[j1] = kk[j0] * (1.0 - 1e-5)
    ref = ORC.head(cfg, q, kk, v, do, guard=parity.GUARD, flag_cap=100000)
    flags, _ = parity.relevant_flags(ref, cfg)
    assert not any(f[0] == i and f[1] == j1 and f[2] == ORC.FLIP_TIE_MAX for f in flags)
    alt = ORC.head(cfg, q, kk, v, do, flips=np.array([(i, j1, ORC.FLIP_TIE_MAX)]))
    with pytest.raises(AssertionError):
        parity.check_head(cfg, q, kk, v, do, _outputs(alt))


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


def _row_decisions(cfg, s):
    r = ORC.row(cfg, s)
    return r["r"], r["ell"], r["tail"], r["amax"], r["nA"], r["amin"], r["nC"]


@pytest.mark.parametrize("calib,recon,K", [("minmax", "nearest", 4), ("minmax", "lerp", 16), ("fwm", "nearest", 8),
                                           ("fwm", "lerp", 32)])
def test_fp32_guard_covers_and_is_tight(calib, recon, K):
    """The flag list against a direct computation.  Each row's scores are rounded to fp32 and the
    decisions retaken on them: every decision that changes (interval, Nearest index, window edge,
    extremum tie) is flagged.  With the guard at 0 every flagged position lies within the fp32
    bound of its boundary, recomputed here from its definition: one fp32 ulp of the score and of
    the extrema u is measured from, over the interval width."""
    cfg = ORC.OracleConfig(calib, recon, "prob", "full", K, 3.0)
    # coarse inputs put many scores near boundaries: integers -2..2 times (1 + 3e-7 N(0,1))
    rng = np.random.default_rng(11)
    T, D = 160, 64
    q = rng.integers(-2, 3, (T, D)) * (1.0 + 3e-7 * rng.standard_normal((T, D)))
    k = rng.integers(-2, 3, (T, D)) * (1.0 + 3e-7 * rng.standard_normal((T, D)))
    v = rng.standard_normal((T, D))
    ref = ORC.head(cfg, q, k, v, None, guard=0.0, flag_cap=1 << 20)
    flags = ref["flags"]
    fl = {(int(a), int(b), int(c)) for a, b, c in flags}
    flagged_pos = {(a, b) for a, b, _ in fl}
    changed = 0
    scale = 1.0 / np.sqrt(D)
    ulp = 2.0 ** -23
    for i in range(1, T):
        s = scale * (q[i] @ k[: i + 1].T)
        s32 = s.astype(np.float32).astype(np.float64)
        a = _row_decisions(cfg, s)
        b = _row_decisions(cfg, s32)
        ell_differs = (a[1] != b[1]) if recon == "nearest" else np.zeros_like(a[1], dtype=bool)
        for j in np.flatnonzero((a[0] != b[0]) | ell_differs | (a[2] != b[2])):
            changed += 1
            assert (i, int(j)) in flagged_pos, f"decision ({i}, {j}) changed by fp32 scores but not flagged"
        if b[4] > a[4]:   # an fp32 tie of the maximum the exact scores do not have
            for j in np.flatnonzero(s32 == s32.max()):
                if j != a[3]:
                    changed += 1
                    assert (i, int(j), ORC.FLIP_TIE_MAX) in fl, f"fp32 tie ({i}, {j}) not flagged"
        # tightness: every flag of this row within the fp32 bound of its boundary
        M, m = s.max(), s.min()
        h = (M - m) / K if calib == "minmax" else cfg.tau / K
        for (ii, j, kind), dist in zip(map(tuple, flags), ref["flag_dist"]):
            if ii != i:
                continue
            ebj = ulp * abs(s[j]) + 1e-15 * scale * np.abs(q[i] * k[j]).sum()
            ebM = ulp * abs(M) + 1e-15 * scale * np.abs(q[i] * k[int(np.argmax(s))]).sum()
            ebm = ulp * abs(m) + 1e-15 * scale * np.abs(q[i] * k[int(np.argmin(s))]).sum()
            if kind in (ORC.FLIP_TIE_MAX, ORC.FLIP_TIE_MIN):
                assert dist <= ebj + (ebM if kind == ORC.FLIP_TIE_MAX else ebm) + 1e-300
            else:
                bound = (ebj + 2 * ebm + ebM) / h if calib == "minmax" else (ebj + ebM) / h
                assert dist < bound * (1 + 1e-9), f"flag ({i}, {j}) at {dist} beyond the fp32 bound {bound}"
    assert changed > 0, "the inputs produced no decision that fp32 scores change"
    # the flagged set is a small part of the pairs, so flips cannot explain arbitrary errors
    assert len(flagged_pos) < 0.05 * T * (T + 1) / 2
