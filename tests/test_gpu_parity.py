"""GPU parity: the HIP path (through the C ABI) against the oracle.

Every case prints its name, shape, seed and variant before touching the GPU.
Tolerance: 1e-5 absolute + 2e-4 relative on O, dQ, dK, dV; bin decisions
bit-exact away from bin boundaries (see tests/parity.py).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import parity
from oracle import oracle as ORC
from quantized_softmax_attention_kia_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

VARIANTS16 = [(c, r, s, g) for c in ("minmax", "fwm") for r in ("lerp", "nearest")
              for s in ("weight", "prob") for g in ("full", "detached")]
# the range_grad ablations: single-channel (max_only, min_only) and the P1 projection
ABLATIONS = [(c, r, s, g) for c in ("minmax", "fwm") for (r, s) in (("lerp", "prob"), ("nearest", "weight"),
             ("nearest", "prob")) for g in ("max_only", "min_only", "p1")]
# the FWM tail policies (floored and resolved tails), as (calib, recon, ste, grad, tail)
TAILS = [("fwm", r, s, g, tp) for tp in ("floor", "resolved") for (r, s) in (("lerp", "prob"), ("nearest", "weight"),
         ("nearest", "prob")) for g in ("full", "detached", "p1")]
# the exponential baselines (softmax, BF16-exp, FP8-rounded exp); calib, K, tau, ste are ignored
EXPS = [("fwm", r, "prob", g) for r in ("softmax", "exp_bf16", "exp_fp8") for g in ("full", "detached", "p1")]
# bin mean and the Nearest-forward / bin-mean-backward hybrid (built for K <= 8)
BINMEANS = [(c, r, "prob", g) for c in ("minmax", "fwm") for r in ("binmean", "nearest_binmean")
            for g in ("full", "detached", "p1")]


@pytest.fixture(scope="module")
def kb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_softmax_attention_kia_amd import binding
    return binding


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _tail(variant):
    """variant: (calib, recon, ste, grad, K, tau[, tail])"""
    return variant[6] if len(variant) > 6 else "zero"


def gpu_run(kb, variant, q, k, v, do, *, causal=True, scale=0.0, dtype="f32"):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cfg = kb.Config(*variant[:4], K=variant[4], tau=variant[5], causal=causal, scale=scale, tail=_tail(variant))
    qt, kt, vt, dot = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(tdt) for x in (q, k, v, do))
    o, rowrec, p = kb.forward(cfg, qt, kt, vt)
    dq, dk, dv = kb.backward(p, qt, kt, vt, o, dot, rowrec)
    torch.cuda.synchronize()
    out = dict(O=o, dQ=dq, dK=dk, dV=dv)
    return {key: t.cpu().numpy().astype(np.float64) for key, t in out.items()}, (qt, kt, rowrec, p)


def ocfg(variant):
    return ORC.OracleConfig(*variant[:4], K=variant[4], tau=variant[5], tail=_tail(variant))


def compare_all_heads(variant, q, k, v, do, got, *, causal=True, scale=None):
    B, H = q.shape[:2]
    reports = []
    for b in range(B):
        for h in range(H):
            gh = {key: got[key][b, h] for key in got}
            reports.append(parity.check_head(ocfg(variant), q[b, h], k[b, h], v[b, h], do[b, h], gh,
                                             causal=causal, scale=scale))
    return reports


# ------------------------------------------------------------------ the tiny workload
def test_tiny_workload(kb):
    wl = WORKLOADS["tiny"]
    q, k, v, do = wl.inputs()
    for var in wl.variants:
        variant = (var.calib, var.recon, var.ste, var.grad, var.K, var.tau)
        say(f"[tiny] {wl.B}x{wl.H}x{wl.T}x{wl.D} seed={wl.seed} {var.name}")
        got, _ = gpu_run(kb, variant, q, k, v, do)
        rep = compare_all_heads(variant, q, k, v, do, got)
        say("   ", rep)


# ------------------------------------------------------------------ every variant, several tiles + ragged tail
SMALL_SHAPES = [
    (1, 2, 200, 64, True, 11, "f32"),
    (2, 1, 77, 128, True, 12, "f32"),
    (1, 2, 96, 64, False, 13, "f32"),
    (1, 1, 161, 128, True, 14, "bf16"),
]


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s[:4])) + ("c" if s[4] else "n") + s[6])
@pytest.mark.parametrize("variant", VARIANTS16, ids=lambda v: "-".join(v))
def test_small_all_variants(kb, variant, shape):
    B, H, T, D, causal, seed, dtype = shape
    q, k, v, do = make_inputs(B, H, T, D, seed, dtype=dtype, q_scale=2.0)
    full = variant + (8, 5.0)
    say(f"[small] {shape} {full}")
    got, _ = gpu_run(kb, full, q, k, v, do, causal=causal, dtype=dtype)
    rep = compare_all_heads(full, q, k, v, do, got, causal=causal)
    say("   ", rep)


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s[:4])) + ("c" if s[4] else "n") + s[6])
@pytest.mark.parametrize("variant", ABLATIONS, ids=lambda v: "-".join(v))
def test_small_ablations(kb, variant, shape):
    B, H, T, D, causal, seed, dtype = shape
    q, k, v, do = make_inputs(B, H, T, D, seed, dtype=dtype, q_scale=2.0)
    full = variant + (8, 5.0)
    say(f"[ablation] {shape} {full}")
    got, _ = gpu_run(kb, full, q, k, v, do, causal=causal, dtype=dtype)
    rep = compare_all_heads(full, q, k, v, do, got, causal=causal)
    say("   ", rep)


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s[:4])) + ("c" if s[4] else "n") + s[6])
@pytest.mark.parametrize("variant", TAILS, ids=lambda v: "-".join(v))
def test_small_tail_policies(kb, variant, shape):
    """Floored and resolved FWM tails: tau = 3 at score std 2 puts many keys below the window."""
    B, H, T, D, causal, seed, dtype = shape
    q, k, v, do = make_inputs(B, H, T, D, seed, dtype=dtype, q_scale=2.0)
    full = variant[:4] + (8, 3.0, variant[4])
    say(f"[tail] {shape} {full}")
    got, _ = gpu_run(kb, full, q, k, v, do, causal=causal, dtype=dtype)
    rep = compare_all_heads(full, q, k, v, do, got, causal=causal)
    say("   ", rep)


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s[:4])) + ("c" if s[4] else "n") + s[6])
@pytest.mark.parametrize("variant", EXPS, ids=lambda v: "-".join(v))
def test_small_exp_baselines(kb, variant, shape):
    B, H, T, D, causal, seed, dtype = shape
    q, k, v, do = make_inputs(B, H, T, D, seed, dtype=dtype, q_scale=2.0)
    full = variant + (4, 8.0)
    say(f"[exp baseline] {shape} {full}")
    got, _ = gpu_run(kb, full, q, k, v, do, causal=causal, dtype=dtype)
    rep = compare_all_heads(full, q, k, v, do, got, causal=causal)
    say("   ", rep)


@pytest.mark.parametrize("shape", SMALL_SHAPES, ids=lambda s: "x".join(map(str, s[:4])) + ("c" if s[4] else "n") + s[6])
@pytest.mark.parametrize("variant", BINMEANS, ids=lambda v: "-".join(v))
def test_small_binmean(kb, variant, shape):
    B, H, T, D, causal, seed, dtype = shape
    q, k, v, do = make_inputs(B, H, T, D, seed, dtype=dtype, q_scale=2.0)
    full = variant + (4, 5.0)
    say(f"[bin mean] {shape} {full}")
    got, _ = gpu_run(kb, full, q, k, v, do, causal=causal, dtype=dtype)
    rep = compare_all_heads(full, q, k, v, do, got, causal=causal)
    say("   ", rep)


@pytest.mark.parametrize("variant", [("minmax", "binmean"), ("fwm", "binmean"), ("fwm", "nearest_binmean")],
                         ids=lambda v: "-".join(v))
@pytest.mark.parametrize("K", [1, 2, 8])
def test_binmean_bins_and_sizes(kb, variant, K):
    """Bin mean at K = 1, 2, 8 (the largest built): bins bit-exact and outputs at parity."""
    import torch
    q, k, v, do = make_inputs(1, 2, 150, 64, 22, q_scale=3.0)
    full = (variant[0], variant[1], "prob", "full", K, 3.0)
    say(f"[bin mean K] 1x2x150x64 seed=22 {full}")
    got, (qt, kt, rowrec, p) = gpu_run(kb, full, q, k, v, do)
    bins = kb.debug_bins(p, rowrec)
    torch.cuda.synchronize()
    bins = bins.cpu().numpy()
    for h in range(2):
        say("   ", parity.check_bins(ocfg(full), q[0, h], k[0, h], bins[0, h]))
    say("   ", compare_all_heads(full, q, k, v, do, got))


@pytest.mark.parametrize("K,tau", [(4, 6.0), (16, 2.0), (64, 1.0)])
@pytest.mark.parametrize("recon,ste", [("lerp", "prob"), ("nearest", "weight")])
def test_resolved_grid_depth(kb, recon, ste, K, tau):
    """Resolved grid far below the window: tau = 1, K = 64 needs more levels than the table holds
    (103 K / tau > 1024), so keys deeper than the table take the computed grid values."""
    B, H, T, D, seed = 1, 2, 130, 64, 61
    q, k, v, do = make_inputs(B, H, T, D, seed, q_scale=6.0)
    full = ("fwm", recon, ste, "full", K, tau, "resolved")
    say(f"[resolved depth] {B}x{H}x{T}x{D} seed={seed} {full}")
    got, _ = gpu_run(kb, full, q, k, v, do)
    rep = compare_all_heads(full, q, k, v, do, got)
    say("   ", rep)


@pytest.mark.parametrize("variant", [("minmax", "lerp"), ("minmax", "nearest"), ("fwm", "lerp"), ("fwm", "nearest"),
                                     ("fwm", "lerp", "floor"), ("fwm", "nearest", "floor"),
                                     ("fwm", "lerp", "resolved"), ("fwm", "nearest", "resolved"),
                                     ("fwm", "softmax"), ("fwm", "exp_bf16"), ("fwm", "exp_fp8")],
                         ids=lambda v: "-".join(v))
@pytest.mark.parametrize("K", [1, 4, 16, 64])
def test_bins_bitexact(kb, variant, K):
    import torch
    q, k, v, do = make_inputs(1, 2, 150, 64, 21, q_scale=3.0)
    tail = variant[2] if len(variant) > 2 else "zero"
    full = (variant[0], variant[1], "prob", "full", K, 3.0, tail)
    say(f"[bins] 1x2x150x64 seed=21 {full}")
    cfg = kb.Config(*full[:4], K=K, tau=3.0, tail=tail)
    qt, kt, vt = (torch.from_numpy(x).cuda() for x in (q, k, v))
    o, rowrec, p = kb.forward(cfg, qt, kt, vt)
    bins = kb.debug_bins(p, rowrec)
    torch.cuda.synchronize()
    bins = bins.cpu().numpy()
    for h in range(2):
        rep = parity.check_bins(ocfg(full), q[0, h], k[0, h], bins[0, h])
        say("   ", rep)


# ------------------------------------------------------------------ edge cases
def test_single_row_and_empty(kb):
    import torch
    for T in (1, 2, 31, 33):
        q, k, v, do = make_inputs(1, 1, T, 64, 30 + T)
        for variant in VARIANTS16[::3]:
            full = variant + (4, 8.0)
            say(f"[edge T={T}] {full}")
            got, _ = gpu_run(kb, full, q, k, v, do)
            compare_all_heads(full, q, k, v, do, got)
            if T == 1:
                assert np.array_equal(got["O"][0, 0, 0], v[0, 0, 0].astype(np.float64))
    # empty inputs: nothing to do, no launch, status OK
    cfg = kb.Config()
    for shape in ((0, 2, 16, 64), (1, 0, 16, 64), (1, 1, 0, 64)):
        say(f"[edge empty] {shape}")
        z = torch.zeros(shape, device="cuda")
        o, rowrec, p = kb.forward(cfg, z, z, z)
        dq, dk, dv = kb.backward(p, z, z, z, o, z, rowrec)
        assert o.numel() == 0 or o.shape == z.shape


def test_degenerate_rows(kb):
    # Q = 0: every score is 0, every MinMax row degenerate (uniform P, zero score gradient)
    q, k, v, do = make_inputs(1, 1, 70, 64, 40)
    q[:] = 0.0
    for variant in VARIANTS16:
        full = variant + (4, 8.0)
        say(f"[degenerate] {full}")
        got, _ = gpu_run(kb, full, q, k, v, do)
        compare_all_heads(full, q, k, v, do, got)
        if variant[0] == "minmax":
            assert np.all(np.abs(got["dQ"]) <= 1e-6) and np.all(np.abs(got["dK"]) <= 1e-6)


def test_tied_extrema(kb):
    # duplicated key rows tie the maximum (and minimum) of many rows
    q, k, v, do = make_inputs(1, 2, 100, 64, 41, q_scale=2.0)
    k[0, :, 3] *= 3.0                      # key 3 holds the max or the min of most rows
    k[0, :, 10] = k[0, :, 3]
    k[0, :, 50] = k[0, :, 3]
    k[0, :, 60] = k[0, :, 20]
    for variant in VARIANTS16:
        full = variant + (4, 8.0)
        say(f"[ties] {full}")
        got, _ = gpu_run(kb, full, q, k, v, do)
        compare_all_heads(full, q, k, v, do, got)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_tied_extrema_in_one_lane(kb, dtype):
    """Copies of one key 64 apart fall to the same wave and lane for every row that sees them: that
    lane holds up to nine tied candidates of the maximum (and, for another key, of the minimum) and
    rescans its ten tiles in batches; D = 128.  The changes keep K exact in bf16 (x4, negation)."""
    q, k, v, do = make_inputs(1, 2, 600, 128, 73, dtype=dtype, q_scale=2.0)
    k[0, :, 3] *= 4.0
    k[0, :, 20] = -k[0, :, 3]
    for j in range(1, 9):
        k[0, :, 3 + 64 * j] = k[0, :, 3]
        k[0, :, 20 + 64 * j] = k[0, :, 20]
    for variant in [("minmax", "lerp", "prob", "full"), ("minmax", "nearest", "weight", "full"),
                    ("fwm", "nearest", "prob", "full")]:
        full = variant + (4, 8.0)
        say(f"[lane-ties] 1x2x600x128 {dtype} seed=73 {full}")
        got, _ = gpu_run(kb, full, q, k, v, do, dtype=dtype)
        compare_all_heads(full, q, k, v, do, got)


def grid_inputs(seed, B, H, T, D, rel):
    """Q, K on the integers -2..2 times (1 + rel N(0,1)): the scores sit on a coarse grid (and the
    row extrema and interval boundaries with them) up to a perturbation of relative size rel."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-2, 3, (B, H, T, D)).astype(np.float32)
    k = rng.integers(-2, 3, (B, H, T, D)).astype(np.float32)
    q *= (1.0 + rel * rng.standard_normal(q.shape)).astype(np.float32)
    k *= (1.0 + rel * rng.standard_normal(k.shape)).astype(np.float32)
    v = rng.standard_normal((B, H, T, D)).astype(np.float32)
    do = rng.standard_normal((B, H, T, D)).astype(np.float32)
    return q, k, v, do


@pytest.mark.parametrize("variant", [("minmax", "lerp", "prob", "full", 4, 8.0),
                                     ("minmax", "nearest", "weight", "full", 8, 8.0),
                                     ("fwm", "nearest", "prob", "full", 4, 2.0),
                                     ("fwm", "lerp", "prob", "full", 16, 3.0)],
                         ids=lambda v: "-".join(str(x) for x in v))
def test_near_boundary_scores(kb, variant):
    # Many decisions fall within the error bound of the forward's bf16 slice-product scores but
    # farther from the boundary than the parity guard: they agree with the oracle only if the
    # forward retakes them on exactly recomputed scores (and patches those into the stored
    # tiles that the backward and the bins hook read).
    import torch
    q, k, v, do = grid_inputs(50, 1, 2, 96, 64, 3e-6)
    say(f"[near-boundary] 1x2x96x64 grid seed=50 {variant}")
    got, (qt, kt, rowrec, p) = gpu_run(kb, variant, q, k, v, do)
    compare_all_heads(variant, q, k, v, do, got)
    bins = kb.debug_bins(p, rowrec)
    torch.cuda.synchronize()
    bins = bins.cpu().numpy()
    for h in range(2):
        say("   ", parity.check_bins(ocfg(variant), q[0, h], k[0, h], bins[0, h]))


def test_near_tied_extrema(kb):
    # keys that are copies of one another up to a relative 1e-7: row maxima / minima closer than
    # the score bound, settled by recomputing every candidate exactly
    q, k, v, do = make_inputs(1, 2, 100, 64, 51, q_scale=2.0)
    k[0, :, 3] *= 3.0
    rng = np.random.default_rng(52)
    for j in (10, 50, 77):
        k[0, :, j] = k[0, :, 3] * (1.0 + 1e-7 * rng.standard_normal(64)).astype(np.float32)
    for variant in [v_ + (4, 8.0) for v_ in VARIANTS16[::2]]:
        say(f"[near-ties] {variant}")
        got, _ = gpu_run(kb, variant, q, k, v, do)
        reps = compare_all_heads(variant, q, k, v, do, got)
        # nothing is excluded: every element of every row is compared, near-tied rows included
        assert all(r["elements"] == 4 * q[0, 0].size for r in reps)
        say("    near ties flagged:", [r["ties"] for r in reps], "flips:", [r["flips"] for r in reps])


def test_window_and_scale_extremes(kb):
    # tiny FWM window (most keys in the tail), large K, large scores
    q, k, v, do = make_inputs(1, 1, 128, 64, 42, q_scale=6.0)
    for variant in [("fwm", "nearest", "weight", "full", 2, 0.5), ("fwm", "lerp", "prob", "full", 64, 1.0),
                    ("minmax", "nearest", "prob", "full", 64, 8.0), ("minmax", "lerp", "prob", "detached", 1, 8.0)]:
        say(f"[extreme] {variant}")
        got, _ = gpu_run(kb, variant, q, k, v, do)
        compare_all_heads(variant, q, k, v, do, got)


def test_explicit_scale(kb):
    q, k, v, do = make_inputs(1, 1, 90, 128, 43)
    variant = ("minmax", "nearest", "weight", "full", 8, 8.0)
    say(f"[scale=0.125] {variant}")
    got, _ = gpu_run(kb, variant, q, k, v, do, scale=0.125)
    compare_all_heads(variant, q, k, v, do, got, scale=0.125)


@pytest.mark.parametrize("variant", [("minmax", "nearest", "prob", "full", 4, 8.0),
                                     ("fwm", "lerp", "prob", "p1", 8, 3.0, "resolved"),
                                     ("fwm", "exp_bf16", "prob", "full", 4, 8.0),
                                     ("minmax", "binmean", "prob", "full", 4, 8.0)], ids=lambda v: "-".join(map(str, v)))
def test_deterministic(kb, variant):
    """Repeated calls give bit-identical outputs: every sum runs in a fixed order (no atomics)."""
    q, k, v, do = make_inputs(2, 2, 130, 64, 44, q_scale=2.0)
    say(f"[determinism] {variant}")
    a, _ = gpu_run(kb, variant, q, k, v, do)
    b, _ = gpu_run(kb, variant, q, k, v, do)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
