"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: the whole batch runs on the GPU and every head is compared
element by element against the oracle, which computes each head independently.
Black-box invariants are checked on every head."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import parity
from oracle import oracle as ORC
from quantized_softmax_attention_kia_amd.inputs import WORKLOADS

pytestmark = pytest.mark.gpu

CASES = [(wl, i) for wl in ("gpt2", "wide", "1b", "long") for i in range(len(WORKLOADS[wl].variants))]


@pytest.fixture(scope="module")
def kb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_softmax_attention_kia_amd import binding
    return binding


_inputs = {}


def inputs(name):
    if name not in _inputs:
        _inputs.clear()
        _inputs[name] = WORKLOADS[name].inputs()
    return _inputs[name]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def compare_heads(cfg, q, k, v, do, got, heads=None):
    """Every listed head (all by default) against the oracle; one summary line."""
    heads = parity.all_heads(q) if heads is None else heads
    out = {key: got[key].cpu().numpy() for key in ("O", "dQ", "dK", "dV")}
    flips = ties = flagged = bad0 = 0
    for b, h in heads:
        gh = {key: out[key][b, h].astype(np.float64) for key in out}
        rep = parity.check_head(cfg, q[b, h], k[b, h], v[b, h], do[b, h], gh)
        flips += len(rep["flips"])
        ties += rep["ties"]
        flagged += rep["nflags"]
        bad0 = max(bad0, rep["bad0"])
    say(f"    {len(heads)} heads equal to the oracle: {flips} flips at {flagged} flagged positions "
        f"({ties} near ties); most elements outside tolerance before flips in one head: {bad0}")


def run(kb, wl, var, q, k, v, do, detach=False):
    import torch
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    cfg = kb.Config.of(var)
    if detach:
        import dataclasses
        cfg = dataclasses.replace(cfg, grad="detached")
    qt, kt, vt, dot = (torch.from_numpy(x).cuda().to(tdt) for x in (q, k, v, do))
    o, rowrec, p = kb.forward(cfg, qt, kt, vt)
    dq, dk, dv = kb.backward(p, qt, kt, vt, o, dot, rowrec)
    torch.cuda.synchronize()
    return dict(O=o, dQ=dq, dK=dk, dV=dv, rowrec=rowrec)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{WORKLOADS[c[0]].variants[c[1]].name}")
def test_workload_all_heads(kb, case):
    name, i = case
    wl = WORKLOADS[name]
    var = wl.variants[i]
    q, k, v, do = inputs(name)
    say(f"[{name}] B={wl.B} H={wl.H} T={wl.T} D={wl.D} {wl.dtype} seed={wl.seed} {var.name}")
    got = run(kb, wl, var, q, k, v, do)
    cfg = ORC.OracleConfig.of(var)
    compare_heads(cfg, q, k, v, do, got)
    # invariants on every head: row sums of P are 1 (V = 1 gives O = 1 is the same check on O's
    # normalization), the full gradient's dK sums to zero over the keys of a head
    if var.grad == "full":
        dk = got["dK"].double()
        ratio = (dk.sum(dim=2).abs() / dk.abs().sum(dim=2).clamp_min(1e-30)).max().item()
        say(f"    max_h |sum_j dK_j| / sum_j |dK_j| = {ratio:.2e}")
        assert ratio < 1e-4, ratio


@pytest.mark.parametrize("grad", ["max_only", "min_only", "p1"])
def test_gpt2_ablations_all_heads(kb, grad):
    """The range_grad ablations at the benchmark shape: every head against the oracle; under
    P1 every head's dK sums to zero over its keys (each score-gradient row sums to zero)."""
    import dataclasses
    wl = WORKLOADS["gpt2"]
    var = dataclasses.replace(wl.variants[0], grad=grad)   # MinMax LERP K=4
    q, k, v, do = inputs("gpt2")
    say(f"[gpt2 ablation] B={wl.B} H={wl.H} T={wl.T} D={wl.D} seed={wl.seed} {var.calib}-{var.recon} {grad}")
    got = run(kb, wl, var, q, k, v, do)
    cfg = ORC.OracleConfig.of(var)
    compare_heads(cfg, q, k, v, do, got)
    if grad == "p1":
        dk = got["dK"].double()
        ratio = (dk.sum(dim=2).abs() / dk.abs().sum(dim=2).clamp_min(1e-30)).max().item()
        say(f"    max_h |sum_j dK_j| / sum_j |dK_j| = {ratio:.2e}")
        assert ratio < 1e-4, ratio


@pytest.mark.parametrize("tail", ["floor", "resolved"])
@pytest.mark.parametrize("ste", ["weight", "prob"])
def test_wide_tail_policies_all_heads(kb, tail, ste):
    """The tail-policy runs of the pages (hard Nearest, K = 4, tau = 6, both surrogates) on the
    wide-span inputs, where many keys fall below the window: every head against the oracle,
    and the full gradient's dK sums to zero over each head's keys."""
    from quantized_softmax_attention_kia_amd.inputs import Variant
    wl = WORKLOADS["wide"]
    var = Variant("fwm", "nearest", ste, "full", 4, 6.0, tail)
    q, k, v, do = inputs("wide")
    say(f"[wide tail] B={wl.B} H={wl.H} T={wl.T} D={wl.D} seed={wl.seed} {var.name}")
    got = run(kb, wl, var, q, k, v, do)
    cfg = ORC.OracleConfig.of(var)
    compare_heads(cfg, q, k, v, do, got)
    dk = got["dK"].double()
    ratio = (dk.sum(dim=2).abs() / dk.abs().sum(dim=2).clamp_min(1e-30)).max().item()
    say(f"    max_h |sum_j dK_j| / sum_j |dK_j| = {ratio:.2e}")
    assert ratio < 1e-4, ratio


@pytest.mark.parametrize("recon", ["softmax", "exp_bf16", "exp_fp8"])
def test_gpt2_exp_baselines_all_heads(kb, recon):
    """The exponential baselines at the benchmark shape: every head against the oracle; the
    full gradient's dK sums to zero over each head's keys (the row maximum's term)."""
    from quantized_softmax_attention_kia_amd.inputs import Variant
    wl = WORKLOADS["gpt2"]
    var = Variant("fwm", recon, "prob", "full", 4)
    q, k, v, do = inputs("gpt2")
    say(f"[gpt2 exp baseline] B={wl.B} H={wl.H} T={wl.T} D={wl.D} seed={wl.seed} {recon}")
    got = run(kb, wl, var, q, k, v, do)
    cfg = ORC.OracleConfig.of(var)
    compare_heads(cfg, q, k, v, do, got)
    dk = got["dK"].double()
    ratio = (dk.sum(dim=2).abs() / dk.abs().sum(dim=2).clamp_min(1e-30)).max().item()
    say(f"    max_h |sum_j dK_j| / sum_j |dK_j| = {ratio:.2e}")
    assert ratio < 1e-4, ratio


@pytest.mark.parametrize("recon", ["binmean", "nearest_binmean"])
def test_gpt2_binmean_all_heads(kb, recon):
    """Bin mean and the hybrid at the benchmark shape (FWM, K = 4, the pages' setting): every head
    against the oracle; every head's dK sums to zero over its keys."""
    from quantized_softmax_attention_kia_amd.inputs import Variant
    wl = WORKLOADS["gpt2"]
    var = Variant("fwm", recon, "prob", "full", 4)
    q, k, v, do = inputs("gpt2")
    say(f"[gpt2 bin mean] B={wl.B} H={wl.H} T={wl.T} D={wl.D} seed={wl.seed} {recon}")
    got = run(kb, wl, var, q, k, v, do)
    cfg = ORC.OracleConfig.of(var)
    compare_heads(cfg, q, k, v, do, got)
    dk = got["dK"].double()
    ratio = (dk.sum(dim=2).abs() / dk.abs().sum(dim=2).clamp_min(1e-30)).max().item()
    say(f"    max_h |sum_j dK_j| / sum_j |dK_j| = {ratio:.2e}")
    assert ratio < 1e-4, ratio


@pytest.mark.parametrize("var", [("fwm", "nearest", "weight", "full", 4, 6.0, "resolved"),
                                 ("fwm", "softmax", "prob", "full", 4, 8.0, "zero"),
                                 ("minmax", "binmean", "prob", "full", 8, 8.0, "zero")],
                         ids=lambda v: f"{v[0]}-{v[1]}-{v[6]}")
def test_long_context_new_modes(kb, var):
    """The long-context workload (T = 8192, D = 128, 1% outlier keys) under a resolved FWM tail,
    the softmax baseline and bin mean: every head against the oracle."""
    from quantized_softmax_attention_kia_amd.inputs import Variant
    wl = WORKLOADS["long"]
    v = Variant(*var)
    q, k, vv, do = inputs("long")
    say(f"[long new modes] B={wl.B} H={wl.H} T={wl.T} D={wl.D} seed={wl.seed} {v.name}")
    got = run(kb, wl, v, q, k, vv, do)
    cfg = ORC.OracleConfig.of(v)
    compare_heads(cfg, q, k, vv, do, got)


def test_full_and_detached_forward_bitwise_identical(kb):
    wl = WORKLOADS["wide"]
    q, k, v, do = inputs("wide")
    for var in wl.variants:
        if var.grad != "full":
            continue
        say(f"[full-vs-detached] wide {var.name}")
        a = run(kb, wl, var, q, k, v, do)
        b = run(kb, wl, var, q, k, v, do, detach=True)
        import torch
        assert torch.equal(a["O"], b["O"]) and torch.equal(a["rowrec"], b["rowrec"])
        # detached drops the extremum terms: its dK no longer sums to zero per head
        dk = b["dK"].double()
        ratio = (dk.sum(dim=2).abs() / dk.abs().sum(dim=2).clamp_min(1e-30)).max().item()
        say(f"    detached max_h |sum_j dK_j| / sum_j |dK_j| = {ratio:.2e}")
        assert ratio > 1e-3


@pytest.mark.parametrize("var", [("minmax", "lerp", "prob", "full", 4, 8.0, "zero"),
                                 ("minmax", "nearest", "prob", "full", 4, 8.0, "zero"),
                                 ("fwm", "nearest", "weight", "full", 4, 8.0, "zero"),
                                 ("fwm", "lerp", "prob", "full", 16, 8.0, "resolved"),
                                 ("minmax", "binmean", "prob", "full", 8, 8.0, "zero"),
                                 ("fwm", "exp_bf16", "prob", "full", 4, 8.0, "zero"),
                                 ("fwm", "softmax", "prob", "full", 4, 8.0, "zero")],
                         ids=lambda v: f"{v[0]}-{v[1]}-{v[3]}-{v[6]}")
def test_split_forward_stages_match(kb, var):
    """kia_forward_scores then kia_forward_weights write the same bits as kia_forward (O and the whole
    row record, stored scores included), on the gpt2-shaped workload."""
    import torch
    from quantized_softmax_attention_kia_amd.inputs import Variant
    wl = WORKLOADS["gpt2"]
    q, k, v, do = inputs("gpt2")
    v_ = Variant(*var)
    say(f"[split forward] gpt2 {v_.name}")
    qt, kt, vt = (torch.from_numpy(x).cuda() for x in (q, k, v))
    o, rowrec, p = kb.forward(kb.Config.of(v_), qt, kt, vt)
    o2 = torch.full_like(o, float("nan"))
    rowrec2 = torch.zeros_like(rowrec)
    kb.kia_forward_scores(p, qt, kt, vt, rowrec2)
    kb.kia_forward_weights(p, qt, kt, vt, o2, rowrec2)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    assert torch.equal(rowrec, rowrec2)


def test_split_backward_stages_match(kb):
    import torch
    wl = WORKLOADS["gpt2"]
    q, k, v, do = inputs("gpt2")
    var = wl.variants[2]
    say(f"[split stages] gpt2 {var.name}")
    qt, kt, vt, dot = (torch.from_numpy(x).cuda() for x in (q, k, v, do))
    o, rowrec, p = kb.forward(kb.Config.of(var), qt, kt, vt)
    dq, dk, dv = kb.backward(p, qt, kt, vt, o, dot, rowrec)
    _, ws = kb.kia_workspace_size(p)
    work = torch.empty(ws, device="cuda", dtype=torch.uint8)
    dq2, dk2, dv2 = (torch.empty_like(dq) for _ in range(3))
    kb.kia_backward_dq(p, qt, kt, vt, o, dot, rowrec, dq2, work)
    kb.kia_backward_dkdv(p, qt, kt, vt, dot, rowrec, dk2, dv2, work)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_shift_and_constant_value_invariance(kb):
    import torch
    wl = WORKLOADS["gpt2"]
    q, k, v, do = inputs("gpt2")
    var = wl.variants[0]          # MinMax LERP: the forward is continuous in the scores
    say(f"[invariance] gpt2 {var.name}")
    base = run(kb, wl, var, q, k, v, do)
    shift = np.random.default_rng(5).standard_normal(wl.D).astype(np.float32) * 0.25
    moved = run(kb, wl, var, q, k + shift, v, do)
    err = (moved["O"] - base["O"]).abs() - (1e-5 + 2e-4 * base["O"].abs())
    assert (err <= 0).all(), err.max().item()
    ones = run(kb, wl, var, q, k, np.ones_like(v), do)
    assert torch.allclose(ones["O"], torch.ones_like(ones["O"]), atol=2e-6, rtol=0)
