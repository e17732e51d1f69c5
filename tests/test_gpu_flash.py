"""The one-pass (online-rescale) exact-softmax kernels against the oracle's softmax (App. B
"Softmax"): small shapes with several tiles and ragged tails (causal and not, fp32 and bf16, D = 64
and 128), the scale argument, and every head of the gpt2-shaped, wide and 1b workloads at their full
sizes.  The harness is the one the K-interval kernels are held to (1e-5 + 2e-4 |x| on every element
of O, dQ, dK, dV)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import parity
from oracle import oracle as ORC
from quantized_softmax_attention_kia_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

SOFTMAX = ORC.OracleConfig("fwm", "softmax", "prob", "full", 4)


@pytest.fixture(scope="module")
def kb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_softmax_attention_kia_amd import binding
    return binding


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def flash_run(kb, q, k, v, do, *, causal=True, scale=0.0, dtype="f32"):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cfg = kb.Config("fwm", "softmax", "prob", "full", 4, causal=causal, scale=scale)
    qt, kt, vt, dot = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(tdt) for x in (q, k, v, do))
    o, rowstats, p = kb.flash_forward(cfg, qt, kt, vt)
    dq, dk, dv = kb.flash_backward(p, qt, kt, vt, o, dot, rowstats)
    torch.cuda.synchronize()
    return {key: t.cpu().numpy().astype(np.float64) for key, t in (("O", o), ("dQ", dq), ("dK", dk), ("dV", dv))}


def compare(q, k, v, do, got, *, causal=True, scale=None):
    flips = 0
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            rep = parity.check_head(SOFTMAX, q[b, h], k[b, h], v[b, h], do[b, h], {x: got[x][b, h] for x in got},
                                    causal=causal, scale=scale)
            flips += len(rep["flips"])
    return flips


SMALL = [
    (1, 2, 200, 64, True, 41, "f32"),
    (2, 1, 77, 128, True, 42, "f32"),
    (1, 2, 96, 64, False, 43, "f32"),
    (1, 1, 161, 128, True, 44, "bf16"),
    (1, 1, 1, 64, True, 45, "f32"),
    (1, 3, 33, 64, False, 46, "bf16"),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s[:4])) + ("c" if s[4] else "n") + s[6])
def test_flash_small(kb, shape):
    B, H, T, D, causal, seed, dtype = shape
    q, k, v, do = make_inputs(B, H, T, D, seed, dtype=dtype, q_scale=3.0)
    say(f"[flash small] {B}x{H}x{T}x{D} causal={causal} {dtype} seed={seed}")
    got = flash_run(kb, q, k, v, do, causal=causal, dtype=dtype)
    say(f"    flips {compare(q, k, v, do, got, causal=causal)}")


def test_flash_scale_argument(kb):
    q, k, v, do = make_inputs(1, 2, 70, 64, 47)
    say("[flash scale] 1x2x70x64 scale=0.3")
    got = flash_run(kb, q, k, v, do, scale=0.3)
    compare(q, k, v, do, got, scale=0.3)


@pytest.mark.parametrize("wl_name", ["gpt2", "wide", "1b"])
def test_flash_workload_all_heads(kb, wl_name):
    wl = WORKLOADS[wl_name]
    q, k, v, do = wl.inputs()
    say(f"[flash {wl_name}] B={wl.B} H={wl.H} T={wl.T} D={wl.D} {wl.dtype} seed={wl.seed}: every head")
    got = flash_run(kb, q, k, v, do, dtype=wl.dtype)
    say(f"    {wl.B * wl.H} heads equal to the oracle; flips {compare(q, k, v, do, got)}")


def test_flash_rejects_other_reconstructions(kb):
    import torch
    q = torch.zeros((1, 1, 40, 64), device="cuda")
    cfg = kb.Config("minmax", "lerp", "prob", "full", 4)
    with pytest.raises(kb.KiaError, match="UNSUPPORTED"):
        kb.flash_forward(cfg, q, q, q)
