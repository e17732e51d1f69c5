"""The autograd wrapper (KIAttention / kia_attention): its forward and backward are the library's
kia_forward and kia_backward, its gradients come back in the inputs' dtype, and the float32 results
behind them equal the oracle's (every head, the parity harness).  float32 and bfloat16 inputs."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import parity
from oracle import oracle as ORC
from quantized_softmax_attention_kia_amd.inputs import Variant, make_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def kb():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_softmax_attention_kia_amd import binding
    return binding


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("var", [Variant("minmax", "nearest", "prob", "full", 4),
                                 Variant("fwm", "lerp", "prob", "full", 8, 8.0)], ids=lambda v: v.name)
def test_autograd_wrapper(kb, dtype, var):
    import torch
    B, H, T, D = 1, 2, 130, 64
    # bf16: every input already a bfloat16 value, so the oracle sees what the kernels see
    q, k, v, do = make_inputs(B, H, T, D, 31, dtype=dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    say(f"[autograd] {B}x{H}x{T}x{D} {dtype} {var.name}")
    qt, kt, vt = (torch.from_numpy(x).cuda().to(tdt).requires_grad_() for x in (q, k, v))
    dot = torch.from_numpy(do).cuda()
    cfg = kb.Config.of(var)
    o = kb.kia_attention(qt, kt, vt, cfg)
    assert o.dtype == torch.float32 and tuple(o.shape) == (B, H, T, D)
    (o * dot).sum().backward()
    for t in (qt, kt, vt):
        assert t.grad is not None and t.grad.dtype == tdt
    # the same calls made directly: the wrapper adds only the casts of the gradients
    with torch.no_grad():
        o2, rowrec, p = kb.forward(cfg, qt.detach(), kt.detach(), vt.detach())
        dq, dk, dv = kb.backward(p, qt.detach(), kt.detach(), vt.detach(), o2, dot.to(tdt), rowrec)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for name, g, ref in (("dQ", qt.grad, dq), ("dK", kt.grad, dk), ("dV", vt.grad, dv)):
        assert torch.equal(g, ref.to(tdt)), name
    # the float32 results against the oracle
    got = {key: x.cpu().numpy() for key, x in (("O", o2), ("dQ", dq), ("dK", dk), ("dV", dv))}
    ocfg = ORC.OracleConfig.of(var)
    for b, h in parity.all_heads(q):
        parity.check_head(ocfg, q[b, h], k[b, h], v[b, h], do[b, h],
                          {key: got[key][b, h].astype(np.float64) for key in got})
