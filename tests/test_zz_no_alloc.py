"""kia_backward_noalloc (the backward on the library's built-in workspace) against kia_backward
with a caller's workspace: the same kernels on the same inputs, so the results must be identical.
Two calls in a row, the second smaller and in another mode, each against its own kia_backward."""
from __future__ import annotations

import sys

import numpy as np
import pytest

from quantized_softmax_attention_kia_amd.inputs import make_inputs

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


def one_call(kb, shape, variant, seed, dtype_name="f32"):
    import torch
    B, H, T, D = shape
    q, k, v, do = make_inputs(B, H, T, D, seed, dtype=dtype_name)
    tdt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    qt, kt, vt, dot = (torch.from_numpy(x).cuda().to(tdt) for x in (q, k, v, do))
    cfg = kb.Config(*variant[:4], K=variant[4], tau=variant[5])
    o, rowrec, p = kb.forward(cfg, qt, kt, vt)
    _, ws = kb.kia_workspace_size(p)
    assert ws <= kb.NOALLOC_WS_BYTES, "the test shapes fit the built-in workspace"
    say(f"[noalloc] shape={shape} {dtype_name} variant={variant} workspace={ws} bytes")
    work = torch.empty(ws, device="cuda", dtype=torch.uint8)
    ref = [torch.empty_like(o) for _ in range(3)]
    kb.kia_backward(p, qt, kt, vt, o, dot, rowrec, *ref, work)
    got = [torch.full_like(o, float("nan")) for _ in range(3)]
    kb.kia_backward_noalloc(p, qt, kt, vt, o, dot, rowrec, *got)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"{name}: max |diff| {(a - b).abs().max().item()}"


def test_noalloc_matches_backward_on_two_calls(kb):
    # the first call fills more of the array than the second reads
    one_call(kb, (2, 3, 384, 64), ("minmax", "lerp", "prob", "full", 4, 8.0), seed=11)
    one_call(kb, (1, 2, 150, 128), ("fwm", "nearest", "weight", "full", 4, 8.0), seed=12)
    one_call(kb, (1, 1, 97, 64), ("minmax", "nearest", "prob", "p1", 8, 8.0), seed=13, dtype_name="bf16")


def test_noalloc_rejects_a_workspace_beyond_its_array(kb):
    import torch
    # 64 heads of T = 1024: 64 x 528 causal tiles x 8 KiB of P and dS tiles, beyond the 64 MiB array
    p = kb.Params(B=4, H=16, T=1024, D=64, causal=1, K=4, tau=8.0, scale=0.125, calib=0, recon=0, ste=0,
                  grad=0, dtype=0, tail=0)
    _, ws = kb.kia_workspace_size(p)
    assert ws > kb.NOALLOC_WS_BYTES
    x = torch.zeros((4, 16, 1024, 64), device="cuda")
    rr, _ = kb.kia_workspace_size(p)
    rowrec = torch.zeros(rr, device="cuda", dtype=torch.uint8)
    with pytest.raises(kb.KiaError, match="KIA_ERR_WORKSPACE"):
        kb.kia_backward_noalloc(p, x, x, x, x, x, rowrec, x, x, x)
