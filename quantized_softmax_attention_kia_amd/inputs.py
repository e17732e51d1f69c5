"""Seeded synthetic inputs for K-interval attention workloads.

This module only draws random tensors; it holds none of the operator's
arithmetic, so that both the HIP path and the CPU oracle can consume the same
arrays without sharing any computation.

Recipe (a reading: the pages train GPT-2-style models on text corpora and do not
fix any synthetic input; the Gaussian draws below stand in for attention
activations of the pages' shapes, 12 heads x 64 at T=1024 for the 124M model):

* ``numpy.random.default_rng(seed)`` (PCG64); draws in the order Q, K, V, dO,
  each ``standard_normal`` float32 of shape [B, H, T, D].
* ``q_scale`` multiplies Q after the draw (score std = q_scale), emulating the
  widened row span that "Pretraining Transformers with Quantized Softmax in
  Attention" reports late in training (§5.4 and App. D.6: spans of 25-32 nats
  under softmax-like training, far wider under MinMax-Weight).
* ``outlier_frac`` > 0: after the four draws, for every (b, h) in order, choose
  round(outlier_frac * T) distinct key rows (``rng.choice`` without
  replacement) and redraw them as ``outlier_std * standard_normal``.
* ``dtype="bf16"``: every array is rounded to bfloat16 (round to nearest even)
  and returned as float32 holding bf16-representable values.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bias = ((bits >> 16) & 1) + 0x7FFF
    out = ((bits + bias) & 0xFFFF0000).astype(np.uint32)
    return out.view(np.float32)


def make_inputs(B: int, H: int, T: int, D: int, seed: int, *, dtype: str = "f32",
                q_scale: float = 1.0, outlier_frac: float = 0.0, outlier_std: float = 8.0):
    """Return float32 arrays (q, k, v, do), each [B, H, T, D] and C-contiguous."""
    rng = np.random.default_rng(seed)
    shape = (B, H, T, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    do = rng.standard_normal(shape, dtype=np.float32)
    if q_scale != 1.0:
        q *= np.float32(q_scale)
    if outlier_frac > 0.0:
        n_out = int(round(outlier_frac * T))
        for b in range(B):
            for h in range(H):
                rows = rng.choice(T, size=n_out, replace=False)
                k[b, h, rows, :] = np.float32(outlier_std) * rng.standard_normal((n_out, D), dtype=np.float32)
    if dtype == "bf16":
        q, k, v, do = (round_to_bf16(a) for a in (q, k, v, do))
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return q, k, v, do


@dataclass(frozen=True)
class Variant:
    """One operator configuration: calibration x reconstruction x surrogate x gradient mode."""
    calib: str          # "minmax" | "fwm"
    recon: str          # "lerp" | "nearest" | "softmax" | "exp_bf16" | "exp_fp8" | "binmean" | "nearest_binmean"
    ste: str            # "weight" | "prob" (Nearest only)
    grad: str           # "full" | "detached" | "max_only" | "min_only" | "p1"
    K: int
    tau: float = 8.0
    tail: str = "zero"  # FWM tail policy: "zero" | "floor" | "resolved"

    @property
    def name(self) -> str:
        if self.recon in ("softmax", "exp_bf16", "exp_fp8"):
            return f"{self.recon}-{self.grad}"
        ste = "" if self.recon in ("lerp", "binmean", "nearest_binmean") else f"-{self.ste}"
        cal = "minmax" if self.calib == "minmax" else f"fwm{self.tau:g}"
        if self.tail != "zero":
            cal += f"-{self.tail}"
        return f"{cal}-{self.recon}{ste}-K{self.K}-{self.grad}"


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    D: int
    seed: int
    dtype: str = "f32"
    q_scale: float = 1.0
    outlier_frac: float = 0.0
    variants: tuple = field(default_factory=tuple)

    def inputs(self):
        return make_inputs(self.B, self.H, self.T, self.D, self.seed, dtype=self.dtype,
                           q_scale=self.q_scale, outlier_frac=self.outlier_frac)

    @property
    def causal_pairs(self) -> int:
        return self.B * self.H * self.T * (self.T + 1) // 2


def _gpt2_variants():
    out = []
    for calib in ("minmax", "fwm"):
        out.append(Variant(calib, "lerp", "prob", "full", 4))
        for ste in ("weight", "prob"):
            out.append(Variant(calib, "nearest", ste, "full", 4))
    return tuple(out)


# The five workloads: a tiny case, the GPT-2-124M attention shape, the same shape with a
# widened score span, a 1B-style bf16 layer and a long-context case with outlier keys.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 64, 64, 0,
                     variants=(Variant("minmax", "lerp", "prob", "full", 4),)),
    "gpt2": Workload("gpt2", 8, 12, 1024, 64, 1, variants=_gpt2_variants()),
    "wide": Workload("wide", 8, 12, 1024, 64, 1, q_scale=4.0, variants=tuple(
        [Variant("fwm", "nearest", "prob", "full", K) for K in (16, 32)]
        + [Variant("minmax", "lerp", "prob", g, K) for K in (16, 32) for g in ("full", "detached")])),
    "1b": Workload("1b", 4, 16, 2048, 128, 2, dtype="bf16", variants=(
        Variant("minmax", "nearest", "weight", "full", 4),
        Variant("fwm", "nearest", "prob", "full", 4))),
    "long": Workload("long", 1, 16, 8192, 128, 3, outlier_frac=0.01, variants=(
        Variant("minmax", "lerp", "prob", "full", 32),
        Variant("minmax", "nearest", "weight", "full", 16),
        Variant("minmax", "nearest", "prob", "full", 16))),
}
