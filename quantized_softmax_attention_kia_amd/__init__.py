"""K-interval attention (quantized softmax in attention) for AMD Instinct MI355X.

The forward and backward run in hand-written HIP kernels for gfx950 behind the
C ABI of include/kia.h (libkia.so); `binding` marshals torch tensors into it.
"""
__all__ = ["binding", "inputs"]
