"""MI355X-native MoE feed-forward layer: sigmoid top-k router, expert-order
permutation, grouped SwiGLU experts plus a shared expert, weighted combine.

The compute runs in hand-written HIP kernels behind the C ABI of ``libmoe.so``
(declared in ``include/moe.h``); ``binding`` marshals torch tensors into it.
"""
from . import configs  # noqa: F401

__all__ = ["configs"]
