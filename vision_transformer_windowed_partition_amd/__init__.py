"""Shifted / interleaved window attention forward for one MI355X (gfx950).

The compute lives in ``libswinattn.so`` (hand-written HIP kernels behind a C
ABI declared in ``include/swin_attn.h``).  ``binding`` marshals torch tensors
onto that ABI and nothing more; ``synth`` draws seeded synthetic inputs.
"""
from . import synth  # noqa: F401

__all__ = ["synth"]
