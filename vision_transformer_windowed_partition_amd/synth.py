"""Seeded synthetic inputs and the workload table.

This module only draws random numbers; it holds none of the attention
arithmetic.  The GPU path and the CPU oracle both read what it returns.

Workloads (stage-1 attention activations of the models on the pages, at their
sizes; seeded N(0, 1) activations stand in for image data):

  0  SwinV2-T stage 1, fp32 parity case: 1 x 64 x 64 x 96, 3 heads, M=8,
     shift 4, scaled cosine attention + log-CPB bias (MLP 2 -> 512 -> 3)
  1  SwinV2-T stage 1 at 256 px, bf16: 64 x 64 x 64 x 96, 3 heads, M=16,
     shift 8, scaled cosine + log-CPB (the headline workload)
  2  Iwin-style interleaved windows, bf16: 64 x 64 x 64 x 192, 6 heads, M=8,
     dot-product attention / sqrt(32), no bias, no shift
  3  FlashSwin dense tokens, bf16: 32 x 128 x 128 x 96, 3 heads, M=32,
     shift 16, dot-product / sqrt(32) with window-local 2D RoPE (base 10000)
  4  SwinV2 1536 px stage-1 share, bf16: 1 x 384 x 384 x 512, 16 heads, M=24,
     shift 12, scaled cosine + log-CPB (MLP 2 -> 512 -> 16)

Draw order (fixed for every workload, so the generator state never depends on
the mode): q, k, v each randn(B, H, W, C) in fp32; log tau ~ U(ln 0.1, ln 1)
per head, tau = exp(log tau) clamped at 0.01; then w1 (512 x 2), b1 (512),
w2 (heads x 512), b2 (heads), each 0.02 * randn.  bf16 workloads round q, k, v
to bf16 (round to nearest even).  Seed = workload index unless given.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    W: int
    C: int
    heads: int
    M: int
    shift: int
    partition: str          # "cyclic" | "interleaved"
    sim: str                # "cosine" | "dot"
    pos: str                # "none" | "table" | "rope2d"
    dtype: str              # "f32" | "bf16"
    hidden: int = 512
    rope_base: float = 10000.0

    @property
    def d(self) -> int:
        return self.C // self.heads

    @property
    def N(self) -> int:
        return self.M * self.M

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.W

    @property
    def n_windows(self) -> int:
        return self.B * (self.H // self.M) * (self.W // self.M)

    @property
    def elem_size(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def flops(self) -> int:
        """4 N C flops per token: QK^T and PV, 2 per multiply-add, dense within
        the window (masked pairs included); softmax, norms, bias not counted."""
        return 4 * self.tokens * self.N * self.C

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: q, k, v read once and o written once."""
        return 4 * self.tokens * self.C * self.elem_size

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = [
    Workload("swinv2t_s1_fp32_m8", 1, 64, 64, 96, 3, 8, 4, "cyclic", "cosine", "table", "f32"),
    Workload("swinv2t_s1_256px_m16", 64, 64, 64, 96, 3, 16, 8, "cyclic", "cosine", "table", "bf16"),
    Workload("iwin_interleaved_m8", 64, 64, 64, 192, 6, 8, 0, "interleaved", "dot", "none", "bf16"),
    Workload("flashswin_dense_m32_rope", 32, 128, 128, 96, 3, 32, 16, "cyclic", "dot", "rope2d", "bf16"),
    Workload("swinv2_1536px_s1_m24", 1, 384, 384, 512, 16, 24, 12, "cyclic", "cosine", "table", "bf16"),
]


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_inputs(wl: Workload, seed: int | None = None, tau_range=(0.1, 1.0)) -> dict:
    """Draw one workload's inputs on the CPU (see the module docstring).

    Returns a dict of CPU tensors: q, k, v (workload dtype, (B, H, W, C)),
    tau (heads, fp32), w1 (hidden, 2), b1 (hidden), w2 (heads, hidden),
    b2 (heads), all fp32.
    """
    if seed is None:
        seed = next((i for i, w in enumerate(WORKLOADS) if w.name == wl.name), 0)
    g = torch.Generator().manual_seed(int(seed))
    shape = (wl.B, wl.H, wl.W, wl.C)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    lo, hi = math.log(tau_range[0]), math.log(tau_range[1])
    log_tau = torch.rand(wl.heads, generator=g, dtype=torch.float32) * (hi - lo) + lo
    tau = torch.exp(log_tau).clamp_min(0.01)
    w1 = 0.02 * torch.randn(wl.hidden, 2, generator=g, dtype=torch.float32)
    b1 = 0.02 * torch.randn(wl.hidden, generator=g, dtype=torch.float32)
    w2 = 0.02 * torch.randn(wl.heads, wl.hidden, generator=g, dtype=torch.float32)
    b2 = 0.02 * torch.randn(wl.heads, generator=g, dtype=torch.float32)
    dt = torch_dtype(wl.dtype)
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), tau=tau, w1=w1, b1=b1, w2=w2, b2=b2)


def make_dout(wl: Workload, seed: int = 1000):
    """Gradient of a loss with respect to the attention output, for backward
    tests: N(0, 1) of the output's shape, in the workload dtype (CPU)."""
    g = torch.Generator().manual_seed(int(seed))
    d = torch.randn((wl.B, wl.H, wl.W, wl.C), generator=g, dtype=torch.float32)
    return d.to(torch_dtype(wl.dtype))


def make_branch_params(wl: Workload, seed: int = 2000, T: int | None = None) -> dict:
    """Inputs of the attention branch's linear layers and post-norm, drawn in
    this order (CPU, fp32): x (T, C) features, o (T, C) attention output,
    w_qkv (3C, C) and w_proj (C, C) each randn / sqrt(C), b_qkv (3C) and
    b_proj (C) each 0.1 randn, gamma = 1 + 0.1 randn (C), beta = 0.1 randn (C),
    then the convolution branch's taps w_dw (C, 3, 3) = randn / 3 and bias
    b_dw (C) = 0.1 randn.  x, o and the linear weights are rounded to the
    workload dtype; biases, gamma, beta and the taps stay fp32.  T defaults to
    the workload's B H W tokens."""
    g = torch.Generator().manual_seed(int(seed))
    C = wl.C
    T = wl.B * wl.H * wl.W if T is None else int(T)
    dt = torch_dtype(wl.dtype)
    x = torch.randn((T, C), generator=g)
    o = torch.randn((T, C), generator=g)
    w_qkv = torch.randn((3 * C, C), generator=g) / math.sqrt(C)
    w_proj = torch.randn((C, C), generator=g) / math.sqrt(C)
    b_qkv = 0.1 * torch.randn(3 * C, generator=g)
    b_proj = 0.1 * torch.randn(C, generator=g)
    gamma = 1.0 + 0.1 * torch.randn(C, generator=g)
    beta = 0.1 * torch.randn(C, generator=g)
    w_dw = torch.randn((C, 3, 3), generator=g) / 3.0
    b_dw = 0.1 * torch.randn(C, generator=g)
    return dict(x=x.to(dt), o=o.to(dt), w_qkv=w_qkv.to(dt), w_proj=w_proj.to(dt), b_qkv=b_qkv, b_proj=b_proj,
                gamma=gamma, beta=beta, w_dw=w_dw, b_dw=b_dw)


def small(name: str = "tiny", *, B=2, H=16, W=16, C=64, heads=2, M=8, shift=4,
          partition="cyclic", sim="cosine", pos="table", dtype="f32", hidden=64) -> Workload:
    """A small workload for tests (same draw recipe)."""
    return Workload(name, B, H, W, C, heads, M, shift, partition, sim, pos, dtype, hidden)


@dataclass(frozen=True)
class VideoWorkload:
    """A video (3D) window workload: (B, T, H, W, C) tokens, windows Mt x M x M."""
    name: str
    B: int
    T: int
    H: int
    W: int
    C: int
    heads: int
    Mt: int
    M: int
    shift_t: int
    shift: int
    partition: str
    sim: str
    pos: str                # "none" | "table"
    dtype: str
    hidden: int = 512

    @property
    def N(self) -> int:
        return self.Mt * self.M * self.M

    @property
    def tokens(self) -> int:
        return self.B * self.T * self.H * self.W

    @property
    def elem_size(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def flops(self) -> int:
        """4 N C flops per token (QK^T and PV, dense within the window)."""
        return 4 * self.tokens * self.N * self.C

    @property
    def bytes(self) -> int:
        """q, k, v read once and o written once."""
        return 4 * self.tokens * self.C * self.elem_size


# The SwinV2 video fine-tuning shapes (appendix A2, Kinetics-400 stages 1
# and 2: 256^2 x 8 frames with 16^2 x 8 windows, 320^2 x 8 frames with
# 20^2 x 8 windows) at the first stage of a Tiny backbone (4 x 4 patches: a
# 64 x 64 or 80 x 80 grid per frame, C = 96, 3 heads), 8 clips, the spatial
# shift M/2 of a shifted block.
VIDEO_WORKLOADS = [
    VideoWorkload("swinv2t_k400_8x256px_w16x8", 8, 8, 64, 64, 96, 3, 8, 16, 0, 8, "cyclic", "cosine", "table",
                  "bf16"),
    VideoWorkload("swinv2t_k400_8x320px_w20x8", 8, 8, 80, 80, 96, 3, 8, 20, 0, 10, "cyclic", "cosine", "table",
                  "bf16"),
]


def make_video_inputs(wl: VideoWorkload, seed: int = 0, tau_range=(0.1, 1.0)) -> dict:
    """q, k, v (B, T, H, W, C) N(0, 1) in the workload dtype; tau as for the 2D
    workloads; the meta network w1 (hidden, 3), b1, w2, b2 at 0.02 N(0, 1)."""
    g = torch.Generator().manual_seed(int(seed))
    shape = (wl.B, wl.T, wl.H, wl.W, wl.C)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    lo, hi = math.log(tau_range[0]), math.log(tau_range[1])
    tau = torch.exp(torch.rand(wl.heads, generator=g, dtype=torch.float32) * (hi - lo) + lo).clamp_min(0.01)
    w1 = 0.02 * torch.randn(wl.hidden, 3, generator=g, dtype=torch.float32)
    b1 = 0.02 * torch.randn(wl.hidden, generator=g, dtype=torch.float32)
    w2 = 0.02 * torch.randn(wl.heads, wl.hidden, generator=g, dtype=torch.float32)
    b2 = 0.02 * torch.randn(wl.heads, generator=g, dtype=torch.float32)
    dt = torch_dtype(wl.dtype)
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), tau=tau, w1=w1, b1=b1, w2=w2, b2=b2)
