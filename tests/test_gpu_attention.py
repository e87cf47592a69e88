"""GPU parity of the window-attention forward against the fp64 oracle, on the
same seeded inputs, through the C ABI.

Bars (written here, from the targets stated for this path): fp32 mode
max-abs <= 1e-5; bf16 mode max-abs <= 2e-2 and relative Frobenius <= 1e-2.
Small cases span several tiles and ragged tails for every mode combination;
the five workloads run at full size in the launch configuration the
benchmark times, compared in full where the oracle is quick and on windows
sampled from every shift-mask class otherwise."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import (compare, f64, gpu_inputs, gpu_table, run_gpu, run_oracle,
                               sample_windows, window_token_mask)
from vision_transformer_windowed_partition_amd import binding, synth

pytestmark = pytest.mark.gpu

SMALL = [
    # H, W, M, shift, partition, sim, pos
    (32, 32, 8, 4, "cyclic", "cosine", "table"),
    (32, 32, 16, 8, "cyclic", "cosine", "table"),
    (32, 48, 8, 0, "interleaved", "dot", "none"),
    (64, 64, 32, 16, "cyclic", "dot", "rope2d"),
    (48, 48, 24, 12, "cyclic", "cosine", "table"),
    (28, 28, 7, 3, "cyclic", "cosine", "table"),       # odd window: padded key rows
    (24, 24, 12, 5, "cyclic", "dot", "table"),         # 12 -> 16 slots per key row
    (16, 16, 4, 2, "cyclic", "dot", "rope2d"),
    (16, 16, 2, 1, "cyclic", "cosine", "none"),
    (32, 32, 16, 0, "cyclic", "cosine", "rope2d"),
    (40, 40, 20, 10, "cyclic", "cosine", "table"),     # 480 slots: two key blocks
    (48, 48, 48, 24, "cyclic", "dot", "none"),         # 2304 tokens per window
    (32, 32, 16, 0, "interleaved", "cosine", "table"),
    (24, 40, 8, 7, "cyclic", "dot", "none"),           # shift M-1
    (30, 30, 10, 0, "interleaved", "cosine", "none"),  # 10 -> 16 slots per row, 6 key chunks
    (26, 26, 13, 6, "cyclic", "dot", "table"),         # 208 of 256 slots in use
    (34, 34, 17, 8, "cyclic", "dot", "none"),          # 17 -> 24 slots per row, 408 -> 416 slots
    (48, 48, 24, 0, "interleaved", "dot", "table"),    # interleaved large windows
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}x{c[1]}-M{c[2]}-s{c[3]}-{c[4][:3]}-{c[5]}-{c[6]}"
                                             for c in SMALL])
def test_small_parity(case, dtype):
    H, W, M, s, part, sim, pos = case
    heads = 3 if M % 2 else 2
    wl = synth.small(B=2, H=H, W=W, C=32 * heads, heads=heads, M=M, shift=s, partition=part,
                     sim=sim, pos=pos, dtype=dtype, hidden=64)
    x = synth.make_inputs(wl, seed=7)
    out = run_gpu(wl, gpu_inputs(x))
    compare(wl, f64(out), run_oracle(wl, x), what=str(case))


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_workload_full(idx):
    """Workloads 0-2 at full size, every output compared."""
    wl = synth.WORKLOADS[idx]
    x = synth.make_inputs(wl)
    out = run_gpu(wl, gpu_inputs(x))
    err, rel = compare(wl, f64(out), run_oracle(wl, x), what=wl.name)
    print(f"{wl.name}: max-abs {err:.3e} rel-fro {rel:.3e}")


@pytest.mark.parametrize("idx", [3, 4])
def test_workload_sampled(idx):
    """Workloads 3-4 at full size; the oracle computes windows sampled from
    every shift-mask class and those tokens are compared."""
    wl = synth.WORKLOADS[idx]
    x = synth.make_inputs(wl)
    out = run_gpu(wl, gpu_inputs(x))
    wins = sample_windows(wl, per_class=3, seed=idx)
    ref = run_oracle(wl, x, windows=wins)
    mask = window_token_mask(wl, wins)
    err, rel = compare(wl, f64(out), ref, mask=mask, what=wl.name)
    print(f"{wl.name}: {len(wins)} windows, max-abs {err:.3e} rel-fro {rel:.3e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tau_below_floor(dtype):
    """tau under 0.01 is clamped; at 0.01 the logits span +-100 and the
    static-shift softmax falls back to the running-max path."""
    wl = synth.small(B=2, H=32, W=32, C=64, heads=2, M=16, shift=8, dtype=dtype, hidden=64)
    x = synth.make_inputs(wl, seed=2)
    x["tau"] = torch.tensor([0.001, 0.05])
    out = run_gpu(wl, gpu_inputs(x))
    compare(wl, f64(out), run_oracle(wl, x), what="tau floor")


@pytest.mark.parametrize("pos", ["table", "rope2d"])
def test_large_window_small_tau(pos):
    """M = 24 with tau below 0.1: without rotation the raw k and 1/||k|| carry
    the precision; with rotation q and k are carried as hi + lo pairs."""
    wl = synth.small(B=1, H=48, W=48, C=64, heads=2, M=24, shift=12, sim="cosine", pos=pos,
                     dtype="bf16", hidden=64)
    x = synth.make_inputs(wl, seed=6)
    x["tau"] = torch.tensor([0.03, 0.5])
    out = run_gpu(wl, gpu_inputs(x))
    compare(wl, f64(out), run_oracle(wl, x), what=f"large window small tau {pos}")


@pytest.mark.parametrize("pos", ["none", "rope2d"])
def test_dot_large_norms(pos):
    """q, k scaled x8 (logits up to ~360): the Cauchy-Schwarz shift would
    underflow, so the running-max path runs; with rotation the rotated
    operands are also carried as hi + lo bf16 pairs."""
    wl = synth.small(B=1, H=64, W=64, C=64, heads=2, M=32, shift=16, sim="dot", pos=pos,
                     dtype="bf16")
    x = synth.make_inputs(wl, seed=4)
    x["q"] = (x["q"].float() * 8).to(torch.bfloat16)
    x["k"] = (x["k"].float() * 8).to(torch.bfloat16)
    out = run_gpu(wl, gpu_inputs(x))
    compare(wl, f64(out), run_oracle(wl, x), what="dot large norms")


def test_windows_layout_matches_grid():
    """attn(GRID) == reverse(attn(WINDOWS, partition(x))), bit for bit."""
    wl = synth.small(B=2, H=32, W=32, C=96, heads=3, M=16, shift=8, dtype="bf16", hidden=64)
    g = gpu_inputs(synth.make_inputs(wl, seed=5))
    table = gpu_table(wl, g)
    grid_out = run_gpu(wl, g, table=table)
    part = {n: binding.swin_window_partition(g[n], wl.M, wl.shift) for n in "qkv"}
    wout = binding.swin_window_attn_fwd(part["q"], part["k"], part["v"], heads=wl.heads, M=wl.M,
                                        shift=wl.shift, sim="cosine", pos="table", tau=g["tau"],
                                        table=table, layout="windows", grid=(wl.B, wl.H, wl.W))
    back = binding.swin_window_reverse(wout, wl.B, wl.H, wl.W, wl.M, wl.shift)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), grid_out.view(torch.int16))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_deterministic(dtype):
    """Two launches give bit-identical outputs (no atomics in the sums)."""
    wl = synth.small(B=2, H=48, W=48, C=96, heads=3, M=24, shift=12, dtype=dtype, hidden=64)
    g = gpu_inputs(synth.make_inputs(wl, seed=6))
    a, b = run_gpu(wl, g), run_gpu(wl, g)
    assert torch.equal(a, b)


def test_rope_frequency_table():
    wl = synth.small(B=2, H=32, W=32, C=64, heads=2, M=16, shift=8, sim="dot", pos="rope2d",
                     dtype="bf16")
    x = synth.make_inputs(wl, seed=8)
    fr = torch.rand(2, 2, 8, generator=torch.Generator().manual_seed(0)) * 1.5 + 0.01
    out = run_gpu(wl, gpu_inputs(x), rope_freqs=fr.to("cuda:0"))
    compare(wl, f64(out), run_oracle(wl, x, rope_freqs=f64(fr)), what="rope freqs")


def test_caller_table_and_single_window():
    """A caller-made bias table (trained-size values, not from the MLP) and a
    window covering the whole grid."""
    wl = synth.small(B=3, H=16, W=16, C=96, heads=3, M=16, shift=0, dtype="bf16")
    x = synth.make_inputs(wl, seed=9)
    tab = torch.randn(31 * 31, 3, generator=torch.Generator().manual_seed(1)) * 3
    out = run_gpu(wl, gpu_inputs(x), table=tab.to("cuda:0"))
    compare(wl, f64(out), run_oracle(wl, x, table=f64(tab)), what="caller table")


def test_empty_batch_writes_nothing():
    wl = synth.small(B=0, H=16, W=16, C=64, heads=2, M=8, shift=4, dtype="bf16")
    q = torch.empty((0, 16, 16, 64), dtype=torch.bfloat16, device="cuda:0")
    out = binding.swin_window_attn_fwd(q, q, q, heads=2, M=8, shift=4, sim="cosine", pos="none",
                                       tau=torch.ones(2, device="cuda:0"))
    torch.cuda.synchronize()
    assert out.shape == q.shape


# Windows of up to 8 x 8 without a table and with an even head count run as
# workgroups of two windows x a head pair: odd window counts (the last
# workgroup's second window inactive), two heads (one pair), padded rows
# (M = 6, 7), shifts, interleaving, dot and cosine.
HEAD_PAIRS = [
    # (B, H, W, M, shift, partition, sim, heads)
    (1, 24, 40, 8, 4, "cyclic", "dot", 2),           # 15 windows
    (1, 21, 35, 7, 3, "cyclic", "cosine", 4),        # 15 windows, 7 -> 8 slots per key row
    (3, 16, 24, 8, 0, "interleaved", "cosine", 6),   # 18 windows over 3 images
    (1, 18, 30, 6, 2, "cyclic", "dot", 4),           # 15 windows, 36 of 48 slots
    (1, 8, 8, 8, 0, "cyclic", "dot", 2),             # one window
]


@pytest.mark.parametrize("case", HEAD_PAIRS, ids=[f"B{c[0]}-{c[1]}x{c[2]}-M{c[3]}-s{c[4]}-{c[5][:3]}-{c[6]}-h{c[7]}"
                                                  for c in HEAD_PAIRS])
def test_head_pair_workgroups(case):
    B, H, W, M, s, part, sim, heads = case
    wl = synth.small(B=B, H=H, W=W, C=32 * heads, heads=heads, M=M, shift=s, partition=part, sim=sim, pos="none",
                     dtype="bf16", hidden=64)
    x = synth.make_inputs(wl, seed=11)
    g = gpu_inputs(x)
    kw = dict(heads=heads, M=M, shift=s, partition=part, sim=sim, pos="none", tau=g["tau"])
    desc = binding.make_desc(B=B, H=H, W=W, C=wl.C, heads=heads, M=M, shift=s, partition=part, sim=sim,
                             pos="none", dtype=g["q"].dtype)
    assert binding.swin_window_attn_kernel(desc) == "attn_small_kernel"
    out, lse = binding.swin_window_attn_fwd_lse(g["q"], g["k"], g["v"], **kw)
    plain = binding.swin_window_attn_fwd(g["q"], g["k"], g["v"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    ref, ref_lse = oracle.window_attn(f64(x["q"]), f64(x["k"]), f64(x["v"]), heads=heads, M=M, shift=s,
                                      partition=part, sim=sim, pos="none", tau=f64(x["tau"]), return_lse=True)
    compare(wl, f64(out), ref, what=str(case))
    # log-sum-exp: the bf16 bar of the exported statistic (logit error from
    # the rounded operands, 2^-8 of the logit scale's bound, plus fp32 sums)
    d = 32
    if sim == "cosine":
        scale = (1.0 / np.maximum(f64(x["tau"]), 0.01))[None, :, None]
    else:
        qn = np.linalg.norm(f64(x["q"]).reshape(B, H, W, heads, d), axis=-1)
        kn = np.linalg.norm(f64(x["k"]).reshape(B, H, W, heads, d), axis=-1)
        qw = oracle.partition(qn, M, s, part).transpose(0, 2, 1)
        kwin = oracle.partition(kn, M, s, part).transpose(0, 2, 1)
        scale = qw * kwin.max(axis=2, keepdims=True) / np.sqrt(d)
    err = np.abs(f64(lse) - ref_lse)
    assert np.all(err <= 2.0 ** -8 * scale + 2.0 ** -8 + 1e-5 * np.abs(ref_lse)), float(err.max())
    # pre-partitioned windows give the grid layout's result bit for bit
    parts = {n: binding.swin_window_partition(g[n], M, s, part) for n in "qkv"}
    wout = binding.swin_window_attn_fwd(parts["q"], parts["k"], parts["v"], layout="windows", grid=(B, H, W), **kw)
    back = binding.swin_window_reverse(wout, B, H, W, M, s, part)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), out.view(torch.int16))
