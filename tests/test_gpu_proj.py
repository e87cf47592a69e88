"""GPU parity of the steps either side of the attention: the branch's linear
layers and residual post-norm (swin_qkv_proj, swin_proj_post_norm) and Iwin's
convolution branch (swin_dwconv_add), against the fp64 oracle, through the C
ABI, on the same seeded inputs.

Bars, derived from the arithmetic.  bf16 mode: the products of bf16 inputs
are exact in fp32 and summed in fp32 over at most 512 terms (relative error
far below 2^-9), and each output is rounded to bf16 once (half an ulp,
2^-9 relative), so every element must satisfy |got - ref| <= 2^-8 |ref| +
1e-3 (one bf16 ulp plus a floor for values near zero, where the fp32 sum's
own error can move the rounding); the convolution adds nine fp32 products to
the given bf16 output and rounds once, the same bar.  fp32 mode: fp32
throughout, |got - ref| <= 1e-5 |ref| + 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import f64
from vision_transformer_windowed_partition_amd import binding, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"bf16": (2.0 ** -8, 1e-3), "f32": (1e-5, 1e-4)}      # (relative, absolute) per element


def _check(name, got, ref, dtype):
    got = np.asarray(got, dtype=np.float64)
    rel, absl = TOL[dtype]
    err = np.abs(got - ref)
    bound = rel * np.abs(ref) + absl
    worst = np.unravel_index(np.argmax(err - bound), err.shape) if err.size else None
    assert np.all(np.isfinite(got)), name
    assert np.all(err <= bound), f"{name}: err {err[worst]:.3e} at {worst} > bound {bound[worst]:.3e}"


def _params(C, T, dtype, seed=2000):
    wl = synth.small("proj", B=1, H=1, W=max(T, 1), C=C, heads=C // 32, dtype=dtype)
    p = synth.make_branch_params(wl, seed=seed, T=T)
    return p, {k: v.to(DEV) for k, v in p.items()}


SHAPES = [
    # C, T: the workloads' channel counts; T ragged against the 64- and
    # 32-token blocks, a single token, and several blocks
    (96, 1000), (192, 517), (512, 333), (32, 1), (64, 64), (128, 4097), (256, 95), (480, 77),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("C,T", SHAPES)
def test_qkv_proj(C, T, dtype):
    p, g = _params(C, T, dtype)
    q, k, v = binding.swin_qkv_proj(g["x"], g["w_qkv"], g["b_qkv"])
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_proj(f64(p["x"]), f64(p["w_qkv"]), f64(p["b_qkv"]))
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        _check(f"{name} C={C} T={T}", f64(got), ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("C,T", SHAPES)
def test_proj_post_norm(C, T, dtype):
    p, g = _params(C, T, dtype)
    y = binding.swin_proj_post_norm(g["o"], g["w_proj"], g["b_proj"], g["x"], g["gamma"], g["beta"], eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.proj_post_norm(f64(p["o"]), f64(p["w_proj"]), f64(p["b_proj"]), f64(p["x"]), f64(p["gamma"]),
                                f64(p["beta"]), 1e-5)
    _check(f"y C={C} T={T}", f64(y), ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_no_bias_and_in_place(dtype):
    """b = NULL means no bias; y may be resid itself (the main path updated in
    place, as the block pseudocode writes it)."""
    C, T = 96, 300
    p, g = _params(C, T, dtype, seed=2001)
    q, k, v = binding.swin_qkv_proj(g["x"], g["w_qkv"], None)
    resid = g["x"].clone()
    y = binding.swin_proj_post_norm(g["o"], g["w_proj"], None, resid, g["gamma"], g["beta"], eps=1e-5, out=resid)
    torch.cuda.synchronize()
    assert y.data_ptr() == resid.data_ptr()
    rq, rk, rv = oracle.qkv_proj(f64(p["x"]), f64(p["w_qkv"]), None)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        _check(name, f64(got), ref, dtype)
    ref = oracle.proj_post_norm(f64(p["o"]), f64(p["w_proj"]), None, f64(p["x"]), f64(p["gamma"]),
                                f64(p["beta"]), 1e-5)
    _check("y in place", f64(y), ref, dtype)


def test_constant_tokens_and_eps():
    """A token whose projection is constant (o = 0, no bias) normalises to
    beta: y = resid + beta; eps = 0 is accepted."""
    C, T = 128, 70
    p, g = _params(C, T, "bf16", seed=2002)
    o = torch.zeros_like(g["o"])
    y = binding.swin_proj_post_norm(o, g["w_proj"], None, g["x"], g["gamma"], g["beta"], eps=1e-5)
    torch.cuda.synchronize()
    ref = f64(p["x"]) + f64(p["beta"])[None, :]
    _check("constant", f64(y), ref, "bf16")
    y0 = binding.swin_proj_post_norm(g["o"], g["w_proj"], g["b_proj"], g["x"], g["gamma"], g["beta"], eps=0.0)
    torch.cuda.synchronize()
    ref0 = oracle.proj_post_norm(f64(p["o"]), f64(p["w_proj"]), f64(p["b_proj"]), f64(p["x"]), f64(p["gamma"]),
                                 f64(p["beta"]), 0.0)
    _check("eps 0", f64(y0), ref0, "bf16")


def test_empty():
    C = 96
    x = torch.empty((0, C), dtype=torch.bfloat16, device=DEV)
    w = torch.empty((3 * C, C), dtype=torch.bfloat16, device=DEV)
    q, k, v = binding.swin_qkv_proj(x, w, None)
    assert q.shape == (0, C)
    wp = torch.empty((C, C), dtype=torch.bfloat16, device=DEV)
    ones = torch.ones(C, device=DEV)
    y = binding.swin_proj_post_norm(x, wp, None, x.clone(), ones, ones)
    assert y.shape == (0, C)


@pytest.mark.parametrize("w", [1, 2, 4])
def test_full_size_sampled(w):
    """The workload's full token count (the launch the bench times), checked
    on a seeded sample of tokens that the oracle computes one by one."""
    wl = synth.WORKLOADS[w]
    p = synth.make_branch_params(wl)
    g = {k: v.to(DEV) for k, v in p.items()}
    q, k, v = binding.swin_qkv_proj(g["x"], g["w_qkv"], g["b_qkv"])
    y = binding.swin_proj_post_norm(g["o"], g["w_proj"], g["b_proj"], g["x"], g["gamma"], g["beta"], eps=1e-5)
    torch.cuda.synchronize()
    T = p["x"].shape[0]
    rows = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(w).integers(0, T, 256)]))
    rq, rk, rv = oracle.qkv_proj(f64(p["x"][rows]), f64(p["w_qkv"]), f64(p["b_qkv"]))
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        _check(f"{wl.name} {name}", f64(got[torch.from_numpy(rows).to(DEV)]), ref, wl.dtype)
    ry = oracle.proj_post_norm(f64(p["o"][rows]), f64(p["w_proj"]), f64(p["b_proj"]), f64(p["x"][rows]),
                               f64(p["gamma"]), f64(p["beta"]), 1e-5)
    _check(f"{wl.name} y", f64(y[torch.from_numpy(rows).to(DEV)]), ry, wl.dtype)


DW_SHAPES = [
    # B, H, W, C: tiles of 8 x 8 with ragged edges, one and two channel chunks
    (2, 13, 21, 96), (1, 8, 8, 192), (1, 17, 9, 512), (3, 5, 7, 32), (1, 64, 64, 40),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,H,W,C", DW_SHAPES)
def test_dwconv_add(B, H, W, C, dtype):
    """Iwin's convolution branch: out += depthwise 3x3 conv of v (zero padding)."""
    if dtype == "bf16" and C % 8:
        pytest.skip("bf16 needs C a multiple of 8")
    gen = torch.Generator().manual_seed(B * 1000 + H * 10 + C)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    v = torch.randn((B, H, W, C), generator=gen).to(dt)
    out = torch.randn((B, H, W, C), generator=gen).to(dt)
    w = torch.randn((C, 3, 3), generator=gen) / 3.0
    b = 0.1 * torch.randn(C, generator=gen)
    o = out.to(DEV)
    res = binding.swin_dwconv_add(v.to(DEV), w.to(DEV), b.to(DEV), o)
    torch.cuda.synchronize()
    assert res.data_ptr() == o.data_ptr()
    ref = oracle.dwconv_add(f64(v), f64(w), f64(b), f64(out))
    _check(f"dwconv {B}x{H}x{W}x{C}", f64(o), ref, dtype)
    o2 = out.to(DEV)
    binding.swin_dwconv_add(v.to(DEV), w.to(DEV), None, o2)
    torch.cuda.synchronize()
    _check("dwconv no bias", f64(o2), oracle.dwconv_add(f64(v), f64(w), None, f64(out)), dtype)


def test_dwconv_full_size_sampled():
    """The interleaved workload's full grid (64 x 64 x 64 x 192, bf16), checked
    on a sample of whole images against the oracle."""
    wl = synth.WORKLOADS[2]
    gen = torch.Generator().manual_seed(77)
    v = torch.randn((wl.B, wl.H, wl.W, wl.C), generator=gen).to(torch.bfloat16)
    out = torch.randn((wl.B, wl.H, wl.W, wl.C), generator=gen).to(torch.bfloat16)
    w = torch.randn((wl.C, 3, 3), generator=gen) / 3.0
    b = 0.1 * torch.randn(wl.C, generator=gen)
    o = out.to(DEV)
    binding.swin_dwconv_add(v.to(DEV), w.to(DEV), b.to(DEV), o)
    torch.cuda.synchronize()
    imgs = [0, 17, wl.B - 1]
    ref = oracle.dwconv_add(f64(v[imgs]), f64(w), f64(b), f64(out[imgs]))
    _check("dwconv full size", f64(o[imgs]), ref, "bf16")
