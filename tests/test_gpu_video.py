"""GPU parity of video (3D) window attention (swin_window_attn3d_fwd) and its
bias table (swin_cpb_table3d) against the fp64 oracle, through the C ABI, on
the same seeded inputs.

Bars: the attention takes the forward's (fp32: max-abs 1e-5; bf16: max-abs
2e-2 and relative Frobenius 1e-2, the output rounded once); the attention
tests hand both sides the same table, so it is checked on its own: a fp32
sum over the hidden units against fp64, within 1e-5 relative and 1e-4
absolute of the oracle, as the 2D table."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import BF16_TOL, F32_TOL, f64
from vision_transformer_windowed_partition_amd import binding, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # T, H, W, Mt, M, shift_t, shift, partition, sim, pos
    (4, 8, 8, 2, 4, 1, 2, "cyclic", "cosine", "table"),       # every axis shifted
    (8, 16, 16, 4, 8, 2, 4, "cyclic", "dot", "table"),
    (4, 16, 16, 4, 8, 0, 0, "interleaved", "cosine", "none"),
    (6, 12, 12, 3, 6, 1, 3, "cyclic", "cosine", "none"),      # 108-token windows
    (2, 8, 8, 1, 8, 0, 4, "cyclic", "cosine", "table"),       # one frame a window: the 2D attention per frame
    (8, 32, 32, 8, 16, 0, 8, "cyclic", "cosine", "table"),    # the pages' 16^2 x 8 windows (2048 tokens)
    (6, 16, 16, 3, 8, 1, 4, "cyclic", "cosine", "table"),     # 3 query frames on 4 wavefronts, every axis shifted
    (4, 32, 32, 2, 16, 1, 8, "cyclic", "dot", "none"),
    (4, 40, 40, 2, 20, 1, 10, "cyclic", "cosine", "table"),   # 20^2 x 2 windows: 8 wavefronts, 24-slot key rows
    (2, 22, 44, 2, 22, 0, 11, "cyclic", "dot", "table"),      # the largest matrix-core window
    (4, 24, 24, 2, 12, 1, 6, "cyclic", "cosine", "table"),    # 12-key rows padded to 16 slots
    (2, 34, 34, 1, 17, 0, 8, "cyclic", "cosine", "none"),     # odd rows in 24 slots, one frame a window
    (4, 10, 15, 2, 5, 1, 2, "cyclic", "dot", "table"),        # 5-key rows padded to 8 slots
    (2, 36, 36, 2, 18, 0, 0, "interleaved", "cosine", "table"),
]
# bf16 runs on the matrix cores (M <= 22), fp32 on the vector ALUs


def _compare(got, ref, dtype, what):
    err = float(np.abs(got - ref).max())
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    assert np.all(np.isfinite(got)), what
    if dtype == "f32":
        assert err <= F32_TOL, f"{what}: fp32 max-abs {err:.3e}"
    else:
        assert err <= BF16_TOL[0] and rel <= BF16_TOL[1], f"{what}: bf16 max-abs {err:.3e} rel-fro {rel:.3e}"


def _inputs(case, dtype, seed, B=1, heads=2):
    T, H, W, Mt, M, st, s, part, sim, pos = case
    gen = torch.Generator().manual_seed(seed)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, v = (torch.randn((B, T, H, W, 32 * heads), generator=gen).to(dt) for _ in range(3))
    tau = torch.exp(torch.rand(heads, generator=gen) * np.log(10.0) + np.log(0.1))
    table = 0.5 * torch.randn(((2 * Mt - 1) * (2 * M - 1) ** 2, heads), generator=gen) if pos == "table" else None
    return q, k, v, tau, table


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}-{c[1]}x{c[2]}-Mt{c[3]}-M{c[4]}-s{c[5]}.{c[6]}-{c[7][:3]}-{c[8]}-"
                                             f"{c[9]}" for c in CASES])
def test_video_parity(case, dtype):
    T, H, W, Mt, M, st, s, part, sim, pos = case
    q, k, v, tau, table = _inputs(case, dtype, seed=T * 100 + M)
    d = lambda t: None if t is None else t.to(DEV)
    out = binding.swin_window_attn3d_fwd(d(q), d(k), d(v), heads=2, Mt=Mt, M=M, shift_t=st, shift=s, partition=part,
                                         sim=sim, pos=pos, tau=d(tau), table=d(table))
    torch.cuda.synchronize()
    ref = oracle.window_attn3d(f64(q), f64(k), f64(v), heads=2, Mt=Mt, M=M, shift_t=st, shift=s, partition=part,
                               sim=sim, pos=pos, tau=f64(tau), table=None if table is None else f64(table))
    _compare(f64(out), ref, dtype, str(case))


@pytest.mark.parametrize("M", [8, 16, 20])
def test_video_small_tau(M):
    """COSINE with tau below 0.1 for one head: the matrix-core kernel keeps
    raw k with 1/||k|| in fp32 instead of rounding k / ||k|| / tau."""
    case = (4, 2 * M, 2 * M, 2, M, 1, M // 2, "cyclic", "cosine", "table")
    q, k, v, tau, table = _inputs(case, "bf16", seed=M)
    tau = torch.tensor([0.03, 0.5])
    d = lambda t: t.to(DEV)
    out = binding.swin_window_attn3d_fwd(d(q), d(k), d(v), heads=2, Mt=2, M=M, shift_t=1, shift=M // 2,
                                         sim="cosine", pos="table", tau=d(tau), table=d(table))
    torch.cuda.synchronize()
    ref = oracle.window_attn3d(f64(q), f64(k), f64(v), heads=2, Mt=2, M=M, shift_t=1, shift=M // 2, sim="cosine",
                               pos="table", tau=f64(tau), table=f64(table))
    _compare(f64(out), ref, "bf16", f"small tau M={M}")


def test_video_kernel_choice():
    d = lambda **kw: binding.make_desc(**{**dict(B=1, H=32, W=32, C=64, heads=2, M=16, shift=8, sim="cosine",
                                                  pos="table", dtype=torch.bfloat16), **kw})
    assert binding.swin_window_attn3d_kernel(d(), 8, 8) == "attn_video_mfma_kernel"
    assert binding.swin_window_attn3d_kernel(d(M=8, shift=4), 8, 4) == "attn_video_mfma_kernel"
    assert binding.swin_window_attn3d_kernel(d(dtype=torch.float32), 8, 8) == "attn_video_kernel"
    assert binding.swin_window_attn3d_kernel(d(M=4, shift=2), 8, 8) == "attn_video_mfma_kernel"
    assert binding.swin_window_attn3d_kernel(d(H=40, W=40, M=20, shift=10), 8, 8) == "attn_video_mfma_kernel"
    assert binding.swin_window_attn3d_kernel(d(H=46, W=46, M=23, shift=11), 2, 2) == "attn_video_kernel"


def test_video_one_frame_windows_match_2d():
    """Mt = 1: each frame is the 2D attention (the 2D entry point on B*T images)."""
    case = (3, 16, 16, 1, 8, 0, 4, "cyclic", "dot", "table")
    q, k, v, tau, table = _inputs(case, "f32", seed=5)
    d = lambda t: t.to(DEV)
    out3 = binding.swin_window_attn3d_fwd(d(q), d(k), d(v), heads=2, Mt=1, M=8, shift=4, sim="dot", pos="table",
                                          table=d(table))
    B, T, H, W, C = q.shape
    out2 = binding.swin_window_attn_fwd(d(q).reshape(B * T, H, W, C), d(k).reshape(B * T, H, W, C),
                                        d(v).reshape(B * T, H, W, C), heads=2, M=8, shift=4, sim="dot", pos="table",
                                        table=d(table))
    torch.cuda.synchronize()
    assert float((out3.reshape(B * T, H, W, C) - out2).abs().max()) <= 1e-5


@pytest.mark.parametrize("Mt,M,heads,hidden", [(8, 16, 3, 512), (2, 4, 2, 37), (1, 8, 5, 512), (3, 7, 16, 64)])
def test_cpb_table3d(Mt, M, heads, hidden):
    gen = torch.Generator().manual_seed(Mt * 100 + M)
    w1, b1 = torch.randn(hidden, 3, generator=gen), torch.randn(hidden, generator=gen)
    w2, b2 = 0.1 * torch.randn(heads, hidden, generator=gen), torch.randn(heads, generator=gen)
    got = binding.swin_cpb_table3d(Mt, M, w1.to(DEV), b1.to(DEV), w2.to(DEV), b2.to(DEV))
    got0 = binding.swin_cpb_table3d(Mt, M, w1.to(DEV), None, w2.to(DEV), None)
    torch.cuda.synchronize()
    want = oracle.cpb_table3d(Mt, M, f64(w1), f64(b1), f64(w2), f64(b2))
    np.testing.assert_allclose(f64(got), want, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(f64(got0), oracle.cpb_table3d(Mt, M, f64(w1), None, f64(w2), None), rtol=1e-5,
                               atol=1e-4)


@pytest.mark.parametrize("idx", range(len(synth.VIDEO_WORKLOADS)),
                         ids=[w.name for w in synth.VIDEO_WORKLOADS])
def test_video_workload_sampled(idx):
    """The video workloads at full size (the launch the bench times), the
    table from swin_cpb_table3d; the oracle computes sampled windows."""
    wl = synth.VIDEO_WORKLOADS[idx]
    x = synth.make_video_inputs(wl)
    g = {k: v.to(DEV) for k, v in x.items()}
    table = binding.swin_cpb_table3d(wl.Mt, wl.M, g["w1"], g["b1"], g["w2"], g["b2"])
    out = binding.swin_window_attn3d_fwd(g["q"], g["k"], g["v"], heads=wl.heads, Mt=wl.Mt, M=wl.M,
                                         shift_t=wl.shift_t, shift=wl.shift, partition=wl.partition, sim=wl.sim,
                                         pos=wl.pos, tau=g["tau"], table=table)
    torch.cuda.synchronize()
    nW = (wl.T // wl.Mt) * (wl.H // wl.M) * (wl.W // wl.M)
    wins = np.array([0, nW - 1, nW + 3, wl.B * nW - 1])                  # interior, last row/column, corner
    tab64 = oracle.cpb_table3d(wl.Mt, wl.M, f64(x["w1"]), f64(x["b1"]), f64(x["w2"]), f64(x["b2"]))
    ref = oracle.window_attn3d(f64(x["q"]), f64(x["k"]), f64(x["v"]), heads=wl.heads, Mt=wl.Mt, M=wl.M,
                               shift_t=wl.shift_t, shift=wl.shift, partition=wl.partition, sim=wl.sim, pos=wl.pos,
                               tau=f64(x["tau"]), table=tab64, windows=wins)
    mask = ref != 0
    got = f64(out)
    _compare(got[mask], ref[mask], wl.dtype, wl.name)
    assert mask.sum() == len(wins) * wl.N * wl.C


def _random_case(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.choice([2, 4, 5, 8, 8, 11, 16, 16, 19, 20]))
    Mt = int(rng.choice([1, 2, 3, 4]))
    nt, nr, nc = int(rng.integers(1, 3)), int(rng.integers(1, 3)), int(rng.integers(1, 3))
    part = "interleaved" if rng.random() < 0.3 else "cyclic"
    st = 0 if part == "interleaved" or nt == 1 else int(rng.integers(0, Mt))
    s = 0 if part == "interleaved" or nr * nc == 1 else int(rng.integers(0, M))
    sim = "cosine" if rng.random() < 0.6 else "dot"
    pos = "table" if rng.random() < 0.6 else "none"
    return (nt * Mt, nr * M, nc * M, Mt, M, st, s, part, sim, pos)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("seed", range(12))
def test_video_random(seed, dtype):
    """Seeded random video geometries (bf16 on the matrix cores, fp32 on the
    vector ALUs)."""
    case = _random_case(seed)
    T, H, W, Mt, M, st, s, part, sim, pos = case
    q, k, v, tau, table = _inputs(case, dtype, seed=500 + seed, B=2)
    d = lambda t: None if t is None else t.to(DEV)
    out = binding.swin_window_attn3d_fwd(d(q), d(k), d(v), heads=2, Mt=Mt, M=M, shift_t=st, shift=s, partition=part,
                                         sim=sim, pos=pos, tau=d(tau), table=d(table))
    torch.cuda.synchronize()
    ref = oracle.window_attn3d(f64(q), f64(k), f64(v), heads=2, Mt=Mt, M=M, shift_t=st, shift=s, partition=part,
                               sim=sim, pos=pos, tau=f64(tau), table=None if table is None else f64(table))
    _compare(f64(out), ref, dtype, f"seed {seed}: {case}")
