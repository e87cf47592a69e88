"""GPU parity of the backward (swin_window_attn_bwd, swin_cpb_table_bwd)
against the fp64 oracle backward, through the C ABI, on the same seeded
inputs.

The oracle is handed what the GPU backward is handed: the forward output
`out` (D_i = dout_i . out_i) and, where the GPU takes one, the log-sum-exp
(p_ij = exp(logit_ij - lse_i)); FLASHSWIN abstract: the backward rebuilds
the weights from the forward's statistics.  Both sides then compute the same
function of the same inputs, and the bars come from the backward's own
arithmetic alone: fp32 mode computes in fp32 from exact inputs, so each
gradient is within 1e-4 of the oracle relative to its largest entry and in
relative Frobenius norm; bf16 mode rounds P and dS to bf16 for the matrix
products and dq, dk, dv once at the end: max-abs <= 2e-2 of the largest
entry and relative Frobenius <= 1e-2.  The same bars hold for dtau and
dtable (fp32 sums over windows)."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import f64, gpu_inputs, run_gpu
from vision_transformer_windowed_partition_amd import binding, synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [
    # H, W, M, shift, partition, sim, pos
    (16, 16, 8, 4, "cyclic", "cosine", "table"),
    (32, 32, 16, 8, "cyclic", "cosine", "table"),
    (16, 24, 8, 0, "interleaved", "dot", "none"),
    (32, 32, 32, 16, "cyclic", "dot", "rope2d"),
    (24, 24, 24, 12, "cyclic", "cosine", "table"),
    (14, 14, 7, 3, "cyclic", "cosine", "rope2d"),
    (24, 24, 12, 5, "cyclic", "dot", "table"),
    (8, 8, 1, 0, "cyclic", "cosine", "table"),          # one token per window: p = 1, dl = 0
    (20, 20, 10, 0, "interleaved", "cosine", "none"),
]

TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-2)}      # (max-abs / max|ref|, relative Frobenius)


def _check(name, got, ref, dtype):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = float(np.abs(got - ref).max()) / scale
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    tmax, trel = TOL[dtype]
    if float(np.abs(ref).max()) == 0.0:
        # e.g. one token per window: dl = dP - D vanishes exactly in the oracle;
        # in fp32 dP (a matrix-core sum) and D (dout . out) round differently
        assert float(np.abs(got).max()) <= 1e-5, f"{name}: expected zeros"
        return
    assert err <= tmax and rel <= trel, f"{name}: max-abs/scale {err:.3e} rel-fro {rel:.3e} > {TOL[dtype]}"


def _run(wl, x, g, dout, table=None, table64=None, lse_from=None):
    """lse_from: None (the backward's own statistics), "gpu" (the forward's
    exported log-sum-exp) or "oracle" (the oracle's, rounded to fp32).  The
    oracle is given the same output and log-sum-exp as the GPU backward."""
    kw = dict(heads=wl.heads, M=wl.M, shift=wl.shift, partition=wl.partition, sim=wl.sim, pos=wl.pos,
              tau=f64(x["tau"]), table=table64, rope_base=wl.rope_base)
    lse = None
    if lse_from == "gpu":
        out, lse = binding.swin_window_attn_fwd_lse(g["q"], g["k"], g["v"], heads=wl.heads, M=wl.M,
                                                    shift=wl.shift, partition=wl.partition, sim=wl.sim,
                                                    pos=wl.pos, tau=g["tau"], table=table, rope_base=wl.rope_base)
    else:
        out = run_gpu(wl, g, table=table)
        if lse_from == "oracle":
            _, lse64 = oracle.window_attn(f64(x["q"]), f64(x["k"]), f64(x["v"]), return_lse=True, **kw)
            lse = torch.from_numpy(lse64).to(DEV, torch.float32)
    got = binding.swin_window_attn_bwd(g["q"], g["k"], g["v"], out, dout.to(DEV), heads=wl.heads, M=wl.M,
                                       shift=wl.shift, partition=wl.partition, sim=wl.sim, pos=wl.pos,
                                       tau=g["tau"], table=table, rope_base=wl.rope_base, lse=lse)
    torch.cuda.synchronize()
    ref = oracle.window_attn_bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(dout), out=f64(out),
                                 lse=None if lse is None else f64(lse), **kw)
    return got, ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}-M{c[2]}-s{c[3]}-{c[4][:3]}-{c[5]}-{c[6]}"
                                             for c in CASES])
def test_backward_parity(case, dtype):
    H, W, M, s, part, sim, pos = case
    heads = 2
    wl = synth.small(B=2, H=H, W=W, C=32 * heads, heads=heads, M=M, shift=s, partition=part, sim=sim, pos=pos,
                     dtype=dtype, hidden=64)
    x = synth.make_inputs(wl, seed=11)
    g = gpu_inputs(x)
    table = table64 = None
    if pos == "table":
        # a table with trained-size spread, so the bias gradient matters
        gen = torch.Generator().manual_seed(5)
        t = 0.5 * torch.randn(((2 * M - 1) ** 2, heads), generator=gen)
        table, table64 = t.to(DEV), f64(t)
    got, ref = _run(wl, x, g, synth.make_dout(wl), table, table64)
    for name in ("dq", "dk", "dv"):
        _check(f"{case} {name}", f64(got[name]), ref[name], dtype)
    if sim == "cosine":
        _check(f"{case} dtau", f64(got["dtau"]), ref["dtau"], dtype)
    if pos == "table":
        _check(f"{case} dtable", f64(got["dtable"]), ref["dtable"], dtype)


@pytest.mark.parametrize("lse_from", ["gpu", "oracle"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}-M{c[2]}-s{c[3]}-{c[4][:3]}-{c[5]}-{c[6]}"
                                             for c in CASES])
def test_backward_with_lse(case, dtype, lse_from):
    """swin_window_attn_bwd_lse: the forward's log-sum-exp (or the oracle's)
    replaces the backward's own pass over the keys; same bars."""
    H, W, M, s, part, sim, pos = case
    heads = 2
    wl = synth.small(B=2, H=H, W=W, C=32 * heads, heads=heads, M=M, shift=s, partition=part, sim=sim, pos=pos,
                     dtype=dtype, hidden=64)
    x = synth.make_inputs(wl, seed=12)
    g = gpu_inputs(x)
    table = table64 = None
    if pos == "table":
        gen = torch.Generator().manual_seed(6)
        t = 0.5 * torch.randn(((2 * M - 1) ** 2, heads), generator=gen)
        table, table64 = t.to(DEV), f64(t)
    got, ref = _run(wl, x, g, synth.make_dout(wl), table, table64, lse_from=lse_from)
    for name in ("dq", "dk", "dv"):
        _check(f"{case} {name}", f64(got[name]), ref[name], dtype)
    if sim == "cosine":
        _check(f"{case} dtau", f64(got["dtau"]), ref["dtau"], dtype)
    if pos == "table":
        _check(f"{case} dtable", f64(got["dtable"]), ref["dtable"], dtype)


@pytest.mark.parametrize("M,shift,tau", [(12, 6, (0.02, 0.5)), (24, 12, (0.3, 0.05)), (7, 3, (0.01, 0.004))])
def test_backward_cosine_rope(M, shift, tau):
    """Cosine attention with rotary positions on the matrix cores (the large
    backward): the cosine is taken of the rotated operands, the score
    products from hi + lo pairs; tau from the floor up.  Given the forward's
    log-sum-exp and not."""
    heads = 2
    wl = synth.small(B=1, H=2 * M, W=2 * M, C=32 * heads, heads=heads, M=M, shift=shift, sim="cosine",
                     pos="rope2d", dtype="bf16", hidden=64)
    x = synth.make_inputs(wl, seed=40 + M)
    x["tau"] = torch.tensor(tau)
    g = gpu_inputs(x)
    desc = binding.make_desc(B=wl.B, H=wl.H, W=wl.W, C=wl.C, heads=heads, M=M, shift=shift, sim="cosine",
                             pos="rope2d", dtype=torch.bfloat16)
    assert binding.swin_window_attn_bwd_kernel(desc) == "attn_bwd_large_kernel"
    for lse_from in (None, "gpu"):
        got, ref = _run(wl, x, g, synth.make_dout(wl), lse_from=lse_from)
        for name in ("dq", "dk", "dv", "dtau"):
            _check(f"M={M} tau={tau} lse={lse_from} {name}", f64(got[name]), ref[name], "bf16")


def test_backward_tau_at_floor():
    """tau below its floor: the clamp passes no gradient to tau."""
    wl = synth.small(B=1, H=16, W=16, C=64, heads=2, M=8, shift=4, sim="cosine", pos="none", dtype="f32")
    x = synth.make_inputs(wl, seed=3)
    x["tau"] = torch.tensor([0.005, 0.5])
    g = gpu_inputs(x)
    got, ref = _run(wl, x, g, synth.make_dout(wl))
    assert float(got["dtau"][0]) == 0.0 and ref["dtau"][0] == 0.0
    _check("dtau", f64(got["dtau"]), ref["dtau"], "f32")
    _check("dq", f64(got["dq"]), ref["dq"], "f32")


def test_backward_empty_batch():
    wl = synth.small(B=0, H=16, W=16, C=64, heads=2, M=8, shift=4, sim="cosine", pos="table", dtype="bf16")
    z = torch.zeros((0, 16, 16, 64), dtype=torch.bfloat16, device=DEV)
    tab = torch.zeros((225, 2), device=DEV)
    got = binding.swin_window_attn_bwd(z, z, z, z, z, heads=2, M=8, shift=4, sim="cosine", pos="table",
                                       tau=torch.ones(2, device=DEV), table=tab)
    torch.cuda.synchronize()
    assert got["dq"].numel() == 0
    assert float(got["dtable"].abs().max()) == 0.0 and float(got["dtau"].abs().max()) == 0.0


@pytest.mark.parametrize("M,norm_M,mode,heads,hidden", [(8, None, 0, 3, 512), (16, None, 3, 3, 512),
                                                        (24, 12, 1, 16, 512), (5, 9, 2, 2, 37),
                                                        (12, None, 3, 20, 300)])
def test_cpb_table_backward(M, norm_M, mode, heads, hidden):
    gen = torch.Generator().manual_seed(M)
    w1, b1 = torch.randn(hidden, 2, generator=gen), torch.randn(hidden, generator=gen)
    w2, b2 = 0.1 * torch.randn(heads, hidden, generator=gen), torch.randn(heads, generator=gen)
    dt = torch.randn(((2 * M - 1) ** 2, heads), generator=gen)
    d = lambda t: t.to(DEV)
    table = binding.swin_cpb_table(M, d(w1), d(b1), d(w2), d(b2), cpb_mode=mode, norm_M=norm_M)
    got = binding.swin_cpb_table_bwd(M, d(w1), d(b1), d(w2), table, d(dt), cpb_mode=mode, norm_M=norm_M)
    torch.cuda.synchronize()
    ref = oracle.cpb_table_bwd(M, f64(w1), f64(b1), f64(w2), f64(b2), f64(dt), mode=mode, norm_M=norm_M)
    for name, gv, rv in zip(("dw1", "db1", "dw2", "db2"), got, ref):
        _check(name, f64(gv), rv, "f32")


LSE_CASES = [
    # H, W, M, shift, partition, sim, pos
    (48, 32, 16, 0, "cyclic", "dot", "table"),         # diagonal bias sums, no shift regions
    (26, 39, 13, 6, "cyclic", "cosine", "none"),       # padded slots (16-slot rows)
    (27, 18, 9, 4, "cyclic", "dot", "table"),
    (22, 22, 11, 0, "interleaved", "cosine", "table"),
    (30, 45, 15, 7, "cyclic", "cosine", "table"),
    (24, 24, 12, 6, "cyclic", "dot", "none"),
    (32, 48, 16, 8, "cyclic", "dot", "table"),         # whole-group exclusions, half-range chunk loops
    (48, 32, 16, 4, "cyclic", "cosine", "table"),      # column split inside a group: every pair masked
    (32, 48, 16, 8, "cyclic", "cosine", "none"),       # half-range loops without a table (per-pair masks)
]


@pytest.mark.parametrize("case", LSE_CASES, ids=[f"{c[0]}x{c[1]}-M{c[2]}-s{c[3]}-{c[4][:3]}-{c[5]}-{c[6]}"
                                                 for c in LSE_CASES])
def test_backward_small_given_lse(case):
    """The small-window backward given the forward's log-sum-exp on window
    sizes 9 to 16 (padded key rows, shift regions, interleaved windows,
    dot and cosine, with and without the table), at the bf16 bars."""
    H, W, M, s, part, sim, pos = case
    heads = 2
    wl = synth.small(B=2, H=H, W=W, C=32 * heads, heads=heads, M=M, shift=s, partition=part, sim=sim, pos=pos,
                     dtype="bf16", hidden=64)
    desc = binding.make_desc(B=wl.B, H=H, W=W, C=wl.C, heads=heads, M=M, shift=s, partition=part, sim=sim, pos=pos,
                             dtype=torch.bfloat16)
    assert binding.swin_window_attn_bwd_kernel(desc) == "attn_bwd_small_kernel"
    x = synth.make_inputs(wl, seed=60 + M)
    g = gpu_inputs(x)
    table = table64 = None
    if pos == "table":
        gen = torch.Generator().manual_seed(7 + M)
        t = 0.5 * torch.randn(((2 * M - 1) ** 2, heads), generator=gen)
        table, table64 = t.to(DEV), f64(t)
    got, ref = _run(wl, x, g, synth.make_dout(wl), table, table64, lse_from="gpu")
    for name in ("dq", "dk", "dv"):
        _check(f"{case} {name}", f64(got[name]), ref[name], "bf16")
    if sim == "cosine":
        _check(f"{case} dtau", f64(got["dtau"]), ref["dtau"], "bf16")
    if pos == "table":
        _check(f"{case} dtable", f64(got["dtable"]), ref["dtable"], "bf16")


LARGE_REGION_CASES = [
    # H, W, M, shift, sim, pos: 2 x 1 or 1 x 2 windows, so one window has one
    # split (rows or columns) and the other both
    (64, 32, 32, 16, "dot", "rope2d"),      # column groups without a table; corner: row halves + groups
    (32, 64, 32, 16, "dot", "rope2d"),      # row halves alone; corner
    (24, 48, 24, 12, "cosine", "rope2d"),   # row halves with hi + lo scores; corner: per-pair masks
    (24, 48, 24, 12, "cosine", "table"),    # row halves alone; corner: halves + per-pair masks
    (48, 24, 24, 12, "cosine", "table"),    # column split inside a group: per-pair masks
    (48, 48, 24, 8, "dot", "table"),        # 2 x 2: plain, column groups, row halves, both
]


@pytest.mark.parametrize("lse_from", [None, "gpu"])
@pytest.mark.parametrize("case", LARGE_REGION_CASES,
                         ids=[f"{c[0]}x{c[1]}-M{c[2]}-s{c[3]}-{c[4]}-{c[5]}" for c in LARGE_REGION_CASES])
def test_backward_large_shift_regions(case, lse_from):
    """The large-window backward on shifted windows of the last row and
    column: exclusions by whole 8-slot groups, chunk loops restricted to the
    query's (or key's) row region, and per-pair masks where the column split
    falls inside a group; bf16 bars."""
    H, W, M, s, sim, pos = case
    heads = 2
    wl = synth.small(B=1, H=H, W=W, C=32 * heads, heads=heads, M=M, shift=s, sim=sim, pos=pos, dtype="bf16",
                     hidden=64)
    desc = binding.make_desc(B=1, H=H, W=W, C=wl.C, heads=heads, M=M, shift=s, sim=sim, pos=pos,
                             dtype=torch.bfloat16)
    assert binding.swin_window_attn_bwd_kernel(desc) == "attn_bwd_large_kernel"
    x = synth.make_inputs(wl, seed=90 + M + s)
    g = gpu_inputs(x)
    table = table64 = None
    if pos == "table":
        gen = torch.Generator().manual_seed(9 + M)
        t = 0.5 * torch.randn(((2 * M - 1) ** 2, heads), generator=gen)
        table, table64 = t.to(DEV), f64(t)
    got, ref = _run(wl, x, g, synth.make_dout(wl), table, table64, lse_from=lse_from)
    for name in ("dq", "dk", "dv"):
        _check(f"{case} {name}", f64(got[name]), ref[name], "bf16")
    if sim == "cosine":
        _check(f"{case} dtau", f64(got["dtau"]), ref["dtau"], "bf16")
    if pos == "table":
        _check(f"{case} dtable", f64(got["dtable"]), ref["dtable"], "bf16")


@pytest.mark.parametrize("M,shift,sim,pos,dtype,lse_from", [(48, 24, "cosine", "table", "bf16", "gpu"),
                                                            (40, 0, "dot", "rope2d", "f32", None),
                                                            (64, 32, "cosine", "none", "bf16", None)])
def test_backward_windows_past_32(M, shift, sim, pos, dtype, lse_from):
    """Windows above 32 x 32 (the forward's key-blocked range) on the
    vector-ALU backward, one window a head, at the bars of the dtype."""
    heads = 2
    wl = synth.small(B=1, H=M, W=M, C=32 * heads, heads=heads, M=M, shift=shift, sim=sim, pos=pos, dtype=dtype,
                     hidden=64)
    desc = binding.make_desc(B=1, H=M, W=M, C=wl.C, heads=heads, M=M, shift=shift, sim=sim, pos=pos,
                             dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    assert binding.swin_window_attn_bwd_kernel(desc) == "attn_bwd_kernel"
    x = synth.make_inputs(wl, seed=M)
    g = gpu_inputs(x)
    table = table64 = None
    if pos == "table":
        gen = torch.Generator().manual_seed(M)
        t = 0.5 * torch.randn(((2 * M - 1) ** 2, heads), generator=gen)
        table, table64 = t.to(DEV), f64(t)
    got, ref = _run(wl, x, g, synth.make_dout(wl), table, table64, lse_from=lse_from)
    for name in ("dq", "dk", "dv"):
        _check(f"M={M} {name}", f64(got[name]), ref[name], dtype)
    if sim == "cosine":
        _check(f"M={M} dtau", f64(got["dtau"]), ref["dtau"], dtype)
    if pos == "table":
        _check(f"M={M} dtable", f64(got["dtable"]), ref["dtable"], dtype)
