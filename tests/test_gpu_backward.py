"""GPU parity of the backward (swin_window_attn_bwd, swin_cpb_table_bwd)
against the fp64 oracle backward, through the C ABI, on the same seeded
inputs.

Bars, derived from the arithmetic: fp32 mode computes in fp32 from exact
inputs, so each gradient is within 1e-4 of the oracle relative to its
largest entry and in relative Frobenius norm.  bf16 mode starts from the
bf16 inputs (exact in the oracle) and from the forward's bf16 output (D_i =
dout_i . out_i, out rounded to 2^-9), and rounds dq, dk, dv to bf16 once:
relative Frobenius <= 1e-2 and max-abs <= 2e-2 of the largest entry.  dtau
and dtable (fp32 sums over windows) take the same bars plus what the given
forward output induces: D_i = dout_i . out_i enters every dl_ij = p_ij (dP_ij
- D_i), so an error dD_i in the bf16 out moves dtau_h by (1/tau_h^2) sum_i
dD_i E_p[cos]_i, at most sum_i |dD_i| / tau_h^2 (|cos| <= 1), and a table
entry by at most sum_i |dD_i| (sum_j p_ij = 1); dD_i is measured against the
oracle's fp64 forward.  These sums cancel (sum_j dl_ij = 0), so their error is
not bounded by a fraction of their own size.

Given the forward's log-sum-exp (swin_window_attn_bwd_lse), the weights are
rebuilt as p_ij = exp(logit_ij - lse_i): an error e_i of lse_i scales query
i's row by exp(-e_i), which moves its share of dtau by at most
|e_i| sum_j p_ij |dP_ij - D_i| / tau_h^2 <= |e_i| 2 ||dout_i|| max_j ||v_j|| /
tau_h^2 (dP_ij = dout_i . v_j, ||out_i|| <= max_j ||v_j||) and a table entry
by at most |e_i| 2 ||dout_i|| max_j ||v_j||; e_i is measured against the
oracle's log-sum-exp and these sums join the allowance.  dq, dk, dv keep
their bars (a row scaled by 1 + e_i is a relative error)."""
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


def _check(name, got, ref, dtype, extra=0.0):
    """extra: an absolute allowance per element (the forward-induced bound)."""
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    extra = np.broadcast_to(np.asarray(extra, dtype=np.float64), np.shape(ref))
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = float((np.abs(got - ref) - extra).max()) / scale
    rel = float(max(np.linalg.norm(got - ref) - np.linalg.norm(extra), 0.0) / max(np.linalg.norm(ref), 1e-30))
    tmax, trel = TOL[dtype]
    if float(np.abs(ref).max()) == 0.0:
        # e.g. one token per window: dl = dP - D vanishes exactly in the oracle;
        # in fp32 dP (a matrix-core sum) and D (dout . out) round differently
        assert float(np.abs(got).max()) <= 1e-5, f"{name}: expected zeros"
        return
    assert err <= tmax and rel <= trel, f"{name}: max-abs/scale {err:.3e} rel-fro {rel:.3e} > {TOL[dtype]}"


def _run(wl, x, g, dout, table=None, table64=None, lse_from=None):
    """lse_from: None (the backward's own statistics), "gpu" (the forward's
    exported log-sum-exp) or "oracle" (the oracle's, rounded to fp32)."""
    kw = dict(heads=wl.heads, M=wl.M, shift=wl.shift, partition=wl.partition, sim=wl.sim, pos=wl.pos,
              tau=f64(x["tau"]), table=table64, rope_base=wl.rope_base)
    out64, lse64 = oracle.window_attn(f64(x["q"]), f64(x["k"]), f64(x["v"]), return_lse=True, **kw)
    lse = None
    if lse_from == "gpu":
        out, lse = binding.swin_window_attn_fwd_lse(g["q"], g["k"], g["v"], heads=wl.heads, M=wl.M,
                                                    shift=wl.shift, partition=wl.partition, sim=wl.sim,
                                                    pos=wl.pos, tau=g["tau"], table=table, rope_base=wl.rope_base)
    else:
        out = run_gpu(wl, g, table=table)
        if lse_from == "oracle":
            lse = torch.from_numpy(lse64).to(DEV, torch.float32)
    got = binding.swin_window_attn_bwd(g["q"], g["k"], g["v"], out, dout.to(DEV), heads=wl.heads, M=wl.M,
                                       shift=wl.shift, partition=wl.partition, sim=wl.sim, pos=wl.pos,
                                       tau=g["tau"], table=table, rope_base=wl.rope_base, lse=lse)
    torch.cuda.synchronize()
    ref = oracle.window_attn_bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(dout), **kw)
    # forward-induced bound of the summed gradients (see the module text)
    B, H, W, C = out64.shape
    d = C // wl.heads
    dD = np.abs(((f64(out) - out64) * f64(dout)).reshape(B, H, W, wl.heads, d).sum(-1))   # per token, head
    sum_dD = dD.reshape(-1, wl.heads).sum(0)
    if lse is not None:
        e = np.abs(f64(lse) - lse64)                                                  # (windows, heads, N)
        gn = np.linalg.norm(f64(dout).reshape(B, H, W, wl.heads, d), axis=-1)
        gw = oracle.partition(gn, wl.M, wl.shift, wl.partition).transpose(0, 2, 1)  # (windows, heads, N)
        vmax = np.linalg.norm(f64(x["v"]).reshape(-1, wl.heads, d), axis=-1).max(0)
        sum_dD = sum_dD + (e * gw).sum(axis=(0, 2)) * 2.0 * vmax
    tau_eff = np.maximum(f64(x["tau"]), 0.01)
    ref["_dtau_extra"] = sum_dD / tau_eff ** 2
    ref["_dtable_extra"] = sum_dD[None, :]
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
        _check(f"{case} dtau", f64(got["dtau"]), ref["dtau"], dtype, ref["_dtau_extra"])
    if pos == "table":
        _check(f"{case} dtable", f64(got["dtable"]), ref["dtable"], dtype, ref["_dtable_extra"])


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
        _check(f"{case} dtau", f64(got["dtau"]), ref["dtau"], dtype, ref["_dtau_extra"])
    if pos == "table":
        _check(f"{case} dtable", f64(got["dtable"]), ref["dtable"], dtype, ref["_dtable_extra"])


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
