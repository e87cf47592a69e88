"""fp64 CPU oracle for windowed multi-head self-attention (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package never imports the GPU library: the two share no code.

Contents
  * ``oracle.c`` (compiled with gcc into ``liboracle.so``): the plain per-window
    definition -- partition / reverse maps, log-spaced offsets, the CPB table,
    the attention itself (with the log-sum-exp a backward
    reuses) and its backward, the attention branch's linear
    layers and residual post-norm, Iwin's depthwise convolution branch and
    LinMapper's in-window linear mapping, and attention over video (3D)
    windows with their three-offset bias table, all in fp64.
  * ``bruteforce.py``: full-grid attention over every token pair with a mask, for
    tiny grids; it shares neither the partition nor the table indexing with
    ``oracle.c`` and serves as that file's independent check.

The pages followed are cited in each source file.  Every function here takes
plain numpy arrays; mode names are strings.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

PART = {"cyclic": 0, "interleaved": 1}
SIM = {"cosine": 0, "dot": 1}
POS = {"none": 0, "table": 1, "rope2d": 2}

_lib = None


def build(force: bool = False, src: str = _SRC, out: str = _SO, defines=()) -> str:
    """Compile ``oracle.c`` with gcc (OpenMP, IEEE arithmetic, no fast-math)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", *[f"-D{d}" for d in defines],
               src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _declare(lib):
    i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    vp = ctypes.c_void_p
    lib.oracle_log_offset.restype = dbl
    lib.oracle_log_offset.argtypes = [dbl]
    lib.oracle_cpb_table.restype = i32
    lib.oracle_cpb_table.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    lib.oracle_cpb_table_mode.restype = i32
    lib.oracle_cpb_table_mode.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, i32, vp]
    lib.oracle_code_offset.restype = ctypes.c_double
    lib.oracle_code_offset.argtypes = [ctypes.c_double, i32]
    for fn in (lib.oracle_partition, lib.oracle_reverse):
        fn.restype = i32
        fn.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32]
    lib.oracle_window_attn.restype = i32
    lib.oracle_window_attn.argtypes = [i32] * 10 + [dbl, dbl] + [vp] * 7 + [i64, vp, vp, vp]
    lib.oracle_window_attn_bwd.restype = i32
    lib.oracle_window_attn_bwd.argtypes = [i32] * 10 + [dbl, dbl] + [vp] * 12
    lib.oracle_window_attn_bwd_given.restype = i32
    lib.oracle_window_attn_bwd_given.argtypes = [i32] * 10 + [dbl, dbl] + [vp] * 14
    lib.oracle_cpb_table_bwd.restype = i32
    lib.oracle_cpb_table_bwd.argtypes = [i32] * 4 + [vp] * 4 + [i32] + [vp] * 5
    lib.oracle_window_cosines.restype = i32
    lib.oracle_window_cosines.argtypes = [i32] * 9 + [dbl, vp, vp, vp, i64, i32, vp]
    lib.oracle_linear.restype = i32
    lib.oracle_linear.argtypes = [vp] * 4 + [i64, i32, i32]
    lib.oracle_post_norm.restype = i32
    lib.oracle_post_norm.argtypes = [vp] * 4 + [dbl, vp, i64, i32]
    lib.oracle_dwconv_add.restype = i32
    lib.oracle_dwconv_add.argtypes = [vp] * 4 + [i32] * 4
    lib.oracle_window_linear.restype = i32
    lib.oracle_window_linear.argtypes = [i32] * 8 + [vp] * 4
    lib.oracle_cpb_table3d.restype = i32
    lib.oracle_cpb_table3d.argtypes = [i32] * 4 + [vp] * 5
    lib.oracle_window_attn3d.restype = i32
    lib.oracle_window_attn3d.argtypes = [i32] * 13 + [dbl] + [vp] * 5 + [vp, i64, vp]
    lib.oracle_table_resize.restype = i32
    lib.oracle_table_resize.argtypes = [i32] * 3 + [vp] * 2
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_max_threads.restype = i32
    lib.oracle_max_threads.argtypes = []
    return lib


def load(path: str | None = None):
    """Load (building first if needed) the oracle library.  A path other than the
    default loads a separately built variant and is returned, not cached."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        build()
        _lib = _declare(ctypes.CDLL(_SO))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def set_threads(n: int, lib=None) -> None:
    (lib or load()).oracle_set_threads(int(n))


def max_threads(lib=None) -> int:
    return int((lib or load()).oracle_max_threads())


def log_offset(x: float, lib=None) -> float:
    """sign(x) * log(1 + |x|)  (SwinV2 eq. 4)."""
    return float((lib or load()).oracle_log_offset(float(x)))


CPB_CODE_NORM, CPB_SIGMOID16 = 1, 2       # flags; 3 = the released code's form


def code_offset(x: float, norm_M: int, lib=None) -> float:
    """Released-code transform: u = 8 x / (norm_M - 1), sign(u) log2(1+|u|) / log2(8)."""
    return float((lib or load()).oracle_code_offset(float(x), int(norm_M)))


def cpb_table(M: int, w1, b1, w2, b2, lib=None, mode: int = 0, norm_M: int | None = None) -> np.ndarray:
    """(2M-1)^2 x heads bias table of the meta network G (SwinV2 eq. 3-4).
    mode 0 is the paper's form; bit 0 the released code's coordinate
    transform (offsets normalised by norm_M - 1, default M - 1), bit 1 its
    16 * sigmoid output bound."""
    w1, w2 = _f64(w1), _f64(w2)
    b1, b2 = _f64(b1), _f64(b2)
    hidden, heads = w1.shape[0], w2.shape[0]
    assert w1.shape == (hidden, 2) and w2.shape == (heads, hidden)
    out = np.empty(((2 * M - 1) ** 2, heads), dtype=np.float64)
    L = lib or load()
    if mode == 0 and norm_M is None:
        rc = L.oracle_cpb_table(M, heads, hidden, _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(out))
    else:
        rc = L.oracle_cpb_table_mode(M, M if norm_M is None else norm_M, heads, hidden, _ptr(w1), _ptr(b1),
                                     _ptr(w2), _ptr(b2), int(mode), _ptr(out))
    if rc:
        raise ValueError(f"oracle_cpb_table: bad argument (rc={rc})")
    return out


def table_resize(table, Ms: int, Md: int, lib=None) -> np.ndarray:
    """A Swin V1 (2Ms-1)^2 x heads bias table resampled bi-cubically to
    (2Md-1)^2 x heads (SwinV2 card, Problem and tab. 1)."""
    t = _f64(table)
    heads = t.shape[1]
    assert t.shape == ((2 * Ms - 1) ** 2, heads)
    out = np.empty(((2 * Md - 1) ** 2, heads), dtype=np.float64)
    rc = (lib or load()).oracle_table_resize(Ms, Md, heads, _ptr(t), _ptr(out))
    if rc:
        raise ValueError(f"oracle_table_resize: bad argument (rc={rc})")
    return out


def partition(x: np.ndarray, M: int, shift: int, part: str, lib=None) -> np.ndarray:
    """Byte-exact window partition of a (B, H, W, C) array of any dtype."""
    x = np.ascontiguousarray(x)
    B, H, W, C = x.shape
    out = np.empty((B * (H // M) * (W // M), M * M, C), dtype=x.dtype)
    rc = (lib or load()).oracle_partition(_ptr(x), _ptr(out), B, H, W, C, M, shift,
                                          PART[part], x.dtype.itemsize)
    if rc:
        raise ValueError("oracle_partition: bad argument")
    return out


def reverse(xw: np.ndarray, B: int, H: int, W: int, M: int, shift: int, part: str,
            lib=None) -> np.ndarray:
    """Byte-exact inverse of :func:`partition`."""
    xw = np.ascontiguousarray(xw)
    C = xw.shape[-1]
    out = np.empty((B, H, W, C), dtype=xw.dtype)
    rc = (lib or load()).oracle_reverse(_ptr(xw), _ptr(out), B, H, W, C, M, shift,
                                        PART[part], xw.dtype.itemsize)
    if rc:
        raise ValueError("oracle_reverse: bad argument")
    return out


def window_attn(q, k, v, *, heads: int, M: int, shift: int = 0, partition: str = "cyclic",
                sim: str = "cosine", pos: str = "none", tau=None, table=None,
                rope_freqs=None, rope_base: float = 10000.0, tau_min: float = 0.01,
                windows=None, return_weights: bool = False, out=None, return_lse: bool = False, lib=None):
    """Windowed attention forward in fp64.

    q, k, v: (B, H, W, C) arrays (converted exactly to fp64).  tau: (heads,);
    table: ((2M-1)^2, heads); rope_freqs: (heads, 2, d/4) or None for the
    base-``rope_base`` schedule.  ``windows``: optional global window ids to
    compute (the rest of ``out`` stays as given, zeros by default).
    Returns ``out`` (B, H, W, C) fp64, followed by the weights
    (n_windows, heads, N, N) when ``return_weights`` and the per-query
    natural-log log-sum-exp of the logits (n_windows, heads, N) when
    ``return_lse``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, W, C = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    tau, table, rope_freqs = _f64(tau), _f64(table), _f64(rope_freqs)
    if out is None:
        out = np.zeros((B, H, W, C), dtype=np.float64)
    win = None if windows is None else np.ascontiguousarray(windows, dtype=np.int64)
    nwin = (B * (H // M) * (W // M)) if win is None else len(win)
    N = M * M
    wts = np.empty((nwin, heads, N, N), dtype=np.float64) if return_weights else None
    lse = np.empty((nwin, heads, N), dtype=np.float64) if return_lse else None
    rc = (lib or load()).oracle_window_attn(
        B, H, W, C, heads, M, shift, PART[partition], SIM[sim], POS[pos],
        float(tau_min), float(rope_base), _ptr(q), _ptr(k), _ptr(v), _ptr(tau),
        _ptr(table), _ptr(rope_freqs), _ptr(win), 0 if win is None else len(win),
        _ptr(out), _ptr(wts), _ptr(lse))
    if rc:
        raise ValueError(f"oracle_window_attn: bad argument (rc={rc})")
    res = (out,) + ((wts,) if return_weights else ()) + ((lse,) if return_lse else ())
    return res if len(res) > 1 else out


def window_attn_bwd(q, k, v, dout, *, heads: int, M: int, shift: int = 0, partition: str = "cyclic",
                    sim: str = "cosine", pos: str = "none", tau=None, table=None,
                    rope_freqs=None, rope_base: float = 10000.0, tau_min: float = 0.01,
                    out=None, lse=None, lib=None):
    """Gradients of sum(dout * window_attn(...)) in fp64: a dict with dq, dk,
    dv (B, H, W, C), dtau (heads,) for COSINE and dtable ((2M-1)^2, heads) for
    TABLE.  out (B, H, W, C) and lse (windows, heads, N) are optional forward
    statistics as a caller holds them: D_i = dout_i . out_i and
    p_ij = exp(logit_ij - lse_i) then come from them instead of the recomputed
    softmax (the same values for the exact forward)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, W, C = q.shape
    assert k.shape == q.shape and v.shape == q.shape and dout.shape == q.shape
    tau, table, rope_freqs = _f64(tau), _f64(table), _f64(rope_freqs)
    out, lse = _f64(out), _f64(lse)
    if out is not None:
        assert out.shape == q.shape
    if lse is not None:
        assert lse.shape == (B * (H // M) * (W // M), heads, M * M)
    g = {n: np.zeros((B, H, W, C), dtype=np.float64) for n in ("dq", "dk", "dv")}
    dtau = np.zeros(heads, dtype=np.float64) if sim == "cosine" else None
    dtable = np.zeros(((2 * M - 1) ** 2, heads), dtype=np.float64) if pos == "table" else None
    rc = (lib or load()).oracle_window_attn_bwd_given(
        B, H, W, C, heads, M, shift, PART[partition], SIM[sim], POS[pos],
        float(tau_min), float(rope_base), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(tau),
        _ptr(table), _ptr(rope_freqs), _ptr(out), _ptr(lse), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
        _ptr(dtau), _ptr(dtable))
    if rc:
        raise ValueError(f"oracle_window_attn_bwd: bad argument (rc={rc})")
    if dtau is not None:
        g["dtau"] = dtau
    if dtable is not None:
        g["dtable"] = dtable
    return g


def cpb_table_bwd(M: int, w1, b1, w2, b2, dtable, lib=None, mode: int = 0, norm_M: int | None = None):
    """Gradients (dw1, db1, dw2, db2) of sum(dtable * cpb_table(...)) in fp64."""
    w1, w2, dtable = _f64(w1), _f64(w2), _f64(dtable)
    b1, b2 = _f64(b1), _f64(b2)
    hidden, heads = w1.shape[0], w2.shape[0]
    assert dtable.shape == ((2 * M - 1) ** 2, heads)
    dw1, db1 = np.empty((hidden, 2)), np.empty(hidden)
    dw2, db2 = np.empty((heads, hidden)), np.empty(heads)
    rc = (lib or load()).oracle_cpb_table_bwd(M, M if norm_M is None else norm_M, heads, hidden, _ptr(w1),
                                              _ptr(b1), _ptr(w2), _ptr(b2), int(mode), _ptr(dtable),
                                              _ptr(dw1), _ptr(db1), _ptr(dw2), _ptr(db2))
    if rc:
        raise ValueError(f"oracle_cpb_table_bwd: bad argument (rc={rc})")
    return dw1, db1, dw2, db2


def window_cosines(q, k, *, heads: int, M: int, shift: int, partition: str, window: int,
                   head: int, pos: str = "none", rope_freqs=None, rope_base: float = 10000.0,
                   lib=None) -> np.ndarray:
    """N x N cosine similarities of one (window, head)."""
    q, k = _f64(q), _f64(k)
    B, H, W, C = q.shape
    N = M * M
    out = np.empty((N, N), dtype=np.float64)
    rc = (lib or load()).oracle_window_cosines(
        B, H, W, C, heads, M, shift, PART[partition], POS[pos], float(rope_base),
        _ptr(q), _ptr(k), _ptr(_f64(rope_freqs)), int(window), int(head), _ptr(out))
    if rc:
        raise ValueError("oracle_window_cosines: bad argument")
    return out


def linear(x, w, b=None, lib=None) -> np.ndarray:
    """x (..., in) times w^T (w: out x in) plus b, in fp64; leading dims kept."""
    x, w = _f64(x), _f64(w)
    out_f, in_f = w.shape
    assert x.shape[-1] == in_f
    xt = np.ascontiguousarray(x.reshape(-1, in_f))
    y = np.empty((xt.shape[0], out_f))
    bb = None if b is None else _f64(b)
    if bb is not None:
        assert bb.shape == (out_f,)
    rc = (lib or load()).oracle_linear(_ptr(xt), _ptr(w), _ptr(bb), _ptr(y), xt.shape[0], in_f, out_f)
    if rc:
        raise ValueError("oracle_linear: bad argument")
    return y.reshape(*x.shape[:-1], out_f)


def qkv_proj(x, w, b=None, lib=None):
    """The attention branch's input projection: (q, k, v), each shaped like x,
    from one linear layer C -> 3C whose outputs are q, k, v in that order."""
    y = linear(x, w, b, lib=lib)
    C = x.shape[-1]
    assert w.shape == (3 * C, C)
    return y[..., :C].copy(), y[..., C:2 * C].copy(), y[..., 2 * C:].copy()


def post_norm(resid, z, gamma, beta, eps: float = 1e-5, lib=None) -> np.ndarray:
    """resid + layer_norm(z) * gamma + beta over the last axis, in fp64."""
    resid, z, gamma, beta = _f64(resid), _f64(z), _f64(gamma), _f64(beta)
    C = z.shape[-1]
    assert resid.shape == z.shape and gamma.shape == (C,) and beta.shape == (C,)
    rt, zt = np.ascontiguousarray(resid.reshape(-1, C)), np.ascontiguousarray(z.reshape(-1, C))
    y = np.empty_like(zt)
    rc = (lib or load()).oracle_post_norm(_ptr(rt), _ptr(zt), _ptr(gamma), _ptr(beta), float(eps), _ptr(y),
                                          zt.shape[0], C)
    if rc:
        raise ValueError("oracle_post_norm: bad argument")
    return y.reshape(z.shape)


def proj_post_norm(o, w, b, resid, gamma, beta, eps: float = 1e-5, lib=None) -> np.ndarray:
    """The attention branch's output side: resid + norm_1(o w^T + b)."""
    return post_norm(resid, linear(o, w, b, lib=lib), gamma, beta, eps, lib=lib)


def dwconv_add(v, w, b, out, lib=None) -> np.ndarray:
    """out + depthwise 3x3 convolution of v (B, H, W, C) with w (C, 3, 3) and
    bias b (C) or None, zero padding, in fp64; returns a new array."""
    v, w, o = _f64(v), _f64(w), np.array(out, dtype=np.float64, copy=True)
    B, H, W, C = v.shape
    assert w.shape == (C, 3, 3) and o.shape == v.shape
    bb = None if b is None else _f64(b)
    rc = (lib or load()).oracle_dwconv_add(_ptr(v), _ptr(w), _ptr(bb), _ptr(o), B, H, W, C)
    if rc:
        raise ValueError(f"oracle_dwconv_add: bad argument (rc={rc})")
    return o


def window_linear(v, A, bias=None, *, heads: int, M: int, shift: int = 0, partition: str = "cyclic",
                  lib=None) -> np.ndarray:
    """Per window and head, out = A_h v (+ bias_h), cross-region pairs of
    shifted windows excluded; v (B, H, W, C), A (heads, N, N), bias (heads, N)."""
    v, A = _f64(v), _f64(A)
    B, H, W, C = v.shape
    N = M * M
    assert A.shape == (heads, N, N)
    bb = None if bias is None else _f64(bias)
    if bb is not None:
        assert bb.shape == (heads, N)
    out = np.empty_like(v)
    rc = (lib or load()).oracle_window_linear(B, H, W, C, heads, M, shift, PART[partition], _ptr(v), _ptr(A),
                                              _ptr(bb), _ptr(out))
    if rc:
        raise ValueError("oracle_window_linear: bad argument")
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return sys.platform


def cpb_table3d(Mt: int, M: int, w1, b1, w2, b2, lib=None) -> np.ndarray:
    """(2Mt-1)(2M-1)^2 x heads bias table of G over the log-spaced offsets
    (dx, dy, dt) of video windows Mt x M x M; w1 is hidden x 3."""
    w1, w2 = _f64(w1), _f64(w2)
    b1, b2 = _f64(b1), _f64(b2)
    hidden, heads = w1.shape[0], w2.shape[0]
    assert w1.shape == (hidden, 3) and w2.shape == (heads, hidden)
    out = np.empty(((2 * Mt - 1) * (2 * M - 1) ** 2, heads), dtype=np.float64)
    rc = (lib or load()).oracle_cpb_table3d(Mt, M, heads, hidden, _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(out))
    if rc:
        raise ValueError(f"oracle_cpb_table3d: bad argument (rc={rc})")
    return out


def window_attn3d(q, k, v, *, heads: int, Mt: int, M: int, shift_t: int = 0, shift: int = 0,
                  partition: str = "cyclic", sim: str = "cosine", pos: str = "none", tau=None, table=None,
                  tau_min: float = 0.01, windows=None, lib=None) -> np.ndarray:
    """Video-window attention forward in fp64 over (B, T, H, W, C) grids,
    windows Mt x M x M (temporal shift ``shift_t``, spatial ``shift``).
    ``windows``: optional global window ids to compute (the rest of the
    output stays zero)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, W, C = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    tau, table = _f64(tau), _f64(table)
    out = np.zeros((B, T, H, W, C), dtype=np.float64)
    win = None if windows is None else np.ascontiguousarray(windows, dtype=np.int64)
    rc = (lib or load()).oracle_window_attn3d(B, T, H, W, C, heads, Mt, M, shift_t, shift, PART[partition],
                                              SIM[sim], POS[pos], float(tau_min), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(tau), _ptr(table), _ptr(win), 0 if win is None else len(win),
                                              _ptr(out))
    if rc:
        raise ValueError(f"oracle_window_attn3d: bad argument (rc={rc})")
    return out
