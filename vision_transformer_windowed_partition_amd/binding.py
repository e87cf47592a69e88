"""Python binding of libswinattn.so (C ABI in include/swin_attn.h).

Argument marshalling only: each function checks that it was handed device
tensors of the sizes its descriptor implies (so a mismatch raises ValueError
here instead of sending a kernel past the end of a tensor), takes their data
pointers and the current HIP stream, and calls the C entry point of the same
name.  Every step of the computation runs in the
library's kernels; if the library is missing this module raises instead of
computing anything another way.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libswinattn.so")

SWIN_OK, SWIN_EINVAL, SWIN_EUNSUPPORTED, SWIN_EHIP = 0, 1, 2, 3
PARTITION = {"cyclic": 0, "interleaved": 1}
SIM = {"cosine": 0, "dot": 1}
POS = {"none": 0, "table": 1, "rope2d": 2}
DTYPE = {torch.float32: 0, torch.bfloat16: 1}
DTYPE_BY_NAME = {"f32": 0, "bf16": 1}
LAYOUT = {"grid": 0, "windows": 1}
CPB_PAPER = 0
CPB_CODE_NORM, CPB_SIGMOID16 = 1, 2       # flags; 3 = the released code


class SwinAttnDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "H", "W", "C", "heads", "M", "shift", "partition", "sim", "pos", "dtype", "layout")] + \
               [("tau_min", ctypes.c_float), ("rope_base", ctypes.c_float)]


class SwinError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{swin_status_string(status)} -- {detail}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        i32, vp, f = ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
        L.swin_cpb_table.restype = i32
        L.swin_cpb_table.argtypes = [i32, i32, i32, vp, vp, vp, vp, i32, vp, vp]
        L.swin_cpb_table_ex.restype = i32
        L.swin_cpb_table_ex.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, i32, vp, vp]
        L.swin_cpb_table_resize.restype = i32
        L.swin_cpb_table_resize.argtypes = [i32, i32, i32, vp, vp, vp]
        for fn in (L.swin_window_partition, L.swin_window_reverse):
            fn.restype = i32
            fn.argtypes = [vp, vp] + [i32] * 8 + [vp]
        L.swin_window_attn_fwd.restype = i32
        L.swin_window_attn_fwd.argtypes = [ctypes.POINTER(SwinAttnDesc)] + [vp] * 8
        L.swin_window_attn_bwd.restype = i32
        L.swin_window_attn_bwd.argtypes = [ctypes.POINTER(SwinAttnDesc)] + [vp] * 14
        L.swin_cpb_table3d.restype = i32
        L.swin_cpb_table3d.argtypes = [i32] * 4 + [vp] * 6
        L.swin_window_attn3d_fwd.restype = i32
        L.swin_window_attn3d_fwd.argtypes = [ctypes.POINTER(SwinAttnDesc), i32, i32, i32] + [vp] * 7
        L.swin_window_attn3d_kernel.restype = ctypes.c_char_p
        L.swin_window_attn3d_kernel.argtypes = [ctypes.POINTER(SwinAttnDesc), i32, i32]
        L.swin_window_attn_fwd_lse.restype = i32
        L.swin_window_attn_fwd_lse.argtypes = [ctypes.POINTER(SwinAttnDesc)] + [vp] * 9
        L.swin_window_attn_bwd_lse.restype = i32
        L.swin_window_attn_bwd_lse.argtypes = [ctypes.POINTER(SwinAttnDesc)] + [vp] * 15
        L.swin_cpb_table_bwd.restype = i32
        L.swin_cpb_table_bwd.argtypes = [i32] * 4 + [vp] * 5 + [i32] + [vp] * 5
        L.swin_qkv_proj.restype = i32
        L.swin_qkv_proj.argtypes = [vp] * 6 + [ctypes.c_int64, i32, i32, vp]
        L.swin_qkv_window_attn_fwd.restype = i32
        L.swin_qkv_window_attn_fwd.argtypes = [ctypes.POINTER(SwinAttnDesc)] + [vp] * 7
        L.swin_proj_post_norm.restype = i32
        L.swin_proj_post_norm.argtypes = [vp] * 6 + [ctypes.c_float, vp, ctypes.c_int64, i32, i32, vp]
        L.swin_dwconv_add.restype = i32
        L.swin_dwconv_add.argtypes = [vp] * 4 + [i32] * 5 + [vp]
        L.swin_window_linear.restype = i32
        L.swin_window_linear.argtypes = [ctypes.POINTER(SwinAttnDesc)] + [vp] * 5
        L.swin_window_attn_kernel.restype = ctypes.c_char_p
        L.swin_window_attn_kernel.argtypes = [ctypes.POINTER(SwinAttnDesc)]
        L.swin_window_attn_bwd_kernel.restype = ctypes.c_char_p
        L.swin_window_attn_bwd_kernel.argtypes = [ctypes.POINTER(SwinAttnDesc)]
        L.swin_status_string.restype = ctypes.c_char_p
        L.swin_status_string.argtypes = [i32]
        L.swin_last_error.restype = ctypes.c_char_p
        L.swin_last_error.argtypes = []
        L.swin_version.restype = i32
        L.swin_version.argtypes = []
        _lib = L
    return _lib


def swin_status_string(status: int) -> str:
    return lib().swin_status_string(int(status)).decode()


def swin_last_error() -> str:
    return lib().swin_last_error().decode()


def swin_version() -> int:
    return int(lib().swin_version())


def _check(rc: int) -> None:
    if rc != SWIN_OK:
        raise SwinError(rc, swin_last_error())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    return t.data_ptr()


def _stream(t, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(t.device).cuda_stream


def _enum(table, v):
    return table[v] if isinstance(v, str) else int(v)


def _check_attn(desc: SwinAttnDesc, q, tau, table, rope_freqs, out=None, *, T=None, Mt: int = 1) -> None:
    """Sizes of what a window-attention call reads and writes, checked against
    the descriptor before the C call, so a mismatch raises here instead of
    sending a kernel past the end of a tensor.  T, Mt: video frames and
    temporal window (T None for the 2D calls)."""
    dev = q.device
    frames = 1 if T is None else T
    if q.numel() != desc.B * frames * desc.H * desc.W * desc.C:
        raise ValueError(f"q holds {q.numel()} elements; the descriptor's grid needs "
                         f"{desc.B * frames * desc.H * desc.W * desc.C}")
    if desc.layout == LAYOUT["grid"] and T is None and tuple(q.shape) != (desc.B, desc.H, desc.W, desc.C):
        raise ValueError(f"q must be (B, H, W, C) = {(desc.B, desc.H, desc.W, desc.C)}, got {tuple(q.shape)}")
    heads, M = desc.heads, desc.M
    d = desc.C // heads if heads > 0 else 0
    need = []
    if desc.sim == SIM["cosine"]:
        need.append(("tau", tau, heads))
    if desc.pos == POS["table"]:
        need.append(("table", table, (2 * Mt - 1) * (2 * M - 1) ** 2 * heads))
    if desc.pos == POS["rope2d"] and rope_freqs is not None:
        need.append(("rope_freqs", rope_freqs, heads * 2 * (d // 4)))
    for name, t, n in need:
        if t is None:
            continue                    # the library rejects a missing required pointer
        if t.numel() != n:
            raise ValueError(f"{name} must hold {n} fp32 values, got {t.numel()}")
    for t in (tau, table, rope_freqs):
        if t is not None and t.device != dev:
            raise ValueError("tau, table and rope_freqs must be on q's device")
    if out is not None:
        if out.shape != q.shape or out.dtype != q.dtype or out.device != dev or not out.is_contiguous():
            raise ValueError("out must be a contiguous tensor of q's shape, dtype and device")


def swin_cpb_table(M: int, w1, b1, w2, b2, *, out=None, cpb_mode: int = CPB_PAPER, norm_M=None, stream=None):
    """(2M-1)^2 x heads fp32 bias table from the meta network parameters.
    cpb_mode: CPB_PAPER, or the flags CPB_CODE_NORM | CPB_SIGMOID16; norm_M:
    the window that normalises the offsets under CPB_CODE_NORM (default M)."""
    heads, hidden = w2.shape
    for t in (w1, b1, w2, b2, out):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("CPB parameters and table must be contiguous fp32")
    if out is None:
        out = torch.empty(((2 * M - 1) ** 2, heads), dtype=torch.float32, device=w1.device)
    if norm_M is None:
        _check(lib().swin_cpb_table(M, heads, hidden, _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2),
                                    cpb_mode, _ptr(out), _stream(w1, stream)))
    else:
        _check(lib().swin_cpb_table_ex(M, norm_M, heads, hidden, _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2),
                                       cpb_mode, _ptr(out), _stream(w1, stream)))
    return out


def swin_cpb_table_resize(table, M_src: int, M_dst: int, *, out=None, stream=None):
    """A (2*M_src-1)^2 x heads fp32 bias table resampled bi-cubically to
    (2*M_dst-1)^2 x heads (the Swin V1 transfer between window sizes)."""
    if table.dtype != torch.float32 or not table.is_contiguous() or table.dim() != 2:
        raise ValueError("the table must be a contiguous 2D fp32 tensor")
    heads = table.shape[1]
    if table.shape[0] != (2 * M_src - 1) ** 2:
        raise ValueError(f"table rows {table.shape[0]} != (2*{M_src}-1)^2")
    if out is None:
        out = torch.empty(((2 * M_dst - 1) ** 2, heads), dtype=torch.float32, device=table.device)
    elif out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != ((2 * M_dst - 1) ** 2, heads):
        raise ValueError("out must be a contiguous fp32 ((2*M_dst-1)^2, heads) tensor")
    if out.device != table.device:
        raise ValueError("table and out must be on one device")
    _check(lib().swin_cpb_table_resize(M_src, M_dst, heads, _ptr(table), _ptr(out), _stream(table, stream)))
    return out


def swin_window_partition(x, M: int, shift: int, partition="cyclic", *, out=None, stream=None):
    """(B, H, W, C) grid -> (B*nW, M*M, C) windows (bit-exact gather)."""
    B, H, W, C = x.shape
    if out is None:
        out = torch.empty((B * (H // max(M, 1)) * (W // max(M, 1)), M * M, C), dtype=x.dtype, device=x.device)
    if not x.is_contiguous() or not out.is_contiguous():
        raise ValueError("tensors must be contiguous")
    _check(lib().swin_window_partition(_ptr(x), _ptr(out), B, H, W, C, M, shift,
                                       _enum(PARTITION, partition), DTYPE[x.dtype], _stream(x, stream)))
    return out


def swin_window_reverse(xw, B: int, H: int, W: int, M: int, shift: int, partition="cyclic", *,
                        out=None, stream=None):
    """(B*nW, M*M, C) windows -> (B, H, W, C) grid (bit-exact scatter)."""
    C = xw.shape[-1]
    if out is None:
        out = torch.empty((B, H, W, C), dtype=xw.dtype, device=xw.device)
    if not xw.is_contiguous() or not out.is_contiguous():
        raise ValueError("tensors must be contiguous")
    _check(lib().swin_window_reverse(_ptr(xw), _ptr(out), B, H, W, C, M, shift,
                                     _enum(PARTITION, partition), DTYPE[xw.dtype], _stream(xw, stream)))
    return out


def make_desc(*, B, H, W, C, heads, M, shift=0, partition="cyclic", sim="cosine", pos="none",
              dtype=torch.bfloat16, layout="grid", tau_min=0.01, rope_base=10000.0) -> SwinAttnDesc:
    return SwinAttnDesc(B, H, W, C, heads, M, shift, _enum(PARTITION, partition), _enum(SIM, sim),
                        _enum(POS, pos), DTYPE[dtype] if isinstance(dtype, torch.dtype) else int(dtype),
                        _enum(LAYOUT, layout), float(tau_min), float(rope_base))


def swin_window_attn_fwd(q, k, v, *, heads: int, M: int, shift: int = 0, partition="cyclic",
                         sim="cosine", pos="none", tau=None, table=None, rope_freqs=None,
                         tau_min: float = 0.01, rope_base: float = 10000.0, layout="grid",
                         grid=None, out=None, desc: SwinAttnDesc | None = None, stream=None):
    """Windowed attention forward.  q, k, v: (B, H, W, C) for layout "grid", or
    (B*nW, M*M, C) for layout "windows" with grid=(B, H, W)."""
    if desc is None:
        if _enum(LAYOUT, layout) == 0:
            B, H, W, C = q.shape
        else:
            B, H, W = grid
            C = q.shape[-1]
        desc = make_desc(B=B, H=H, W=W, C=C, heads=heads, M=M, shift=shift, partition=partition,
                         sim=sim, pos=pos, dtype=q.dtype, layout=layout, tau_min=tau_min,
                         rope_base=rope_base)
    for t in (q, k, v):
        if not t.is_contiguous() or t.dtype != q.dtype or t.shape != q.shape or t.device != q.device:
            raise ValueError("q, k, v must be contiguous tensors of one shape, dtype and device")
    for t in (tau, table, rope_freqs):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("tau, table and rope_freqs must be contiguous fp32")
    _check_attn(desc, q, tau, table, rope_freqs, out)
    if out is None:
        out = torch.empty_like(q)
    _check(lib().swin_window_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                      _ptr(tau), _ptr(table), _ptr(rope_freqs), _stream(q, stream)))
    return out


def swin_window_attn_fwd_lse(q, k, v, *, heads: int, M: int, shift: int = 0, partition="cyclic",
                             sim="cosine", pos="none", tau=None, table=None, rope_freqs=None,
                             tau_min: float = 0.01, rope_base: float = 10000.0, layout="grid",
                             grid=None, out=None, lse=None, desc: SwinAttnDesc | None = None, stream=None):
    """swin_window_attn_fwd that also returns the per-query natural-log
    log-sum-exp of the logits, fp32 (n_windows, heads, M*M): (out, lse)."""
    if desc is None:
        if _enum(LAYOUT, layout) == 0:
            B, H, W, C = q.shape
        else:
            B, H, W = grid
            C = q.shape[-1]
        desc = make_desc(B=B, H=H, W=W, C=C, heads=heads, M=M, shift=shift, partition=partition,
                         sim=sim, pos=pos, dtype=q.dtype, layout=layout, tau_min=tau_min,
                         rope_base=rope_base)
    for t in (q, k, v):
        if not t.is_contiguous() or t.dtype != q.dtype or t.shape != q.shape or t.device != q.device:
            raise ValueError("q, k, v must be contiguous tensors of one shape, dtype and device")
    for t in (tau, table, rope_freqs):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("tau, table and rope_freqs must be contiguous fp32")
    _check_attn(desc, q, tau, table, rope_freqs, out)
    nwin = desc.B * (desc.H // max(desc.M, 1)) * (desc.W // max(desc.M, 1))
    shape = (nwin, desc.heads, desc.M * desc.M)
    if lse is None:
        lse = torch.empty(shape, dtype=torch.float32, device=q.device)
    elif lse.shape != shape or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError(f"lse must be contiguous fp32 of shape {shape}")
    if out is None:
        out = torch.empty_like(q)
    _check(lib().swin_window_attn_fwd_lse(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                          _ptr(tau), _ptr(table), _ptr(rope_freqs), _ptr(lse),
                                          _stream(q, stream)))
    return out, lse


def swin_cpb_table3d(Mt: int, M: int, w1, b1, w2, b2, *, out=None, stream=None):
    """((2Mt-1)(2M-1)^2, heads) fp32 bias table of video windows; w1 is (hidden, 3)."""
    hidden, heads = w1.shape[0], w2.shape[0]
    for t in (w1, b1, w2, b2):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("w1, b1, w2, b2 must be contiguous fp32")
    if w1.shape != (hidden, 3) or w2.shape != (heads, hidden):
        raise ValueError("w1 must be (hidden, 3) and w2 (heads, hidden)")
    if out is None:
        out = torch.empty(((2 * Mt - 1) * (2 * M - 1) ** 2, heads), dtype=torch.float32, device=w1.device)
    _check(lib().swin_cpb_table3d(Mt, M, heads, hidden, _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(out),
                                  _stream(w1, stream)))
    return out


def swin_window_attn3d_fwd(q, k, v, *, heads: int, Mt: int, M: int, shift_t: int = 0, shift: int = 0,
                           partition="cyclic", sim="cosine", pos="none", tau=None, table=None,
                           tau_min: float = 0.01, out=None, stream=None):
    """Video-window attention forward: q, k, v (B, T, H, W, C), windows Mt x M x M."""
    for t in (q, k, v):
        if not t.is_contiguous() or t.dtype != q.dtype or t.shape != q.shape or t.dim() != 5:
            raise ValueError("q, k, v must be contiguous (B, T, H, W, C) tensors of one shape and dtype")
    for t in (tau, table):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("tau and table must be contiguous fp32")
    B, T, H, W, C = q.shape
    desc = make_desc(B=B, H=H, W=W, C=C, heads=heads, M=M, shift=shift, partition=partition, sim=sim, pos=pos,
                     dtype=q.dtype, tau_min=tau_min)
    _check_attn(desc, q, tau, table, None, out, T=T, Mt=Mt)
    if out is None:
        out = torch.empty_like(q)
    _check(lib().swin_window_attn3d_fwd(ctypes.byref(desc), T, Mt, shift_t, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                        _ptr(tau), _ptr(table), _stream(q, stream)))
    return out


def swin_window_attn3d_kernel(desc: SwinAttnDesc, T: int, Mt: int) -> str:
    """Name of the kernel swin_window_attn3d_fwd runs for this descriptor."""
    return lib().swin_window_attn3d_kernel(ctypes.byref(desc), T, Mt).decode()


def swin_window_attn_bwd(q, k, v, out, dout, *, heads: int, M: int, shift: int = 0, partition="cyclic",
                         sim="cosine", pos="none", tau=None, table=None, rope_freqs=None,
                         tau_min: float = 0.01, rope_base: float = 10000.0, layout="grid", grid=None,
                         want_dtau: bool = True, want_dtable: bool = True, desc: SwinAttnDesc | None = None,
                         stream=None, lse=None) -> dict:
    """Backward of swin_window_attn_fwd: dq, dk, dv (like q), and dtau
    (heads fp32, COSINE) and dtable ((2M-1)^2 x heads fp32, TABLE) when wanted.
    ``lse``: the forward's log-sum-exp from swin_window_attn_fwd_lse; when
    given, the call goes to swin_window_attn_bwd_lse."""
    if desc is None:
        if _enum(LAYOUT, layout) == 0:
            B, H, W, C = q.shape
        else:
            B, H, W = grid
            C = q.shape[-1]
        desc = make_desc(B=B, H=H, W=W, C=C, heads=heads, M=M, shift=shift, partition=partition,
                         sim=sim, pos=pos, dtype=q.dtype, layout=layout, tau_min=tau_min,
                         rope_base=rope_base)
    for t in (q, k, v, out, dout):
        if not t.is_contiguous() or t.dtype != q.dtype or t.shape != q.shape:
            raise ValueError("q, k, v, out, dout must be contiguous tensors of one shape and dtype")
    for t in (tau, table, rope_freqs):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("tau, table and rope_freqs must be contiguous fp32")
    _check_attn(desc, q, tau, table, rope_freqs)
    for t in (k, v, out, dout):
        if t.device != q.device:
            raise ValueError("q, k, v, out, dout must be on one device")
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(q), "dv": torch.empty_like(q)}
    dtau = dtable = None
    if want_dtau and _enum(SIM, sim) == 0:
        dtau = g["dtau"] = torch.empty(heads, dtype=torch.float32, device=q.device)
    if want_dtable and _enum(POS, pos) == 1:
        dtable = g["dtable"] = torch.empty(((2 * M - 1) ** 2, heads), dtype=torch.float32, device=q.device)
    if lse is None:
        _check(lib().swin_window_attn_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                                          _ptr(tau), _ptr(table), _ptr(rope_freqs), _ptr(g["dq"]), _ptr(g["dk"]),
                                          _ptr(g["dv"]), _ptr(dtau), _ptr(dtable), _stream(q, stream)))
    else:
        nwin = desc.B * (desc.H // max(desc.M, 1)) * (desc.W // max(desc.M, 1))
        if lse.shape != (nwin, desc.heads, desc.M * desc.M) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse must be the forward's contiguous fp32 (n_windows, heads, M*M)")
        _check(lib().swin_window_attn_bwd_lse(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                              _ptr(dout), _ptr(tau), _ptr(table), _ptr(rope_freqs), _ptr(lse),
                                              _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(dtau), _ptr(dtable),
                                              _stream(q, stream)))
    return g


def swin_window_attn_bwd_lse(q, k, v, out, dout, lse, **kw) -> dict:
    """swin_window_attn_bwd given the forward's log-sum-exp (see there)."""
    return swin_window_attn_bwd(q, k, v, out, dout, lse=lse, **kw)


def swin_cpb_table_bwd(M: int, w1, b1, w2, table, dtable, *, cpb_mode: int = CPB_PAPER, norm_M=None,
                       stream=None):
    """Gradients (dw1, db1, dw2, db2) of the meta network from dtable; table is
    the forward's table (needed for CPB_SIGMOID16)."""
    heads, hidden = w2.shape
    for t in (w1, b1, w2, table, dtable):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("CPB parameters and tables must be contiguous fp32")
    dw1, dw2 = torch.empty_like(w1), torch.empty_like(w2)
    db1 = torch.empty(hidden, dtype=torch.float32, device=w1.device)
    db2 = torch.empty(heads, dtype=torch.float32, device=w1.device)
    _check(lib().swin_cpb_table_bwd(M, M if norm_M is None else norm_M, heads, hidden, _ptr(w1), _ptr(b1),
                                    _ptr(w2), _ptr(table), _ptr(dtable), cpb_mode, _ptr(dw1), _ptr(db1),
                                    _ptr(dw2), _ptr(db2), _stream(w1, stream)))
    return dw1, db1, dw2, db2


def _proj_dtype(x):
    if x.dtype not in DTYPE:
        raise ValueError("features must be bf16 or fp32")
    return DTYPE[x.dtype]


def swin_qkv_proj(x, w, b=None, *, out=None, stream=None):
    """(q, k, v) = split(x w^T + b) of the attention branch's input layer:
    x (..., C), w (3C, C) in x's dtype, b (3C) fp32 or None.  Returns three
    tensors shaped like x (or fills out=(q, k, v))."""
    C = x.shape[-1]
    dt = _proj_dtype(x)
    if w.dtype != x.dtype or tuple(w.shape) != (3 * C, C) or not (x.is_contiguous() and w.is_contiguous()):
        raise ValueError("w must be a contiguous (3C, C) tensor of x's dtype; x contiguous")
    if b is not None and (b.dtype != torch.float32 or tuple(b.shape) != (3 * C,) or not b.is_contiguous()):
        raise ValueError("b must be contiguous fp32 of 3C")
    q, k, v = out if out is not None else (torch.empty_like(x), torch.empty_like(x), torch.empty_like(x))
    _check(lib().swin_qkv_proj(_ptr(x), _ptr(w), _ptr(b), _ptr(q), _ptr(k), _ptr(v), x.numel() // C, C, dt,
                               _stream(x, stream)))
    return q, k, v


def swin_qkv_window_attn_fwd(x, w_qkv, b_qkv=None, *, heads: int, M: int, shift: int = 0, partition="cyclic",
                             sim="cosine", pos="none", tau=None, table=None, tau_min: float = 0.01, out=None,
                             stream=None):
    """Window attention of q, k, v = split(x w_qkv^T + b_qkv), the input layer
    fused in: x (B, H, W, C) bf16, w_qkv (3C, C) bf16, b_qkv (3C,) fp32 or
    None; returns the attention output (B, H, W, C)."""
    if x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous (B, H, W, C) tensor")
    B, H, W, C = x.shape
    if w_qkv.shape != (3 * C, C) or w_qkv.dtype != x.dtype or not w_qkv.is_contiguous() or w_qkv.device != x.device:
        raise ValueError("w_qkv must be a contiguous (3C, C) tensor of x's dtype and device")
    if b_qkv is not None and (b_qkv.shape != (3 * C,) or b_qkv.dtype != torch.float32 or not b_qkv.is_contiguous()
                              or b_qkv.device != x.device):
        raise ValueError("b_qkv must be contiguous fp32 of 3C on x's device")
    for t in (tau, table):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("tau and table must be contiguous fp32")
    desc = make_desc(B=B, H=H, W=W, C=C, heads=heads, M=M, shift=shift, partition=partition, sim=sim, pos=pos,
                     dtype=x.dtype, tau_min=tau_min)
    _check_attn(desc, x, tau, table, None, out)
    if out is None:
        out = torch.empty_like(x)
    _check(lib().swin_qkv_window_attn_fwd(ctypes.byref(desc), _ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(out),
                                          _ptr(tau), _ptr(table), _stream(x, stream)))
    return out


def swin_proj_post_norm(o, w, b, resid, gamma, beta, *, eps: float = 1e-5, out=None, stream=None):
    """resid + layer_norm(o w^T + b) * gamma + beta over the channels: the
    attention branch's output layer and residual post-norm.  o, resid (..., C)
    and w (C, C) share a dtype; b (or None), gamma, beta are fp32 (C).
    out may be resid itself."""
    C = o.shape[-1]
    dt = _proj_dtype(o)
    if (w.dtype != o.dtype or resid.dtype != o.dtype or tuple(w.shape) != (C, C) or resid.shape != o.shape
            or not (o.is_contiguous() and w.is_contiguous() and resid.is_contiguous())):
        raise ValueError("o, resid (same shape) and w (C, C) must be contiguous and share a dtype")
    for t in (b, gamma, beta):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (C,) or not t.is_contiguous()):
            raise ValueError("b, gamma and beta must be contiguous fp32 of C")
    y = out if out is not None else torch.empty_like(o)
    _check(lib().swin_proj_post_norm(_ptr(o), _ptr(w), _ptr(b), _ptr(resid), _ptr(gamma), _ptr(beta), float(eps),
                                     _ptr(y), o.numel() // C, C, dt, _stream(o, stream)))
    return y


def swin_dwconv_add(v, w, b, out, *, stream=None):
    """out += depthwise 3x3 convolution of v (zero padding) with w (C, 3, 3)
    fp32 and bias b (C) fp32 or None; v and out (B, H, W, C) of one dtype.
    Returns out."""
    if v.dim() != 4 or out.shape != v.shape or out.dtype != v.dtype:
        raise ValueError("v and out must be (B, H, W, C) tensors of one dtype")
    B, H, W, C = v.shape
    if w.dtype != torch.float32 or tuple(w.shape) != (C, 3, 3) or not w.is_contiguous():
        raise ValueError("w must be contiguous fp32 (C, 3, 3)")
    if b is not None and (b.dtype != torch.float32 or tuple(b.shape) != (C,) or not b.is_contiguous()):
        raise ValueError("b must be contiguous fp32 of C")
    if not (v.is_contiguous() and out.is_contiguous()):
        raise ValueError("v and out must be contiguous")
    _check(lib().swin_dwconv_add(_ptr(v), _ptr(w), _ptr(b), _ptr(out), B, H, W, C, _proj_dtype(v),
                                 _stream(v, stream)))
    return out


def swin_window_linear(v, A, bias=None, *, heads: int, M: int, shift: int = 0, partition="cyclic", out=None,
                       stream=None):
    """LinMapper's in-window linear mapping: per window and head
    out_i = bias_h[i] + sum_j A_h[i][j] v_j (shifted-window regions excluded).
    v (B, H, W, C); A (heads, M*M, M*M) in v's dtype; bias (heads, M*M) fp32."""
    B, H, W, C = v.shape
    N = M * M
    if A.dtype != v.dtype or tuple(A.shape) != (heads, N, N) or not (A.is_contiguous() and v.is_contiguous()):
        raise ValueError("A must be a contiguous (heads, M*M, M*M) tensor of v's dtype")
    if bias is not None and (bias.dtype != torch.float32 or tuple(bias.shape) != (heads, N) or not bias.is_contiguous()):
        raise ValueError("bias must be contiguous fp32 (heads, M*M)")
    desc = make_desc(B=B, H=H, W=W, C=C, heads=heads, M=M, shift=shift, partition=partition, sim="dot",
                     pos="none", dtype=v.dtype)
    o = out if out is not None else torch.empty_like(v)
    _check(lib().swin_window_linear(ctypes.byref(desc), _ptr(v), _ptr(A), _ptr(bias), _ptr(o), _stream(v, stream)))
    return o


def swin_window_attn_kernel(desc: SwinAttnDesc) -> str:
    """Name of the kernel swin_window_attn_fwd launches for desc (for
    matching profiler output).  Raises SwinError if the descriptor is rejected."""
    name = lib().swin_window_attn_kernel(ctypes.byref(desc))
    if name is None:
        raise SwinError(SWIN_EINVAL, swin_last_error())
    return name.decode()


def swin_window_attn_bwd_kernel(desc: SwinAttnDesc) -> str:
    """Name of the kernel swin_window_attn_bwd launches for desc (for
    matching profiler output).  Raises SwinError if the descriptor is rejected."""
    name = lib().swin_window_attn_bwd_kernel(ctypes.byref(desc))
    if name is None:
        raise SwinError(SWIN_EUNSUPPORTED, swin_last_error())
    return name.decode()
