"""Host-side checks of libswinattn.so (no GPU needed, nothing is launched):
the library loads, exports every function include/swin_attn.h declares, and
rejects bad arguments with the documented status before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

from vision_transformer_windowed_partition_amd import binding
from vision_transformer_windowed_partition_amd.binding import (SWIN_EINVAL, SWIN_EUNSUPPORTED,
                                                               SWIN_OK, SwinAttnDesc)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swin_attn.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|char\s*\*|const char\s*\*)\s*\**\s*(swin_\w+)\s*\(",
                                 src, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libswinattn.so not built")
    return binding.lib()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(["swin_cpb_table", "swin_cpb_table_ex", "swin_cpb_table_bwd",
                                           "swin_window_attn_bwd", "swin_window_partition",
                                           "swin_window_reverse",
                                           "swin_window_attn_fwd", "swin_window_attn_kernel",
                                           "swin_window_attn_fwd_lse", "swin_window_attn_bwd_lse",
                                           "swin_cpb_table3d", "swin_window_attn3d_fwd",
                                           "swin_window_attn3d_kernel",
                                           "swin_window_attn_bwd_kernel", "swin_cpb_table_resize",
                                           "swin_qkv_proj", "swin_qkv_window_attn_fwd", "swin_proj_post_norm",
                                           "swin_dwconv_add",
                                           "swin_window_linear",
                                           "swin_status_string",
                                           "swin_last_error", "swin_version"])


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True)
    if out.returncode == 0:
        for name in declared_functions():
            assert re.search(rf"\bT {name}$", out.stdout, flags=re.M), name


def test_version_and_status_strings(L):
    assert binding.swin_version() == 1
    for s in (0, 1, 2, 3):
        assert binding.swin_status_string(s).startswith("SWIN_")
    assert "unknown" in binding.swin_status_string(99)


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first


def _desc(**kw):
    d = dict(B=1, H=16, W=16, C=64, heads=2, M=8, shift=4, partition=0, sim=0, pos=1, dtype=1,
             layout=0, tau_min=0.01, rope_base=10000.0)
    d.update(kw)
    return SwinAttnDesc(*[d[f] for f, _ in SwinAttnDesc._fields_])


def _attn(L, desc, q=FAKE, k=FAKE, v=FAKE, out=ctypes.c_void_p(0x20000000), tau=FAKE, table=FAKE):
    return L.swin_window_attn_fwd(ctypes.byref(desc) if desc is not None else None,
                                  q, k, v, out, tau, table, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=12), SWIN_EUNSUPPORTED),          # H % M != 0 (no padding built)
    (dict(M=32), SWIN_EUNSUPPORTED),          # window larger than the grid
    (dict(C=96, heads=2), SWIN_EUNSUPPORTED), # head dim 48
    (dict(C=64, heads=3), SWIN_EINVAL),       # C % heads
    (dict(shift=8), SWIN_EINVAL),             # shift >= M
    (dict(shift=-1), SWIN_EINVAL),
    (dict(partition=1, shift=4), SWIN_EINVAL),  # interleaved windows take no shift
    (dict(partition=2), SWIN_EINVAL),
    (dict(sim=5), SWIN_EINVAL),
    (dict(pos=7), SWIN_EINVAL),
    (dict(dtype=3), SWIN_EINVAL),
    (dict(layout=2), SWIN_EINVAL),
    (dict(tau_min=0.0), SWIN_EINVAL),
    (dict(B=-1), SWIN_EINVAL),
    (dict(H=0), SWIN_EINVAL),
])
def test_attn_rejects_bad_descriptors(L, kw, status):
    assert _attn(L, _desc(**kw)) == status
    assert binding.swin_last_error() != ""


def test_attn_rejects_bad_pointers(L):
    d = _desc()
    assert _attn(L, None) == SWIN_EINVAL
    assert _attn(L, d, q=None) == SWIN_EINVAL
    assert _attn(L, d, out=None) == SWIN_EINVAL
    assert _attn(L, d, tau=None) == SWIN_EINVAL                     # COSINE needs tau
    assert _attn(L, d, table=None) == SWIN_EINVAL                   # TABLE needs the table
    assert _attn(L, d, q=ctypes.c_void_p(0x10008)) == SWIN_EINVAL   # misaligned
    assert _attn(L, d, out=ctypes.c_void_p(0x10000 + 64)) == SWIN_EINVAL   # out overlaps q
    assert _attn(L, _desc(pos=2, rope_base=0.0)) == SWIN_EINVAL


def _bwd(L, desc, q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, dq=ctypes.c_void_p(0x20000000),
         dk=ctypes.c_void_p(0x30000000), dv=ctypes.c_void_p(0x40000000), tau=FAKE, table=FAKE,
         dtau=None, dtable=None):
    return L.swin_window_attn_bwd(ctypes.byref(desc) if desc is not None else None, q, k, v, out, dout, tau,
                                  table, None, dq, dk, dv, dtau, dtable, None)


def test_lse_entries_reject(L):
    """The log-sum-exp variants: a missing, misaligned or overlapping lse is
    refused before anything is launched."""
    d = _desc()
    fwd = lambda lse, out=ctypes.c_void_p(0x20000000): L.swin_window_attn_fwd_lse(
        ctypes.byref(d), FAKE, FAKE, FAKE, out, FAKE, FAKE, None, lse, None)
    assert fwd(None) == SWIN_EINVAL
    assert fwd(ctypes.c_void_p(0x30000002)) == SWIN_EINVAL                  # misaligned
    assert fwd(ctypes.c_void_p(0x20000000 + 64)) == SWIN_EINVAL             # overlaps out
    assert fwd(ctypes.c_void_p(0x10000 + 4096)) == SWIN_EINVAL              # overlaps q
    bwd = lambda lse: L.swin_window_attn_bwd_lse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                                 lse, ctypes.c_void_p(0x20000000), ctypes.c_void_p(0x30000000),
                                                 ctypes.c_void_p(0x40000000), None, None, None)
    assert bwd(None) == SWIN_EINVAL
    assert bwd(ctypes.c_void_p(0x50000001)) == SWIN_EINVAL                  # misaligned
    assert L.swin_window_attn_fwd_lse(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == SWIN_EINVAL


def test_video_entries_reject(L):
    """Video windows: bad temporal geometry, rotary positions, the windows
    layout, missing tensors and misalignment are refused before any launch."""
    f = lambda d=None, T=4, Mt=2, st=1, q=FAKE, out=ctypes.c_void_p(0x20000000), tau=FAKE, table=FAKE: \
        L.swin_window_attn3d_fwd(ctypes.byref(d if d is not None else _desc()), T, Mt, st, q, FAKE, FAKE, out, tau,
                                 table, None)
    assert f(T=5) == SWIN_EINVAL                          # T % Mt
    assert f(T=0) == SWIN_EINVAL
    assert f(st=2) == SWIN_EINVAL                         # shift_t >= Mt
    assert f(st=-1) == SWIN_EINVAL
    assert f(d=_desc(partition=1, shift=0), st=1) == SWIN_EINVAL      # interleaved takes no shift
    assert f(d=_desc(pos=2)) == SWIN_EUNSUPPORTED         # no rotary form in 3D
    assert f(d=_desc(layout=1)) == SWIN_EUNSUPPORTED
    assert f(Mt=65, T=65, st=0) == SWIN_EUNSUPPORTED
    assert f(q=None) == SWIN_EINVAL
    assert f(tau=None) == SWIN_EINVAL                     # COSINE needs tau
    assert f(table=None) == SWIN_EINVAL                   # TABLE needs the table
    assert f(q=ctypes.c_void_p(0x10008)) == SWIN_EINVAL   # misaligned
    assert f(out=ctypes.c_void_p(0x10000 + 64)) == SWIN_EINVAL       # out overlaps q
    t3 = lambda Mt=2, M=4, heads=2, hidden=8, table=ctypes.c_void_p(0x20000000): L.swin_cpb_table3d(
        Mt, M, heads, hidden, FAKE, None, ctypes.c_void_p(0x30000000), None, table, None)
    assert t3(Mt=0) == SWIN_EINVAL and t3(M=65) == SWIN_EINVAL and t3(heads=0) == SWIN_EINVAL
    assert t3(hidden=0) == SWIN_EINVAL and t3(table=None) == SWIN_EINVAL
    assert t3(table=ctypes.c_void_p(0x10000 + 16)) == SWIN_EINVAL      # overlaps w1


def _qkv(L, x=FAKE, w=ctypes.c_void_p(0x30000000), b=None, q=ctypes.c_void_p(0x40000000),
         k=ctypes.c_void_p(0x50000000), v=ctypes.c_void_p(0x60000000), T=64, C=96, dtype=1):
    return L.swin_qkv_proj(x, w, b, q, k, v, T, C, dtype, None)


def _pnorm(L, o=FAKE, w=ctypes.c_void_p(0x30000000), b=None, resid=ctypes.c_void_p(0x40000000),
           gamma=ctypes.c_void_p(0x50000000), beta=ctypes.c_void_p(0x50001000),
           y=ctypes.c_void_p(0x60000000), eps=1e-5, T=64, C=96, dtype=1):
    return L.swin_proj_post_norm(o, w, b, resid, gamma, beta, eps, y, T, C, dtype, None)


def test_projection_rejects(L):
    """Host validation of the branch's linear layers: nothing is launched."""
    assert _qkv(L, C=80) == SWIN_EUNSUPPORTED                                   # not a multiple of 32
    assert _qkv(L, C=544) == SWIN_EUNSUPPORTED                                  # above 512
    assert _qkv(L, C=0) == SWIN_EINVAL
    assert _qkv(L, T=-1) == SWIN_EINVAL
    assert _qkv(L, dtype=2) == SWIN_EINVAL
    assert _qkv(L, x=None) == SWIN_EINVAL
    assert _qkv(L, v=None) == SWIN_EINVAL
    assert _qkv(L, q=ctypes.c_void_p(0x40000008)) == SWIN_EINVAL                # misaligned
    assert _qkv(L, b=ctypes.c_void_p(0x70000004)) == SWIN_EINVAL                # misaligned bias
    assert _qkv(L, q=ctypes.c_void_p(0x10000 + 128)) == SWIN_EINVAL             # q overlaps x
    assert _qkv(L, k=ctypes.c_void_p(0x40000000 + 64)) == SWIN_EINVAL           # k overlaps q
    assert _qkv(L, x=None, w=None, q=None, k=None, v=None, T=0) == SWIN_OK      # empty: no-op
    assert _pnorm(L, C=48) == SWIN_EUNSUPPORTED
    assert _pnorm(L, eps=-1.0) == SWIN_EINVAL
    assert _pnorm(L, eps=float("nan")) == SWIN_EINVAL
    assert _pnorm(L, gamma=None) == SWIN_EINVAL
    assert _pnorm(L, y=ctypes.c_void_p(0x10000 + 64)) == SWIN_EINVAL            # y overlaps o
    assert _pnorm(L, y=ctypes.c_void_p(0x40000000 + 32)) == SWIN_EINVAL         # partial overlap of resid
    assert _pnorm(L, y=ctypes.c_void_p(0x50000000 - 64)) == SWIN_EINVAL         # y overlaps gamma
    assert _pnorm(L, beta=ctypes.c_void_p(0x50001008)) == SWIN_EINVAL           # misaligned
    assert _pnorm(L, o=None, w=None, resid=None, gamma=None, beta=None, y=None, T=0) == SWIN_OK


def _fused(L, d=None, x=ctypes.c_void_p(0x10000), w=ctypes.c_void_p(0x30000000), b=None,
           out=ctypes.c_void_p(0x40000000), tau=FAKE, table=FAKE, **kw):
    desc = d if d is not None else _desc(**{**dict(B=1, H=32, W=32, C=96, heads=3, M=16, shift=8), **kw})
    return L.swin_qkv_window_attn_fwd(ctypes.byref(desc), x, w, b, out, tau, table, None)


def test_fused_input_layer_rejects(L):
    """Host validation of the fused input layer + attention: nothing is launched."""
    assert _fused(L, dtype=0) == SWIN_EUNSUPPORTED                              # fp32
    assert _fused(L, M=8, H=16, W=16, shift=4) == SWIN_EUNSUPPORTED             # M <= 8
    assert _fused(L, M=24, H=48, W=48, shift=12) == SWIN_EUNSUPPORTED           # M > 16
    assert _fused(L, pos=2) == SWIN_EUNSUPPORTED                                # rotary positions
    assert _fused(L, C=512, heads=16) == SWIN_EUNSUPPORTED                      # C > 192
    assert _fused(L, layout=1) == SWIN_EUNSUPPORTED                             # windows layout
    assert _fused(L, shift=16) == SWIN_EINVAL                                   # bad descriptor
    assert _fused(L, x=None) == SWIN_EINVAL
    assert _fused(L, w=ctypes.c_void_p(0x30000008)) == SWIN_EINVAL              # misaligned
    assert _fused(L, b=ctypes.c_void_p(0x50000002)) == SWIN_EINVAL              # misaligned bias
    assert _fused(L, out=ctypes.c_void_p(0x10000 + 4096)) == SWIN_EINVAL        # out overlaps x
    assert _fused(L, tau=None) == SWIN_EINVAL                                   # COSINE needs tau
    assert _fused(L, table=None) == SWIN_EINVAL                                 # TABLE needs a table
    assert _fused(L, B=0, x=None, w=None, out=None) == SWIN_OK                  # empty: no-op


def test_dwconv_rejects(L):
    """Host validation of the convolution branch: nothing is launched."""
    out = ctypes.c_void_p(0x60000000)
    w = ctypes.c_void_p(0x30000000)
    assert L.swin_dwconv_add(FAKE, w, None, out, 1, 8, 8, 20, 1, None) == SWIN_EUNSUPPORTED   # 20 % 8
    assert L.swin_dwconv_add(FAKE, w, None, out, 1, 0, 8, 32, 1, None) == SWIN_EINVAL
    assert L.swin_dwconv_add(FAKE, w, None, out, 1, 8, 8, 32, 5, None) == SWIN_EINVAL
    assert L.swin_dwconv_add(None, w, None, out, 1, 8, 8, 32, 1, None) == SWIN_EINVAL
    assert L.swin_dwconv_add(FAKE, w, None, ctypes.c_void_p(0x60000008), 1, 8, 8, 32, 1, None) == SWIN_EINVAL
    assert L.swin_dwconv_add(FAKE, w, None, ctypes.c_void_p(0x10000 + 64), 1, 8, 8, 32, 1, None) == SWIN_EINVAL
    assert L.swin_dwconv_add(FAKE, ctypes.c_void_p(0x30000002), None, out, 1, 8, 8, 32, 1, None) == SWIN_EINVAL
    assert L.swin_dwconv_add(None, None, None, None, 0, 8, 8, 32, 1, None) == SWIN_OK           # empty batch


def test_window_linear_rejects(L):
    """Host validation of the in-window linear mapping: nothing is launched."""
    out = ctypes.c_void_p(0x60000000)
    A = ctypes.c_void_p(0x30000000)
    f = lambda d, v=FAKE, A=A, b=None, o=out: L.swin_window_linear(ctypes.byref(d) if d else None, v, A, b, o, None)
    assert f(None) == SWIN_EINVAL
    assert f(_desc(H=12)) == SWIN_EUNSUPPORTED                      # H % M
    assert f(_desc(C=96, heads=2)) == SWIN_EUNSUPPORTED             # head dim 48
    assert f(_desc(), v=None) == SWIN_EINVAL
    assert f(_desc(), A=ctypes.c_void_p(0x30000008)) == SWIN_EINVAL # misaligned
    assert f(_desc(), o=ctypes.c_void_p(0x10000 + 64)) == SWIN_EINVAL   # out overlaps v
    assert f(_desc(), o=ctypes.c_void_p(0x30000000 - 64)) == SWIN_EINVAL # out overlaps A
    assert f(_desc(B=0), v=None, A=None, o=None) == SWIN_OK         # empty batch


def test_backward_rejects(L):
    d = _desc()
    assert _bwd(L, None) == SWIN_EINVAL
    assert _bwd(L, _desc(H=12)) == SWIN_EUNSUPPORTED
    assert _bwd(L, _desc(H=56, W=56, M=56, shift=0)) == SWIN_EUNSUPPORTED       # table and statistics past LDS
    assert _bwd(L, _desc(H=72, W=72, M=72, shift=0)) == SWIN_EUNSUPPORTED       # M > 64
    assert _bwd(L, d, dout=None) == SWIN_EINVAL
    assert _bwd(L, d, out=None) == SWIN_EINVAL
    assert _bwd(L, d, dk=None) == SWIN_EINVAL
    assert _bwd(L, d, tau=None) == SWIN_EINVAL                                  # COSINE needs tau
    assert _bwd(L, d, table=None) == SWIN_EINVAL                                # TABLE needs the table
    assert _bwd(L, d, dq=ctypes.c_void_p(0x20000008)) == SWIN_EINVAL            # misaligned
    assert _bwd(L, d, dq=ctypes.c_void_p(0x10000 + 64)) == SWIN_EINVAL          # dq overlaps q
    assert _bwd(L, d, dv=ctypes.c_void_p(0x20000000 + 64)) == SWIN_EINVAL       # dv overlaps dq
    assert _bwd(L, d, dtable=FAKE) == SWIN_EINVAL                               # dtable overlaps table
    # an empty batch with no summed gradients enqueues nothing
    assert _bwd(L, _desc(B=0), q=None, k=None, v=None, out=None, dout=None, dq=None, dk=None,
                dv=None) == SWIN_OK


def test_cpb_backward_rejects(L):
    X = L.swin_cpb_table_bwd
    A, B_, C_, D_ = (ctypes.c_void_p(0x20000000 + i * 0x1000000) for i in range(4))
    assert X(8, 8, 3, 512, FAKE, None, FAKE, FAKE, FAKE, 4, A, B_, C_, D_, None) == SWIN_EINVAL     # mode
    assert X(8, 8, 3, 512, FAKE, None, FAKE, None, FAKE, 2, A, B_, C_, D_, None) == SWIN_EINVAL     # no table
    assert X(8, 1, 3, 512, FAKE, None, FAKE, FAKE, FAKE, 1, A, B_, C_, D_, None) == SWIN_EINVAL     # norm_M
    assert X(8, 8, 3, 512, FAKE, None, FAKE, FAKE, None, 0, A, B_, C_, D_, None) == SWIN_EINVAL     # dtable
    assert X(8, 8, 3, 512, FAKE, None, FAKE, FAKE, FAKE, 0, None, B_, C_, D_, None) == SWIN_EINVAL  # dw1
    assert X(8, 8, 3, 512, FAKE, None, FAKE, FAKE, FAKE, 0, FAKE, B_, C_, D_, None) == SWIN_EINVAL  # dw1 = w1
    assert X(8, 8, 3, 512, FAKE, None, FAKE, FAKE, FAKE, 0, A, A, C_, D_, None) == SWIN_EINVAL      # db1 = dw1


def test_kernel_query_names_the_dispatch(L):
    """Which kernel each workload shape reaches: fp32 -> vector ALUs; bf16
    windows of at most 256 key slots (M rounded up to 8 per key row) without
    rotary positions -> the register-resident kernel; other windows up to
    M = 32 (larger, or rotary) -> the large-window kernel; beyond -> the
    block-staged MFMA kernel."""
    from vision_transformer_windowed_partition_amd import synth
    want = ["attn_valu_kernel", "attn_small_kernel", "attn_small_kernel", "attn_large_kernel",
            "attn_large_kernel"]
    for wl, name in zip(synth.WORKLOADS, want):
        d = binding.make_desc(B=wl.B, H=wl.H, W=wl.W, C=wl.C, heads=wl.heads, M=wl.M, shift=wl.shift,
                              partition=wl.partition, sim=wl.sim, pos=wl.pos,
                              dtype=binding.DTYPE_BY_NAME[wl.dtype])
        assert binding.swin_window_attn_kernel(d) == name, wl.name
    assert binding.swin_window_attn_kernel(_desc(M=12, H=24, W=24, dtype=1)) == "attn_small_kernel"  # 192 slots
    assert binding.swin_window_attn_kernel(_desc(M=17, H=34, W=34, dtype=1, shift=0)) == "attn_large_kernel"
    assert binding.swin_window_attn_kernel(_desc(M=8, dtype=1, pos=2)) == "attn_large_kernel"
    assert binding.swin_window_attn_kernel(_desc(M=48, H=48, W=48, dtype=1, shift=0)) == "attn_mfma_kernel"
    assert L.swin_window_attn_kernel(ctypes.byref(_desc(shift=8))) is None
    assert "shift" in binding.swin_last_error()
    assert L.swin_window_attn_kernel(None) is None


def test_backward_kernel_query_names_the_dispatch(L):
    """The backward's dispatch: bf16 windows of at most 256 key slots without
    rotary positions -> the small matrix-core kernel; other bf16 windows up to
    M = 32 whose rows fit in LDS (cosine with rotary positions also keeps the
    remainders of its rotated rows, which fit up to M = 24) -> the large
    matrix-core kernel; fp32 and the rest -> the vector-ALU kernel (M <= 64
    where its statistics and table fit LDS); d != 32 and the rest are
    rejected."""
    from vision_transformer_windowed_partition_amd import synth
    want = ["attn_bwd_kernel", "attn_bwd_small_kernel", "attn_bwd_small_kernel", "attn_bwd_large_kernel",
            "attn_bwd_large_kernel"]
    for wl, name in zip(synth.WORKLOADS, want):
        d = binding.make_desc(B=wl.B, H=wl.H, W=wl.W, C=wl.C, heads=wl.heads, M=wl.M, shift=wl.shift,
                              partition=wl.partition, sim=wl.sim, pos=wl.pos,
                              dtype=binding.DTYPE_BY_NAME[wl.dtype])
        assert binding.swin_window_attn_bwd_kernel(d) == name, wl.name
    assert binding.swin_window_attn_bwd_kernel(_desc(M=12, H=24, W=24)) == "attn_bwd_small_kernel"
    assert binding.swin_window_attn_bwd_kernel(_desc(M=8, pos=2, sim=1)) == "attn_bwd_large_kernel"
    assert binding.swin_window_attn_bwd_kernel(_desc(M=8, pos=2, sim=0)) == "attn_bwd_large_kernel"
    assert binding.swin_window_attn_bwd_kernel(_desc(M=24, H=48, W=48, shift=12, pos=2, sim=0)) == \
        "attn_bwd_large_kernel"
    assert binding.swin_window_attn_bwd_kernel(_desc(M=32, H=32, W=32, shift=16, pos=2, sim=0)) == "attn_bwd_kernel"
    assert binding.swin_window_attn_bwd_kernel(_desc(M=8, dtype=0)) == "attn_bwd_kernel"
    assert binding.swin_window_attn_bwd_kernel(_desc(M=48, H=48, W=48, shift=0)) == "attn_bwd_kernel"
    assert binding.swin_window_attn_bwd_kernel(_desc(M=64, H=64, W=64, shift=0, pos=0)) == "attn_bwd_kernel"
    assert L.swin_window_attn_bwd_kernel(ctypes.byref(_desc(M=56, H=56, W=56, shift=0))) is None
    assert "M=56" in binding.swin_last_error()
    assert L.swin_window_attn_bwd_kernel(ctypes.byref(_desc(C=128))) is None
    assert L.swin_window_attn_bwd_kernel(None) is None


def test_attn_empty_batch_is_a_no_op(L):
    assert _attn(L, _desc(B=0), q=None, k=None, v=None, out=None) == SWIN_OK


def test_partition_rejects(L):
    P = L.swin_window_partition
    assert P(FAKE, ctypes.c_void_p(0x900000), 1, 12, 12, 8, 5, 0, 0, 1, None) == SWIN_EUNSUPPORTED
    assert P(FAKE, ctypes.c_void_p(0x900000), 1, 16, 16, 8, 8, 8, 0, 1, None) == SWIN_EINVAL
    assert P(FAKE, ctypes.c_void_p(0x900000), 1, 16, 16, 8, 8, 2, 1, 1, None) == SWIN_EINVAL
    assert P(FAKE, FAKE, 1, 16, 16, 8, 8, 0, 0, 1, None) == SWIN_EINVAL            # x == xw
    assert P(None, ctypes.c_void_p(0x900000), 1, 16, 16, 8, 8, 0, 0, 1, None) == SWIN_EINVAL
    assert P(FAKE, ctypes.c_void_p(0x900000), 1, 16, 16, 8, 8, 0, 0, 9, None) == SWIN_EINVAL
    assert P(None, None, 0, 16, 16, 8, 8, 0, 0, 1, None) == SWIN_OK               # empty
    R = L.swin_window_reverse
    assert R(FAKE, ctypes.c_void_p(0x900000), 1, 16, 16, 8, 8, 9, 0, 1, None) == SWIN_EINVAL


def test_cpb_rejects(L):
    C = L.swin_cpb_table
    T = ctypes.c_void_p(0x900000)
    assert C(8, 3, 512, FAKE, None, FAKE, None, 4, T, None) == SWIN_EINVAL        # unknown mode flag
    assert C(8, 3, 512, FAKE, None, FAKE, None, -1, T, None) == SWIN_EINVAL
    assert C(1, 3, 512, FAKE, None, FAKE, None, 1, T, None) == SWIN_EINVAL        # code form needs M >= 2
    X = L.swin_cpb_table_ex
    assert X(8, 1, 3, 512, FAKE, None, FAKE, None, 3, T, None) == SWIN_EINVAL     # normalising window < 2
    assert X(8, 5000, 3, 512, FAKE, None, FAKE, None, 1, T, None) == SWIN_EINVAL
    assert X(8, 3, 0, 512, FAKE, None, FAKE, None, 1, T, None) == SWIN_EINVAL
    assert X(8, 12, 3, 512, FAKE, None, FAKE, None, 3, FAKE, None) == SWIN_EINVAL  # table over w1
    assert C(0, 3, 512, FAKE, None, FAKE, None, 0, T, None) == SWIN_EINVAL
    assert C(8, 0, 512, FAKE, None, FAKE, None, 0, T, None) == SWIN_EINVAL
    assert C(8, 3, 0, FAKE, None, FAKE, None, 0, T, None) == SWIN_EINVAL
    assert C(8, 3, 512, None, None, FAKE, None, 0, T, None) == SWIN_EINVAL
    assert C(8, 3, 512, FAKE, None, FAKE, None, 0, None, None) == SWIN_EINVAL
    assert C(8, 3, 512, FAKE, None, FAKE, None, 0, FAKE, None) == SWIN_EINVAL      # table over w1
    R = L.swin_cpb_table_resize
    assert R(0, 8, 3, FAKE, T, None) == SWIN_EINVAL                                # window sizes
    assert R(8, 65, 3, FAKE, T, None) == SWIN_EINVAL
    assert R(8, 12, 0, FAKE, T, None) == SWIN_EINVAL                               # heads
    assert R(8, 12, 3, None, T, None) == SWIN_EINVAL
    assert R(8, 12, 3, FAKE, None, None) == SWIN_EINVAL
    assert R(8, 12, 3, FAKE, FAKE, None) == SWIN_EINVAL                            # dst over src


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        binding.lib()


def test_binding_checks_sizes_before_the_call():
    """The Python binding rejects tensors whose sizes disagree with the
    descriptor before anything reaches the library (CPU tensors: the check runs
    before the device-pointer check, so a size error is what raises)."""
    import torch
    bf = torch.bfloat16
    q = torch.zeros((2, 16, 16, 64), dtype=bf)
    tau, table = torch.ones(2), torch.zeros((225, 2))
    base = dict(heads=2, M=8, shift=4, sim="cosine", pos="table")
    with pytest.raises(ValueError, match="tau must hold 2"):
        binding.swin_window_attn_fwd(q, q, q, tau=torch.ones(1), table=table, **base)
    with pytest.raises(ValueError, match="table must hold 450"):
        binding.swin_window_attn_fwd(q, q, q, tau=tau, table=torch.zeros((224, 2)), **base)
    with pytest.raises(ValueError, match="rope_freqs must hold 32"):
        binding.swin_window_attn_fwd(q, q, q, heads=2, M=8, sim="dot", pos="rope2d", rope_freqs=torch.zeros(31))
    with pytest.raises(ValueError, match="out must be"):
        binding.swin_window_attn_fwd(q, q, q, tau=tau, table=table, out=torch.zeros((2, 16, 16, 64)), **base)
    with pytest.raises(ValueError, match="out must be"):
        binding.swin_window_attn_fwd_lse(q, q, q, tau=tau, table=table, out=torch.zeros((2, 16, 16, 32), dtype=bf),
                                         **base)
    # pre-partitioned windows: q's element count must match the grid it is paired with
    qw = torch.zeros((8, 64, 64), dtype=bf)
    with pytest.raises(ValueError, match="descriptor's grid"):
        binding.swin_window_attn_fwd(qw, qw, qw, tau=tau, table=table, layout="windows", grid=(2, 16, 24), **base)
    with pytest.raises(ValueError, match="tau must hold 2"):
        binding.swin_window_attn_bwd(q, q, q, q, q, tau=torch.ones(3), table=table, **base)
    with pytest.raises(ValueError, match="table must hold 450"):
        binding.swin_window_attn_bwd(q, q, q, q, q, tau=tau, table=torch.zeros(10), **base)
    # video windows: the table covers (2Mt-1)(2M-1)^2 offsets
    qv = torch.zeros((1, 4, 16, 16, 64), dtype=bf)
    with pytest.raises(ValueError, match="table must hold 1350"):
        binding.swin_window_attn3d_fwd(qv, qv, qv, heads=2, Mt=2, M=8, sim="cosine", pos="table", tau=tau,
                                       table=torch.zeros((225, 2)))
    # correctly sized CPU tensors get past the size checks and stop at the device check
    with pytest.raises(ValueError, match="GPU"):
        binding.swin_window_attn_fwd(q, q, q, tau=tau, table=table, **base)
