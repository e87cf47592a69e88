"""Build libswinattn.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libswinattn.so")
SOURCES = ["api.hip", "partition.hip", "cpb_table.hip", "attn_valu.hip", "attn_mfma.hip", "attn_small.hip", "attn_large.hip", "attn_bwd.hip", "attn_bwd_small.hip", "attn_bwd_large.hip", "proj.hip", "attn_fused.hip", "dwconv.hip", "window_linear.hip", "attn_video.hip", "attn_video_mfma.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", INCLUDE, "-I", CSRC,
    # no packed-fp32 VALU instructions (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs (no AGPR <-> VGPR copies around the softmax)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def _compile(src: str, obj: str) -> None:
    subprocess.run(["hipcc", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], check=True)


def build(jobs: int = 8) -> str:
    """Compile every HIP source and link libswinattn.so (always rebuilds)."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.run(["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
