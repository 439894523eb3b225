"""Build libgdr.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m gated_delta_rule_amd.build [-v]

Every source is compiled on each call (one hipcc process per file, in
parallel) and linked into gated_delta_rule_amd/libgdr.so in place, next to
libgdr_roofline.so (the roofline probes of include/gdr_roofline.h, which the
benchmark uses).  Cross-compiles without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdr.so")
ROOFLINE_LIB = os.path.join(PKG, "libgdr_roofline.so")

SOURCES = [
    "gdr_api.cpp",
    "kernels/decode.hip",
    "kernels/decode_layer.hip",
    "kernels/chunk_f32.hip",
    "kernels/chunk_bf16.hip",
    "kernels/conv_front.hip",
    "kernels/gated_rmsnorm.hip",
    "kernels/linear_bf16.hip",
    "kernels/attention.hip",
]
ROOFLINE_SOURCES = ["roofline/roofline.hip"]

ARCH = os.environ.get("GDR_OFFLOAD_ARCH", "gfx950")

# Packed fp32 instructions stay off: hipcc would otherwise form v_pk_*_f32
# from ordinary float code.  Matrix-core results go to ordinary VGPRs (not the
# accumulation registers), so the VALU work on them needs no copies.
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgdr)")


# The GEMM and the attention kernel keep their accumulators in the
# accumulation registers, so they are built without the VGPR form.
NO_VGPR_FORM = {"kernels/linear_bf16.hip", "kernels/attention.hip"}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
    lang = ["-x", "hip"]
    flags = FLAGS
    if src in NO_VGPR_FORM:
        flags = [f for f in FLAGS if f not in ("-mllvm", "-amdgpu-mfma-vgpr-form=1")]
    cmd = [_hipcc(), *lang, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(lib)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source and link libgdr.so and libgdr_roofline.so; returns
    the path of libgdr.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + ROOFLINE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], ROOFLINE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
