"""Builds the HIP library libvcattn.so for gfx950 with hipcc (cross-compiles
without a GPU).  Usage: python -m bit_attention_video_smooth_amd.build"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libvcattn.so")
SOURCES = ["vc_abi.hip", "vc_host.hip", "vc_prepare.hip", "vc_sage_prepare.hip", "vc_kmeans.hip", "vc_attn_fp8.hip",
           "vc_attn_sage.hip", "vc_attn_fp4.hip", "vc_attn_bf16.hip", "vc_debug.hip"]
ARCH = os.environ.get("VC_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            # packed fp32 instructions stay off (the host pass ignores the flag)
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-disable-promote-alloca-to-lds",
            "-Wno-unused-result"]


# NaN inputs are outside the library's contract; without NaN semantics the
# compiler drops the quieting moves it otherwise puts around every max.
EXTRA = {src: ["-fno-honor-nans"] for src in
         ("vc_attn_fp8.hip", "vc_attn_sage.hip", "vc_attn_fp4.hip", "vc_attn_bf16.hip", "vc_kmeans.hip")}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [hipcc(), *flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
