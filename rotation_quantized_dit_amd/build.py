"""Build the gfx950 HIP library ``libconvrot.so`` in place with hipcc.

    python -m rotation_quantized_dit_amd.build

Every source is compiled for gfx950 only, with IEEE fp32 semantics (correctly
rounded division, no contraction of multiply-add, denormals kept) and with the
packed-fp32 VALU instructions disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libconvrot.so")
SOURCES = ["convrot_api.cpp", "rotate_quant.hip", "gemm_i8.hip", "weight_ops.hip", "attention.hip", "mx_quant.hip",
           "gemm_mx.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I" + os.path.join(ROOT, "include"),
]


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))


def build() -> str:
    """Compile every source for gfx950 and link libconvrot.so (always rebuilds)."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(len(SOURCES)) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
