"""Build libqpack.so (HIP, gfx950) in-tree.

Every translation unit is compiled with hipcc for gfx950 only, in parallel,
into `_build/`, then linked into `weight_only_quantized_qgemv_amd/libqpack.so`.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqpack.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

BITS = (2, 3, 4, 6, 8)
# (source, object name, defines): kernels with many template instantiations are
# compiled once per bit width (and MoE form) so the work spreads over cores.
UNITS = ([("api.cpp", "api", {}), ("quantize.hip", "quantize", {}), ("moe.hip", "moe", {}),
          ("qgemm.hip", "qgemm", {}),
          ("dequantize.hip", "dequantize", {}), ("mx_gemv.hip", "mx_gemv", {}),
          ("moe_ffn.hip", "moe_ffn", {}), ("int8_tensor.hip", "int8_tensor", {}),
          ("qgemv_t.hip", "qgemv_t", {})]
         + [("qgemv.hip", f"qgemv_b{b}", {"QP_BITS": b}) for b in BITS]
         + [("moe_compute.hip", f"moe_b{b}_n{n}", {"QP_BITS": b, "QP_NMAT": n})
            for b in BITS for n in (1, 2)])

# Packed-fp32 VALU forms are kept out of generated code; contraction follows
# each kernel's own pragmas (the quantizer turns it off).
CFLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


def _compile(unit) -> str:
    src, name, defines = unit
    obj = os.path.join(BUILD, name + ".o")
    cmd = [HIPCC, *CFLAGS, *[f"-D{k}={v}" for k, v in defines.items()], "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, sorted(UNITS, key=lambda u: u[0] != "moe_compute.hip")))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
