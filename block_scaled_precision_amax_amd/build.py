"""Builds libfp8q.so (the HIP kernels and the C ABI) for gfx950 with hipcc,
and libfp8q_stream.so, the streaming-bandwidth reference the benchmark sets
the quantizers against (not part of the library's ABI).

Each csrc/*.hip is compiled to an object in parallel, then linked into the
package directory, where the Python binding loads it.  Flags:
  -ffp-contract=off                       every fused multiply-add is written out
  -fhip-fp32-correctly-rounded-divide-sqrt  '/' is the IEEE fp32 division
  -target-feature -packed-fp32-ops        no packed fp32 math is generated
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
LIB = os.path.join(HERE, "libfp8q.so")
STREAM_LIB = os.path.join(HERE, "libfp8q_stream.so")
ARCH = os.environ.get("FP8Q_ARCH", "gfx950")

SOURCES = ["fp8q_api.hip", "fp8q_quant.hip", "fp8q_gemm.hip"]
STREAM_SOURCES = ["fp8q_stream.hip"]

COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(extra: list[str] | None = None, save_temps: bool = False) -> str:
    """Compile every HIP source and link libfp8q.so and libfp8q_stream.so.
    Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    if save_temps:
        extra += ["-save-temps=obj"]
    srcs = SOURCES + STREAM_SOURCES
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], STREAM_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
