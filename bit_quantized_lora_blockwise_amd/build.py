"""Build libqlora.so (the gfx950 HIP kernels and the C ABI) and libqlprobe.so
(the benchmark's measurement helpers) in-tree with hipcc.

    python -m bit_quantized_lora_blockwise_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqlora.so")
PROBE_SRC = os.path.join(PKG, "probe", "probe.hip")
PROBE_LIB = os.path.join(PKG, "libqlprobe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# No fast-math: the encoder relies on correctly rounded fp32 division and the
# dequantiser on unfused fp32 products.  Packed-fp32 instructions are disabled.
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast-honor-pragmas", "-Wall", "-Wno-unused-result",
    f"-I{os.path.join(os.path.dirname(PKG), 'include')}",
]


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, tag: str = "") -> str:
    obj = os.path.join(BUILD, tag + os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        probe = ex.submit(_compile, PROBE_SRC, "probe_")
        objs = list(ex.map(_compile, srcs))
        probe_obj = probe.result()
    _link(objs, LIB)
    _link([probe_obj], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
