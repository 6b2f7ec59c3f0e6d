"""Build a copy of libqlora.so whose host code (the C ABI's argument checks,
workspace sizing, the NF4 table construction, the launch wrappers) carries
AddressSanitizer and UndefinedBehaviorSanitizer instrumentation.  Device code
is compiled as usual; the instrumentation applies to the host pass only.

    python -m bit_quantized_lora_blockwise_amd.build_hostsan

The result, _build_hostsan/libqlora_hostsan.so, is loaded through the
QLORA_LIBRARY environment variable by a process that preloads clang's ASan
runtime (see tests/test_host_sanitizers.py); it is a checking build, not the
product.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import hashlib
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_build_hostsan")
LIB = os.path.join(OUT, "libqlora_hostsan.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-x", "hip",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=fast-honor-pragmas", f"-I{os.path.join(os.path.dirname(PKG), 'include')}",
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]


def asan_runtime() -> str | None:
    """clang's shared ASan runtime (it also carries the UBSan handlers)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".h")))


def _stamp() -> str:
    h = hashlib.sha256(" ".join(FLAGS).encode())
    for f in _sources():
        h.update(open(f, "rb").read())
    return h.hexdigest()


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.basename(src) + ".o")
    res = subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build() -> str:
    """Build (or reuse, when no source changed) the host-sanitized library."""
    stamp_file = os.path.join(OUT, "stamp")
    stamp = _stamp()
    if os.path.exists(LIB) and os.path.exists(stamp_file) and open(stamp_file).read() == stamp:
        return LIB
    os.makedirs(OUT, exist_ok=True)
    srcs = [s for s in _sources() if not s.endswith(".h")]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    res = subprocess.run([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    open(stamp_file, "w").write(stamp)
    return LIB


if __name__ == "__main__":
    print(build())
