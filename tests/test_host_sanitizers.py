"""The host-only ABI checks (tests/test_abi_host.py) run again against a build
of the library whose host code carries AddressSanitizer and
UndefinedBehaviorSanitizer (bit_quantized_lora_blockwise_amd/build_hostsan.py),
in a child process that preloads clang's ASan runtime.  Every call there fails
validation before any kernel is launched, so no GPU is needed; a heap overflow,
use after free or undefined behaviour on those host paths (argument checks,
workspace sizing with 64-bit products, the NF4 table bisection) aborts the run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_checks_under_asan_and_ubsan():
    if shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")) is None:
        pytest.skip("hipcc not available")
    sys.path.insert(0, ROOT)
    try:
        import bit_quantized_lora_blockwise_amd.build_hostsan as B
    except ImportError:
        pytest.skip("the host-sanitized builder is not present in this copy")
    rt = B.asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    lib = B.build()
    env = dict(os.environ)
    env.update({"QLORA_LIBRARY": lib, "LD_PRELOAD": rt,
                "ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
                "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_host.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out and " failed" not in out and " skipped" not in out, out[-2000:]
