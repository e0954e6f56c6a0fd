"""The host-side tests under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the oracle (oracle.build(sanitize=True)) and the library's host C ABI
layer (build.build_sanitized: abi.cpp under -fsanitize=address,undefined,
the kernels as usual) and runs the oracle pins and the host ABI tests against
those builds in a child process that preloads clang's shared ASan runtime.
Any sanitizer finding aborts the child (UBSan does not recover), so the
child must exit cleanly.  Leak detection is off: the interpreter and torch
keep allocations alive until exit by design.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

CLANG = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")


def _asan_runtime():
    if not os.path.exists(CLANG):
        return None
    out = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if out.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


CHECK_LOADED = (
    "import sys; sys.path.insert(0, {root!r})\n"
    "import oracle, fp8_quantized_linear_amd as mxl\n"
    "oracle.lib(); maps = open('/proc/self/maps').read()\n"
    "assert 'libmxoracle_san.so' in maps and 'libmxlinear_san.so' in maps, 'sanitized builds not loaded'\n"
    "print('sanitized builds loaded')\n"
)


def test_host_tests_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("clang's shared ASan runtime is not available")
    import oracle
    import fp8_quantized_linear_amd.build as b
    oracle.build(force=True, sanitize=True)
    b.build_sanitized()
    env = dict(os.environ)
    env.update({"MXL_SANITIZED": "1", "LD_PRELOAD": rt,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    chk = subprocess.run([sys.executable, "-c", CHECK_LOADED.format(root=ROOT)], env=env, cwd=ROOT,
                         capture_output=True, text=True, timeout=300)
    assert chk.returncode == 0, chk.stdout[-2000:] + chk.stderr[-4000:]
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                          "tests/test_abi_host.py", "tests/test_oracle_pins.py"],
                         env=env, cwd=ROOT, capture_output=True, text=True, timeout=1200)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-6000:]
