"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only; no GPU is touched).

Every source of the library is compiled with the sanitizers on its host side
only (device code is unchanged) into a separate library under _build/. The
host ABI tests (tests/test_abi_host.py: export list, argument validation of
every call, workspace sizes, the no-fallback behaviour) then run in a child
process that loads that library with the sanitizer runtime preloaded. Any
out-of-bounds access, use after free, signed overflow or other undefined
behaviour in the validation, layout and launch-preparation code aborts the
child, and the test fails with its report.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(ROOT, "_build", "host_sanitized")
SAN_LIB = os.path.join(SAN_DIR, "libsga_host_sanitized.so")


def _runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(_runtime() is None, reason="clang's sanitizer runtime is not installed")
def test_host_abi_under_sanitizers():
    sys.path.insert(0, ROOT)
    from sparse_attention_global_amd.build import build

    # host side only: the device code objects are built exactly as usual
    san = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    build(lib=SAN_LIB, obj_dir=os.path.join(SAN_DIR, "obj"), extra_flags=san,
          link_flags=["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-shared-libsan"])
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": _runtime(),
        "SGA_LIBRARY": SAN_LIB,
        # the interpreter and torch are not instrumented; their allocations at
        # exit are not this library's leaks
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HIP_VISIBLE_DEVICES": "",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = r.stdout[-6000:] + "\n" + r.stderr[-6000:]
    print(report)
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
