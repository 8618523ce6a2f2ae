"""Host-sanitizer tier (CPU): the library's host code (argument validation,
the split planner, status strings, the binding's checks) runs under
AddressSanitizer and UBSan.

Builds the host-sanitized variant of libattn.so (``build(sanitize=True)``,
GPU code unchanged) when it is missing or older than a source, then runs the
C-ABI and split-planner CPU tests against it in a subprocess that preloads
the sanitizer runtime.  Any sanitizer report aborts that subprocess.
"""

import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
build = pytest.importorskip("io_aware_softmax_amd.build")


def _stale(lib: Path) -> bool:
    if not lib.exists():
        return True
    t = lib.stat().st_mtime
    srcs = list((ROOT / "io_aware_softmax_amd" / "csrc").iterdir()) + [ROOT / "include" / "attn.h"]
    return any(p.stat().st_mtime > t for p in srcs)


@pytest.mark.slow
def test_abi_and_planner_under_host_sanitizers():
    lib = build.SANITIZE_LIB
    if _stale(lib):
        build.build(sanitize=True)
    syms = subprocess.run(["nm", "-D", str(lib)], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "host code is not instrumented"
    env = dict(os.environ, LD_PRELOAD=str(build.asan_runtime()), IO_AWARE_SOFTMAX_LIB=str(lib),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi.py", "tests/test_split_plan.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = "\n".join((r.stdout + r.stderr).splitlines()[-30:])
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    # the sanitized library is what the subprocess loaded
    assert str(lib) in subprocess.run(
        [sys.executable, "-c", "from io_aware_softmax_amd import binding; print(binding.library_loaded_path())"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=120).stdout
