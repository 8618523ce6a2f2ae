"""Build libattn.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m io_aware_softmax_amd.build`` or ``build()`` from Python.
Objects go to ``_build/`` at the repository root; the library is written to
``io_aware_softmax_amd/libattn.so`` (atomically replaced).
``python -m io_aware_softmax_amd.build --sanitize`` builds the host-sanitized
variant ``_build/sanitize/libattn_sanitize.so`` for the CPU tests instead.
The measurement probe ``probes/gfx950_probe.hip`` (not part of the library)
is built next to the objects as ``_build/gfx950_probe``.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SOURCES = ["api.hip", "device_info.hip", "prefill_mfma.hip", "prefill_pp.hip", "prefill_f32.hip", "decode.hip",
           "backward.hip", "prefill_ex.hip"]
LIB = PKG / "libattn.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in generated code.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{ROOT / 'include'}", f"-I{PKG / 'csrc'}",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


# Host-side sanitizers for the CPU test tier (argument validation, the
# split planner, the status strings): AddressSanitizer and UBSan on the
# host code only; the GPU code is built as usual.  Each -fsanitize= follows
# -Xarch_host so that it never reaches the device compilation.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZE_LIB = ROOT / "_build" / "sanitize" / "libattn_sanitize.so"


def asan_runtime() -> Path:
    """The shared AddressSanitizer runtime of the ROCm LLVM toolchain (to be
    preloaded into a process that loads the sanitized library)."""
    hits = sorted(Path("/opt/rocm/llvm/lib/clang").glob("*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm/lib/clang")
    return hits[-1]


def build(verbose: bool = False, sanitize: bool = False) -> Path:
    """Compile every source and link the library.  sanitize=True builds the
    host-sanitized variant SANITIZE_LIB instead (CPU tests only)."""
    out = ROOT / "_build" / ("sanitize" if sanitize else "")
    out.mkdir(parents=True, exist_ok=True)
    flags = FLAGS + (SANITIZE_FLAGS if sanitize else [])
    jobs = []
    for src in SOURCES:
        obj = out / (Path(src).stem + ".o")
        jobs.append((obj, [HIPCC, *flags, "-c", str(PKG / "csrc" / src), "-o", str(obj)]))
    with ThreadPoolExecutor(min(len(jobs), os.cpu_count() or 1)) as ex:
        msgs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for m in msgs:
            if m.strip():
                print(m, file=sys.stderr)
    lib = SANITIZE_LIB if sanitize else LIB
    tmp = lib.with_suffix(".so.tmp")
    # --no-undefined: a kernel whose host stub was not emitted must fail the
    # build, not the first launch.  The sanitized variant links the shared
    # sanitizer runtime, which the test process preloads.
    link = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"] \
        if sanitize else []
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-Wl,--no-undefined", *link, "-o", str(tmp),
          *[str(o) for o, _ in jobs]])
    os.replace(tmp, lib)
    if not sanitize:
        build_probe()
    return lib


PROBE = ROOT / "_build" / "gfx950_probe"


def build_probe() -> Path:
    """The stand-alone issue-cost / LDS-throughput probe executable."""
    PROBE.parent.mkdir(parents=True, exist_ok=True)
    tmp = PROBE.with_name(PROBE.name + ".tmp")
    _run([HIPCC, *FLAGS, "-o", str(tmp), str(PKG / "probes" / "gfx950_probe.hip")])
    os.replace(tmp, PROBE)
    return PROBE


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
