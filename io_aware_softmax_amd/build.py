"""Build libattn.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m io_aware_softmax_amd.build`` or ``build()`` from Python.
Objects go to ``_build/`` at the repository root; the library is written to
``io_aware_softmax_amd/libattn.so`` (atomically replaced).
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


def build(verbose: bool = False) -> Path:
    out = ROOT / "_build"
    out.mkdir(exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = out / (Path(src).stem + ".o")
        jobs.append((obj, [HIPCC, *FLAGS, "-c", str(PKG / "csrc" / src), "-o", str(obj)]))
    with ThreadPoolExecutor(min(len(jobs), os.cpu_count() or 1)) as ex:
        msgs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for m in msgs:
            if m.strip():
                print(m, file=sys.stderr)
    tmp = LIB.with_suffix(".so.tmp")
    # --no-undefined: a kernel whose host stub was not emitted must fail the
    # build, not the first launch.
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-Wl,--no-undefined", "-o", str(tmp),
          *[str(o) for o, _ in jobs]])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
