"""Helpers shared by the GPU test modules: upload seeded inputs, run the HIP
path through the C ABI, compare with the float64 oracle."""

import sys

import numpy as np
import pytest

from io_aware_softmax_amd import inputs

# Max abs error bounds on O for each storage type; LSE bound is
# 1e-4 * max(1, |LSE_ref|) for all types.
O_TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 2e-2}
LSE_REL = 1e-4


def torch_mod():
    import torch
    return torch


def gpu_available():
    try:
        torch = torch_mod()
        return torch.cuda.is_available()
    except Exception:
        return False


def require_gpu():
    if not gpu_available():
        pytest.skip("needs a GPU")


def to_device(bits, dtype):
    torch = torch_mod()
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        t = t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)
    return t.to("cuda", non_blocking=False)


def to_host_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def round_ref(x, dtype):
    """The float64 reference rounded once, to nearest-even, to the storage
    type of the output (no detour through float32 for bf16)."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        return x.astype(np.float16).astype(np.float64)
    m, e = np.frexp(x)  # x = m 2^e, 0.5 <= |m| < 1: bf16 keeps 8 significant bits
    return np.ldexp(np.rint(m * 256.0), e - 8)


def compare(name, dtype, O_gpu, L_gpu, O_ref, L_ref, o_tol=None):
    """Max-abs comparison with the documented tolerances; returns the errors.

    Also reports max|O - round(O_ref)|, the distance to the reference
    rounded to the output's storage type: the part of the error that the
    kernel adds beyond the output's own rounding (for bf16 half an ulp is
    0.0078 for |O| in [2, 4) and 0.0156 in [4, 8)).  The bound applies to
    max|O - O_ref|."""
    o_tol = O_TOL[dtype] if o_tol is None else o_tol
    assert np.all(np.isfinite(O_gpu)), f"{name}: non-finite output"
    assert np.all(np.isfinite(L_gpu)), f"{name}: non-finite lse"
    eo = float(np.max(np.abs(O_gpu - O_ref))) if O_ref.size else 0.0
    er = float(np.max(np.abs(O_gpu - round_ref(O_ref, dtype)))) if O_ref.size else 0.0
    el = float(np.max(np.abs(L_gpu - L_ref) / np.maximum(1.0, np.abs(L_ref)))) if L_ref.size else 0.0
    say(f"  {name}: max|dO|={eo:.3e} (tol {o_tol:.0e})  max rel|dLSE|={el:.3e} (tol {LSE_REL:.0e})"
        f"  max|O-rnd(O_ref)|={er:.3e}")
    assert eo <= o_tol, f"{name}: O error {eo} > {o_tol}"
    assert el <= LSE_REL, f"{name}: LSE error {el} > {LSE_REL}"
    return eo, el
