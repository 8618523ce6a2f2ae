"""GPU test of attn_decode_fwd_noalloc (the decode entry point that
allocates nothing, its split partials in the library's fixed scratch)
through the C ABI: bit-identical to attn_decode_fwd with the same split
count, and within the decode tolerance of the float64 oracle, on two calls
in a row whose second input is smaller (the scratch keeps the first call's
contents)."""

import ctypes

import numpy as np
import pytest

import oracle
from io_aware_softmax_amd import inputs
from tests.gpu_common import compare, require_gpu, say, to_device, to_host_f64

pytestmark = pytest.mark.gpu

CODES = {"f32": 0, "f16": 1, "bf16": 2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield


def _call(fn, q, k, v, o, lse, B, H, Lk, D, scale, splits, stream, dtype):
    return fn(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
              ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()), B, H, Lk, D, ctypes.c_float(scale),
              splits, ctypes.c_void_p(stream), CODES[dtype])


def test_noalloc_decode_matches_decode_twice():
    import torch
    from io_aware_softmax_amd import binding
    lib = binding.load()
    stream = torch.cuda.current_stream().cuda_stream
    cases = [  # the second input is smaller than the first
        ("noalloc_big", 4, 8, 1, 20000, 128, "bf16", 0),
        ("noalloc_small", 2, 3, 1, 777, 64, "f16", 3),
    ]
    for name, B, H, Lq, Lk, D, dtype, splits in cases:
        say(f"case {name}: B{B} H{H} Lk{Lk} D{D} {dtype} splits={splits}")
        wl = inputs.custom(name, B, H, Lq, Lk, D, dtype, False, seed=Lk + D)
        bits = inputs.generate(wl)
        q, k, v = (to_device(bits[t], dtype) for t in "qkv")
        o_ref = torch.empty_like(q)
        lse_ref = torch.empty((B, H, 1), dtype=torch.float32, device="cuda")
        o_na = torch.full_like(q, float("nan"))
        lse_na = torch.full((B, H, 1), float("nan"), dtype=torch.float32, device="cuda")
        assert _call(lib.attn_decode_fwd, q, k, v, o_ref, lse_ref, B, H, Lk, D, wl.scale, splits, stream,
                     dtype) == 0
        assert _call(lib.attn_decode_fwd_noalloc, q, k, v, o_na, lse_na, B, H, Lk, D, wl.scale, splits, stream,
                     dtype) == 0
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ref) and torch.equal(lse_na, lse_ref), f"{name}: not bit-identical"
        vals = {t: inputs.to_float32(bits[t], dtype) for t in "qkv"}
        Or, Lr = oracle.attention(vals["q"], vals["k"], vals["v"], wl.scale, False)
        compare(name, dtype, to_host_f64(o_na), to_host_f64(lse_na), Or, Lr)


def test_noalloc_rejects_oversized_partials():
    """B * H * splits * (D + 2) * 4 bytes beyond ATTN_NOALLOC_SCRATCH_BYTES:
    128 x 256 partials of 130 floats need 17 MB of the 16 MiB, so the call
    is refused (ATTN_ERR_WORKSPACE) before it launches anything."""
    import torch
    from io_aware_softmax_amd import binding
    lib = binding.load()
    H, Lk, D, splits = 128, 256, 128, 256
    assert H * splits * (D + 2) * 4 > binding.ATTN_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((1, H, 1, D), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, H, Lk, D), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(x)
    lse = torch.empty((1, H, 1), dtype=torch.float32, device="cuda")
    st = _call(lib.attn_decode_fwd_noalloc, x, kv, kv, o, lse, 1, H, Lk, D, 0.1, splits,
               torch.cuda.current_stream().cuda_stream, "bf16")
    assert st == -13, st
