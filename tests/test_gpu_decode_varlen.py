"""GPU parity of the ragged-length KV-cache decode against the float64 oracle.

``attn_decode_varlen_fwd`` attends each (b, h) to the first seqlens[b] keys
of a [B, H, Lk_max, D] cache.  Rows past a length are filled with NaN here,
so any read of them would show in the output.  Lengths include 0 (O = 0,
lse = -inf), 1, Lk_max, one past Lk_max and a negative one (both clamped).
Bounds as for the other cases: max |dO| 1e-5 / 1e-2 / 2e-2 for
fp32 / fp16 / bf16; LSE within 1e-4 * max(1, |LSE_ref|).
"""

import numpy as np
import pytest

import oracle
from io_aware_softmax_amd import inputs
from tests.gpu_common import O_TOL, compare, require_gpu, say, to_device, to_host_f64

pytestmark = pytest.mark.gpu

NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import io_aware_softmax_amd as m
    m.load()
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _poison(bits, lens, dtype):
    """Rows past each sequence's length become NaN."""
    for b, n in enumerate(lens):
        n = max(0, min(int(n), bits.shape[2]))
        if dtype == "f32":
            bits[b, :, n:] = np.nan
        else:
            bits[b, :, n:] = NAN_BITS[dtype]


def _run(wl, bits, lens, num_splits=0, bh=None):
    import torch
    from io_aware_softmax_amd import binding
    q, k, v = (to_device(bits[t], wl.dtype) for t in "qkv")
    sl = torch.tensor(np.asarray(lens, dtype=np.int32), device="cuda")
    O, L = binding.attn_decode_varlen_fwd(q, k, v, sl, scale=wl.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return to_host_f64(O), to_host_f64(L)


def _check(wl, bits, lens, num_splits=0, slabs=None):
    O, L = _run(wl, bits, lens, num_splits)
    vals = {t: inputs.to_float32(bits[t], wl.dtype) for t in "qkv"}
    if slabs is None:
        Or, Lr = oracle.decode_varlen(vals["q"], vals["k"], vals["v"], lens, wl.scale)
        empty = np.isneginf(Lr)
        assert np.all(O[empty[..., 0]] == 0) and np.all(np.isneginf(L[empty])), "empty sequence"
        keep = ~empty[:, :, 0]
        return compare(f"{wl.name} splits={num_splits}", wl.dtype, O[keep], L[keep], Or[keep], Lr[keep])
    errs = []
    for b, h in slabs:
        Or, Lr = oracle.decode_varlen(vals["q"][b:b + 1, h:h + 1], vals["k"][b:b + 1, h:h + 1],
                                      vals["v"][b:b + 1, h:h + 1], [lens[b]], wl.scale)
        errs.append(compare(f"{wl.name} b{b} h{h}", wl.dtype, O[b:b + 1, h:h + 1], L[b:b + 1, h:h + 1], Or, Lr))
    return errs


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_varlen_parity(dtype, D):
    Lk_max = 3000
    wl = inputs.custom(f"varlen_{dtype}_{D}", 8, 3, 1, Lk_max, D, dtype, False, seed=61 + D)
    bits = inputs.generate(wl)
    lens = [0, 1, Lk_max, Lk_max + 7, -3, 64, 1001, 2999]
    _poison(bits["k"], lens, dtype)
    _poison(bits["v"], lens, dtype)
    say(f"case varlen {dtype} D{D} lens={lens}")
    _check(wl, bits, lens)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_varlen_split_independence(dtype):
    Lk_max = 5000
    wl = inputs.custom(f"varlen_splits_{dtype}", 4, 2, 1, Lk_max, 128, dtype, False, seed=71)
    bits = inputs.generate(wl)
    lens = inputs.ragged_lengths(71, 4, Lk_max)
    _poison(bits["k"], lens, dtype)
    _poison(bits["v"], lens, dtype)
    base = None
    for s in (1, 3, 16, 256):
        say(f"case varlen splits={s} {dtype}")
        _check(wl, bits, lens, num_splits=s)
        O, _ = _run(wl, bits, lens, num_splits=s)
        if base is None:
            base = O
        else:
            assert np.max(np.abs(O - base)) <= O_TOL[dtype]


def test_varlen_decode_full_size():
    """B16 H32 D128 bf16 over a 32768-key cache with seeded ragged lengths
    (the decode workload's shape), checked on 12 (b, h) slabs."""
    base = inputs.WORKLOADS["decode_bf16_32k"]
    wl = inputs.custom("varlen_decode_bf16_32k", base.B, base.H, 1, base.Lk, base.D, "bf16", False, seed=4)
    bits = inputs.generate(wl)
    lens = inputs.ragged_lengths(4, wl.B, wl.Lk)
    _poison(bits["k"], lens, "bf16")
    _poison(bits["v"], lens, "bf16")
    rng = np.random.default_rng(4)
    slabs = [(int(b), int(h)) for b, h in zip(rng.integers(0, wl.B, 12), rng.integers(0, wl.H, 12))]
    say(f"case varlen full size lens={lens.tolist()}")
    _check(wl, bits, lens, slabs=slabs)
