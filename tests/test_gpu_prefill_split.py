"""GPU parity of the split-KV prefill (two-group kernel, D = 128) against the
float64 oracle.

Shapes with fewer 256-row query tiles than half the compute units cut every
tile's keys into ranges; each range writes its rows' normalised partial O
and log-sum-exp, and a merge applies the guide's output correction over the
ranges.  ATTN_PREFILL_SPLITS=n forces n ranges (capped so that none is
empty), so small shapes exercise: ranges in which some rows have no key
(their partials drop out), ragged Lq and Lk tails, ×8 queries (the row
reference moves inside a range) and the largest count (16).  Bounds as for
the plain forward: max |dO| 1e-2 fp16 / 2e-2 bf16, LSE within
1e-4 * max(1, |LSE_ref|).
"""

import numpy as np
import pytest

import oracle
from io_aware_softmax_amd import inputs
from tests.gpu_common import compare, require_gpu, say, to_device, to_host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import io_aware_softmax_amd as m
    m.load()
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _run(wl, bits, causal):
    import torch
    from io_aware_softmax_amd import binding
    q, k, v = (to_device(bits[t], wl.dtype) for t in "qkv")
    O, L = binding.attn_fwd(q, k, v, causal=causal, scale=wl.scale)
    torch.cuda.synchronize()
    return to_host_f64(O), to_host_f64(L)


@pytest.mark.parametrize("B,H,Lq,Lk,dtype,causal,splits,qmult", [
    (1, 2, 700, 700, "bf16", True, 3, ()),                 # first tile: 4 key tiles in 3 ranges
    (1, 2, 300, 1000, "f16", False, 5, ()),                # ragged Lq and Lk
    (2, 1, 257, 2000, "bf16", True, 16, ()),               # 16 ranges, chunk of 257 queries
    (1, 4, 520, 4096, "bf16", True, 6, ((0, 8.0), (1, 8.0))),  # x8 queries
    (1, 2, 64, 640, "f16", True, 9, ()),                   # one partial query tile
])
def test_forced_splits(B, H, Lq, Lk, dtype, causal, splits, qmult, monkeypatch):
    wl = inputs.custom(f"split_{Lq}x{Lk}", B, H, Lq, Lk, 128, dtype, causal, seed=Lq + Lk + splits, q_head_mult=qmult)
    bits = inputs.generate(wl)
    monkeypatch.setenv("ATTN_PREFILL_SPLITS", str(splits))
    say(f"case split {Lq}x{Lk} B{B} H{H} {dtype} causal={causal} splits={splits}")
    O, L = _run(wl, bits, causal)
    full = {t: inputs.to_float32(bits[t], dtype) for t in "qkv"}
    Or, Lr = oracle.attention(full["q"], full["k"], full["v"], wl.scale, causal)
    compare(f"split{splits} {Lq}x{Lk} {dtype}", dtype, O, L, Or, Lr)
    monkeypatch.setenv("ATTN_PREFILL_SPLITS", "1")
    O1, L1 = _run(wl, bits, causal)
    compare(f"unsplit {Lq}x{Lk} {dtype}", dtype, O1, L1, Or, Lr)


def test_auto_split_single_head_sampled_rows():
    """One head, 16384 causal: 64 query tiles, split automatically; 128
    seeded rows against the oracle, and the result is deterministic."""
    import torch
    from io_aware_softmax_amd import binding
    wl = inputs.custom("split_one_head_16k", 1, 1, 16384, 16384, 128, "bf16", True, seed=77)
    bits = inputs.generate(wl)
    say("case auto split one head 16k")
    q, k, v = (to_device(bits[t], "bf16") for t in "qkv")
    O, L = binding.attn_fwd(q, k, v, causal=True, scale=wl.scale)
    O2, L2 = binding.attn_fwd(q, k, v, causal=True, scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(O, O2) and torch.equal(L, L2)
    rows = inputs.sample_rows(wl, 0, 128)
    rows = np.unique(np.concatenate([rows, [0, 1, 63, 64, 255, 256, 8191, 16383]])).astype(np.int64)
    vals = {t: inputs.to_float32(bits[t][0, 0], "bf16")[None, None] for t in "qkv"}
    Or, Lr = oracle.attention(vals["q"], vals["k"], vals["v"], wl.scale, True, rows=rows)
    O, L = to_host_f64(O), to_host_f64(L)
    compare("auto split 1x16384", "bf16", O[0, 0, rows][None, None], L[0, 0, rows][None, None], Or, Lr)
