"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Every case draws its inputs from the seeded generator, runs them through
``attn_fwd`` / ``attn_decode_fwd`` of libattn.so and compares element by
element with ``oracle.attention`` on the same rounded inputs.  Bounds: max
abs error on O of 1e-5 (fp32), 1e-2 (fp16), 2e-2 (bf16); LSE within
1e-4 * max(1, |LSE_ref|).  The causal bf16 8k prefill and the decode
workload are checked in full (every row, every slab), in the launch
configuration the benchmark times; the 64k long-context workload and the
longest sweep lengths on seeded sampled rows.
"""

import math
from pathlib import Path

import numpy as np
import pytest

import oracle
from io_aware_softmax_amd import inputs
from tests.gpu_common import compare, require_gpu, say, to_device, to_host_f64

pytestmark = pytest.mark.gpu

GOLDEN = Path(__file__).parent / "golden" / "worked_example_1234.txt"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import io_aware_softmax_amd as m
    m.load()
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _binding():
    from io_aware_softmax_amd import binding
    return binding


def _run(wl, bits, num_splits=None, scale=None):
    import torch
    b = _binding()
    q, k, v = (to_device(bits[t], wl.dtype) for t in "qkv")
    scale = wl.scale if scale is None else scale
    if num_splits is None:
        O, L = b.attn_fwd(q, k, v, causal=wl.causal, scale=scale)
    else:
        O, L = b.attn_decode_fwd(q, k, v, scale=scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return O, L


def _values(wl, bits):
    return {t: inputs.to_float32(bits[t], wl.dtype) for t in "qkv"}


def _check_full(wl, scale=None, num_splits=None, bits=None, o_tol=None):
    say(f"case {wl.name}: B{wl.B} H{wl.H} Lq{wl.Lq} Lk{wl.Lk} D{wl.D} {wl.dtype} causal={wl.causal}"
        f" splits={num_splits}")
    bits = inputs.generate(wl) if bits is None else bits
    O, L = _run(wl, bits, num_splits, scale)
    vals = _values(wl, bits)
    scale = wl.scale if scale is None else scale
    Or, Lr = oracle.attention(vals["q"], vals["k"], vals["v"], scale, wl.causal)
    return compare(wl.name, wl.dtype, to_host_f64(O), to_host_f64(L), Or, Lr, o_tol)


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------

def test_check_f32_full():
    _check_full(inputs.WORKLOADS["check_f32"])


@pytest.mark.parametrize("L", inputs.SWEEP_LENGTHS)
def test_sweep_f16(L):
    wl = inputs.WORKLOADS[f"sweep_f16_L{L}"]
    if L <= 1024:
        _check_full(wl)
        return
    say(f"case {wl.name}: 64 sampled rows per head")
    bits = inputs.generate(wl)
    O, Lse = _run(wl, bits)
    O, Lse = to_host_f64(O), to_host_f64(Lse)
    vals = _values(wl, bits)
    for h in range(wl.H):
        rows = inputs.sample_rows(wl, h, 64)
        for b in range(wl.B):
            Or, Lr = oracle.attention(vals["q"][b:b + 1, h:h + 1], vals["k"][b:b + 1, h:h + 1],
                                      vals["v"][b:b + 1, h:h + 1], wl.scale, False, rows=rows)
            compare(f"{wl.name} b{b} h{h}", wl.dtype, O[b, h, rows][None, None],
                    Lse[b, h, rows][None, None], Or, Lr)


def _sampled_prefill(wl, rows_per_head, extra_rows=()):
    import torch
    say(f"case {wl.name}: full size, {rows_per_head} sampled rows per head")
    bits = inputs.generate(wl)
    O, L = _run(wl, bits)
    O, L = to_host_f64(O), to_host_f64(L)
    worst = [0.0, 0.0]
    for h in range(wl.H):
        rows = inputs.sample_rows(wl, h, rows_per_head)
        rows = np.unique(np.concatenate([rows, [r for r in extra_rows if r < wl.Lq]])).astype(np.int64)
        for b in range(wl.B):
            q = inputs.to_float32(bits["q"][b, h], wl.dtype)[None, None]
            k = inputs.to_float32(bits["k"][b, h], wl.dtype)[None, None]
            v = inputs.to_float32(bits["v"][b, h], wl.dtype)[None, None]
            Or, Lr = oracle.attention(q, k, v, wl.scale, wl.causal, rows=rows)
            eo, el = compare(f"{wl.name} b{b} h{h}", wl.dtype, O[b, h, rows][None, None],
                             L[b, h, rows][None, None], Or, Lr)
            worst = [max(worst[0], eo), max(worst[1], el)]
    say(f"  {wl.name}: worst max|dO|={worst[0]:.3e} worst rel|dLSE|={worst[1]:.3e}")
    del O, L
    torch.cuda.empty_cache()


def test_causal_bf16_8k():
    """The causal bf16 8k workload in full: every row of every head (one
    head of the oracle at a time, to bound host memory)."""
    import torch
    wl = inputs.WORKLOADS["causal_bf16_8k"]
    say(f"case {wl.name}: full size, every row of every head")
    bits = inputs.generate(wl)
    O, L = _run(wl, bits)
    O, L = to_host_f64(O), to_host_f64(L)
    worst = [0.0, 0.0]
    for h in range(wl.H):
        q, k, v = (inputs.to_float32(bits[t][0, h], wl.dtype)[None, None] for t in "qkv")
        Or, Lr = oracle.attention(q, k, v, wl.scale, True)
        eo, el = compare(f"{wl.name} b0 h{h}", wl.dtype, O[0, h][None, None], L[0, h][None, None], Or, Lr)
        worst = [max(worst[0], eo), max(worst[1], el)]
    say(f"  {wl.name}: worst max|dO|={worst[0]:.3e} worst rel|dLSE|={worst[1]:.3e}")
    del O, L, bits
    torch.cuda.empty_cache()


def test_long_causal_bf16_64k():
    _sampled_prefill(inputs.WORKLOADS["long_causal_bf16_64k"], 256, extra_rows=(127, 128, 32768))


def test_decode_bf16_32k():
    """The decode workload in full: all B x H = 512 (batch, head) slabs."""
    import torch
    wl = inputs.WORKLOADS["decode_bf16_32k"]
    say(f"case {wl.name}: full size, auto splits, every (b, h) slab")
    bits = inputs.generate(wl)
    O, L = _run(wl, bits)
    O, L = to_host_f64(O), to_host_f64(L)
    worst = [0.0, 0.0]
    for b in range(wl.B):
        for h in range(wl.H):
            q, k, v = (inputs.to_float32(bits[t][b, h], wl.dtype)[None, None] for t in "qkv")
            Or, Lr = oracle.attention(q, k, v, wl.scale, False)
            eo, el = compare(f"{wl.name} b{b} h{h}", wl.dtype, O[b, h][None, None], L[b, h][None, None], Or, Lr)
            worst = [max(worst[0], eo), max(worst[1], el)]
    say(f"  {wl.name}: worst max|dO|={worst[0]:.3e} worst rel|dLSE|={worst[1]:.3e}")
    del bits
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# Edge shapes: ragged tails, Lq != Lk, one query, one key
# --------------------------------------------------------------------------

EDGE = [(7, 7), (63, 63), (65, 65), (127, 129), (129, 127), (1000, 1000), (1, 1000), (7, 1000),
        (65, 1), (1, 1), (129, 7), (200, 333)]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_edge_shapes(dtype, D, causal):
    for i, (Lq, Lk) in enumerate(EDGE):
        if causal and Lq > Lk:
            continue
        wl = inputs.custom(f"edge_{dtype}_D{D}_c{int(causal)}_{Lq}x{Lk}", 2, 3, Lq, Lk, D, dtype, causal,
                           seed=i + 10 * D + int(causal))
        _check_full(wl)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_q_scaled_heads_rescale_path(dtype):
    """x8 queries on some heads: row maxima jump late across key tiles.

    For fp32 the bound is the fp32 bound times 8: the rounding error of an
    fp32 dot product grows linearly with the magnitude of its terms, and x8
    queries make every score (and its rounding error) 8 times larger, which
    the exponential passes on to the weights.  The 16-bit bounds already
    cover it (they are set by the 16-bit rounding of P and O).
    """
    wl = inputs.custom(f"x8_{dtype}", 1, 4, 700, 700, 128, dtype, True, seed=77,
                       q_head_mult=((0, 8.0), (2, 8.0)))
    _check_full(wl, o_tol=8e-5 if dtype == "f32" else None)


# --------------------------------------------------------------------------
# Closed forms on the GPU
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_mean_of_values(dtype, causal):
    import torch
    wl = inputs.custom(f"idkeys_{dtype}", 1, 2, 300, 300, 64, dtype, causal, seed=5)
    bits = inputs.generate(wl)
    bits["k"][:] = bits["k"][:, :, :1, :]  # every key equals key 0
    O, L = _run(wl, bits)
    vals = _values(wl, bits)
    v = vals["v"].astype(np.float64)
    ref = (np.cumsum(v, axis=2) / np.arange(1, 301)[None, None, :, None]) if causal else \
        np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    a = wl.scale * np.einsum("bhid,bhd->bhi", vals["q"].astype(np.float64), vals["k"][:, :, 0].astype(np.float64))
    lref = a + (np.log(np.arange(1, 301))[None, None] if causal else math.log(300))
    say(f"case identical keys {dtype} causal={causal}")
    compare("identical keys", dtype, to_host_f64(O), to_host_f64(L), ref, lref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_values_expose_weights(dtype):
    # V = I (Lk = D): O rows are the attention weights themselves.
    wl = inputs.custom(f"vident_{dtype}", 1, 2, 50, 64, 64, dtype, True, seed=6)
    bits = inputs.generate(wl)
    eye = inputs.round_to(np.tile(np.eye(64, dtype=np.float32), (1, 2, 1, 1)), dtype)
    bits["v"] = eye.reshape(bits["v"].shape)
    say(f"case identity values {dtype}")
    O, L = _run(wl, bits)
    vals = _values(wl, bits)
    Or, Lr = oracle.attention(vals["q"], vals["k"], vals["v"], wl.scale, True)
    compare("identity values", dtype, to_host_f64(O), to_host_f64(L), Or, Lr)
    assert np.allclose(to_host_f64(O).sum(axis=-1), 1.0, atol=0.05)


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.9])
def test_scale_values(scale):
    wl = inputs.custom("scale", 2, 2, 150, 150, 64, "bf16", True, seed=8)
    _check_full(wl, scale=scale)
    wld = inputs.custom("scale_dec", 2, 2, 1, 900, 64, "f16", False, seed=9)
    _check_full(wld, scale=scale)


# --------------------------------------------------------------------------
# Split-KV decode
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_split_independence(dtype, D):
    wl = inputs.custom(f"dec_{dtype}_{D}", 2, 4, 1, 5000, D, dtype, False, seed=21 + D)
    bits = inputs.generate(wl)
    base = None
    for s in (1, 2, 3, 7, 16, 64, 256):
        eo, _ = _check_full(wl, num_splits=s, bits=bits)
        O, _ = _run(wl, bits, num_splits=s)
        O = to_host_f64(O)
        if base is None:
            base = O
        else:
            tol = {"f32": 1e-5, "f16": 2e-3, "bf16": 1.6e-2}[dtype]
            assert np.max(np.abs(O - base)) <= tol


def test_decode_more_splits_than_keys():
    wl = inputs.custom("dec_tiny", 3, 2, 1, 5, 128, "bf16", False, seed=31)
    for s in (1, 4, 5, 9, 256):
        _check_full(wl, num_splits=s)


def test_worked_example_through_decode():
    """[1,2,3,4] in two chunks: Lk = 4 keys, 2 splits of exactly [1,2] | [3,4]."""
    import torch
    vals = {}
    for line in GOLDEN.read_text().splitlines():
        if line and not line.startswith("#"):
            n, rest = line.split(":", 1)
            vals[n] = np.array([float(x) for x in rest.split()])
    D = 64
    q = torch.zeros(1, 1, 1, D, device="cuda")
    q[0, 0, 0, 0] = 1.0
    k = torch.zeros(1, 1, 4, D, device="cuda")
    k[0, 0, :, 0] = torch.tensor([1.0, 2.0, 3.0, 4.0])
    v = torch.zeros(1, 1, 4, D, device="cuda")
    v[0, 0, :, :4] = torch.eye(4)
    b = _binding()
    for splits in (2, 1, 4):
        O, L = b.attn_decode_fwd(q, k, v, scale=1.0, num_splits=splits)
        torch.cuda.synchronize()
        O = O.double().cpu().numpy()[0, 0, 0]
        say(f"case worked example splits={splits}: O={O[:4]} lse={float(L):.9f}")
        np.testing.assert_allclose(O[:4], vals["O2"], atol=2e-7)
        assert np.all(O[4:] == 0)
        np.testing.assert_allclose(float(L), vals["LSE"][0], rtol=1e-6)
    # The same problem through the prefill path (Lq = 2, both rows equal).
    q2 = q.expand(1, 1, 2, D).contiguous()
    O, L = b.attn_fwd(q2, k, v, causal=False, scale=1.0)
    torch.cuda.synchronize()
    np.testing.assert_allclose(O.double().cpu().numpy()[0, 0, :, :4], np.tile(vals["O2"], (2, 1)), atol=2e-7)


# --------------------------------------------------------------------------
# Determinism
# --------------------------------------------------------------------------

def test_repeatable_bitwise():
    import torch
    wl = inputs.custom("repeat", 2, 4, 777, 777, 128, "bf16", True, seed=41)
    bits = inputs.generate(wl)
    O1, L1 = _run(wl, bits)
    O2, L2 = _run(wl, bits)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)
    wd = inputs.custom("repeat_dec", 2, 4, 1, 7777, 128, "bf16", False, seed=42)
    bd = inputs.generate(wd)
    D1, M1 = _run(wd, bd, num_splits=0)
    D2, M2 = _run(wd, bd, num_splits=0)
    assert torch.equal(D1, D2) and torch.equal(M1, M2)
