"""GPU parity of the attention backward (``attn_bwd``) against the float64 oracle.

The HIP forward produces O and LSE, the HIP backward then produces dQ, dK,
dV from them and a seeded upstream gradient dO; the oracle differentiates
the exact definition on the same rounded q, k, v, dO.

Bound: for each of dQ, dK, dV, max |x - x_ref| <= tau * max |x_ref| with
tau = 4 u, u the unit roundoff of the storage type (2^-8 for bf16, 2^-11
for fp16): the weights P and the score gradients dS enter the products
rounded to the storage type (relative error <= u / 2 each), the output is
rounded once more (u / 2), and Dv = rowsum(dO o O) is formed from the
16-bit O of the forward; all sums are fp32.
"""

import numpy as np
import pytest

import oracle
from io_aware_softmax_amd import inputs
from tests.gpu_common import require_gpu, say, to_device, to_host_f64

pytestmark = pytest.mark.gpu

TAU = {"bf16": 4 * 2.0 ** -8, "f16": 4 * 2.0 ** -11}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    import io_aware_softmax_amd as m
    m.load()
    yield
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _run(bits, dtype, causal, scale):
    import torch
    from io_aware_softmax_amd import binding
    q, k, v, do = (to_device(bits[t], dtype) for t in ("q", "k", "v", "do"))
    O, L = binding.attn_fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = binding.attn_bwd(q, k, v, O, L, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return tuple(to_host_f64(t) for t in (dq, dk, dv))


def _values(bits, dtype):
    return {t: inputs.to_float32(bits[t], dtype) for t in bits}


def _compare(name, dtype, got, ref):
    errs = []
    for tname, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert np.all(np.isfinite(g)), f"{name}: non-finite {tname}"
        scale = float(np.max(np.abs(r)))
        err = float(np.max(np.abs(g - r)))
        rel = err / scale if scale > 0 else err
        errs.append(rel)
        say(f"  {name} {tname}: max|err|={err:.3e}  max|ref|={scale:.3e}  ratio={rel:.3e} (tol {TAU[dtype]:.2e})")
    for tname, rel in zip(("dQ", "dK", "dV"), errs):
        assert rel <= TAU[dtype], f"{name}: {tname} error ratio {rel} > {TAU[dtype]}"
    return errs


def _case(name, B, H, Lq, Lk, D, dtype, causal, seed, scale=None, q_mult=()):
    wl = inputs.custom(name, B, H, Lq, Lk, D, dtype, causal, seed=seed, q_head_mult=q_mult)
    bits = inputs.generate(wl, ("q", "k", "v", "do"))
    scale = wl.scale if scale is None else scale
    say(f"case {name} B{B} H{H} Lq{Lq} Lk{Lk} D{D} {dtype} causal={causal} scale={scale:.4g}")
    got = _run(bits, dtype, causal, scale)
    vals = _values(bits, dtype)
    ref = oracle.attention_bwd(vals["q"], vals["k"], vals["v"], vals["do"], scale, causal)
    return _compare(name, dtype, got, ref), got, bits


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_parity(dtype, D, causal):
    """333 x 333: six 64-row tiles and three 128-row blocks, ragged tails."""
    _case(f"bwd_{dtype}_D{D}_c{int(causal)}", 1, 2, 333, 333, D, dtype, causal, seed=40 + D + causal)


@pytest.mark.parametrize("Lq,Lk,causal", [(200, 517, True), (200, 517, False), (517, 200, False),
                                          (1, 300, False), (64, 64, True), (130, 1000, True)])
def test_backward_rectangular(Lq, Lk, causal):
    """Lq != Lk (chunked prefill, causal aligned bottom-right), a single
    query, and exact tile multiples."""
    _case(f"bwd_rect_{Lq}x{Lk}", 2, 2, Lq, Lk, 128, "bf16", causal, seed=Lq + 7 * Lk)


@pytest.mark.parametrize("Lq,Lk,D,causal", [(768, 768, 128, True), (832, 832, 128, True), (640, 896, 128, True),
                                            (832, 832, 128, False), (768, 832, 64, True)])
def test_backward_tile_loops(Lq, Lk, D, causal):
    """Whole query tiles only (Lq % 64 == 0), even and odd tile counts and
    diagonal offsets: the dK/dV kernel splits its tiles into generic ones
    before the slot-scheduled range, the range (which starts in the first
    stage), and generic ones after it, per wave; the dQ kernel runs its
    unmasked tiles in a loop of their own."""
    _case(f"bwd_loops_{Lq}x{Lk}_D{D}_c{int(causal)}", 1, 2, Lq, Lk, D, "bf16", causal, seed=Lq + 3 * Lk + D)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_backward_sharp_weights(dtype):
    """Queries x8 on half the heads and scale 1: near one-hot weights."""
    _case(f"bwd_sharp_{dtype}", 1, 4, 300, 300, 128, dtype, True, seed=77, scale=1.0,
          q_mult=((0, 8.0), (1, 8.0)))


def test_backward_negative_and_zero_scale():
    for s in (-0.2, 0.0):
        _case(f"bwd_scale_{s}", 1, 2, 150, 190, 64, "bf16", False, seed=88, scale=s)


def test_backward_zero_upstream_gradient():
    import torch
    from io_aware_softmax_amd import binding
    wl = inputs.custom("bwd_zero_do", 1, 2, 200, 200, 128, "bf16", True, seed=91)
    bits = inputs.generate(wl)
    q, k, v = (to_device(bits[t], "bf16") for t in "qkv")
    O, L = binding.attn_fwd(q, k, v, causal=True)
    do = torch.zeros_like(q)
    for g in binding.attn_bwd(q, k, v, O, L, do, causal=True):
        assert torch.count_nonzero(g).item() == 0


def test_backward_deterministic():
    import torch
    from io_aware_softmax_amd import binding
    wl = inputs.custom("bwd_det", 1, 8, 1000, 1000, 128, "bf16", True, seed=92)
    bits = inputs.generate(wl, ("q", "k", "v", "do"))
    q, k, v, do = (to_device(bits[t], "bf16") for t in ("q", "k", "v", "do"))
    O, L = binding.attn_fwd(q, k, v, causal=True)
    a = binding.attn_bwd(q, k, v, O, L, do, causal=True)
    b = binding.attn_bwd(q, k, v, O, L, do, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_full_size_sampled():
    """The causal bf16 prefill shape (B1 H32 L8192 D128, queries x8 on heads
    0-3): dQ on 64 seeded query rows and dK, dV on 64 seeded key rows of
    four heads (two of them x8), against the oracle on those rows; the key
    gradients of every head sum to zero over the keys."""
    import torch
    from io_aware_softmax_amd import binding
    wl = inputs.WORKLOADS["causal_bf16_8k"]
    bits = inputs.generate(wl, ("q", "k", "v", "do"))
    q, k, v, do = (to_device(bits[t], "bf16") for t in ("q", "k", "v", "do"))
    O, L = binding.attn_fwd(q, k, v, causal=True, scale=wl.scale)
    dq, dk, dv = binding.attn_bwd(q, k, v, O, L, do, causal=True, scale=wl.scale)
    torch.cuda.synchronize()
    say("case full size causal_bf16_8k backward")
    # sum_j dK_j = 0 per head (float32 sums of the bf16 outputs)
    s = dk.float().sum(dim=2).abs().amax().item()
    mag = dk.float().abs().sum(dim=2).amax().item()
    say(f"  |sum_j dK_j| max {s:.3e} vs sum_j |dK_j| {mag:.3e}")
    assert s <= 1e-2 * mag
    dq, dk, dv = (to_host_f64(t) for t in (dq, dk, dv))
    for h in (0, 3, 17, 31):
        rows = inputs.sample_rows(wl, h, 64)
        vals = {t: inputs.slab_values(wl, t, 0, h)[None, None] for t in ("q", "k", "v")}
        vals["do"] = inputs.to_float32(bits["do"][0, h], "bf16")[None, None]
        rq, rk, rv = oracle.attention_bwd(vals["q"], vals["k"], vals["v"], vals["do"], wl.scale, True,
                                          q_rows=rows, k_rows=rows)
        _compare(f"causal_bf16_8k h{h}", "bf16", (dq[0, h][rows], dk[0, h][rows], dv[0, h][rows]),
                 (rq[0, 0], rk[0, 0], rv[0, 0]))
