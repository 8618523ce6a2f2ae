"""GPU parity of the prefill kernels' own paths, against the float64 oracle.

16-bit inputs at D = 128 run the two-group kernel; ATTN_PREFILL_KERNEL=single
sends them to the single-group kernel instead, so both are checked on the
same inputs.  The two-group kernel moves a row's reference maximum only when
a lane's weight sum passes 2^8 (for bf16 then 24 above the tile maximum);
the cases below force that path on every few tiles (scores rising along the
keys), never after the first tile (falling scores), and through an
exponential that overflows to inf (scores of thousands).  The item schedule
has three branches (one item per workgroup with and without per-XCD ranges,
persistent workgroups over uneven ranges); each gets a case.  A persistent
workgroup starts its next item inside the current item's last step; the
transition cases reach its branches (V_0 of the next item issued early or
after the step, one-tile items, rows past Lq, Lq < Lk).  Bounds are the
documented ones: max |dO| 1e-2 (fp16), 2e-2 (bf16); LSE within
1e-4 * max(1, |LSE_ref|).
"""

import numpy as np
import pytest

import oracle
from io_aware_softmax_amd import inputs
from tests.gpu_common import O_TOL, compare, require_gpu, say, to_device, to_host_f64

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


def _fwd(vals, dtype, causal, scale):
    import torch
    from io_aware_softmax_amd import binding
    q, k, v = (to_device(inputs.round_to(vals[t], dtype), dtype) for t in "qkv")
    O, L = binding.attn_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return to_host_f64(O), to_host_f64(L)


def _exact(vals, dtype):
    """float32 values of the rounded inputs (what both sides compute on)."""
    return {t: inputs.to_float32(inputs.round_to(vals[t], dtype), dtype) for t in "qkv"}


def _check(name, vals, dtype, causal, scale):
    ex = _exact(vals, dtype)
    Or, Lr = oracle.attention(ex["q"], ex["k"], ex["v"], scale, causal)
    O, L = _fwd(vals, dtype, causal, scale)
    return compare(name, dtype, O, L, Or, Lr), O


def _normal(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape, dtype=np.float32)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_kernels_agree(dtype, causal, monkeypatch):
    """Both 16-bit prefill kernels at D = 128 on several tiles and a ragged tail."""
    B, H, L, D = 1, 4, 700, 128
    vals = {t: _normal((B, H, L, D), 500 + i + 10 * causal) for i, t in enumerate("qkv")}
    scale = 1.0 / np.sqrt(D)
    say(f"case kernels agree {dtype} causal={causal}")
    _, O_two = _check(f"two-group {dtype} c{int(causal)}", vals, dtype, causal, scale)
    monkeypatch.setenv("ATTN_PREFILL_KERNEL", "single")
    _, O_one = _check(f"single-group {dtype} c{int(causal)}", vals, dtype, causal, scale)
    assert np.max(np.abs(O_two - O_one)) <= 2 * O_TOL[dtype]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("pattern", ["rising", "falling"])
def test_reference_moves(dtype, pattern):
    """Row maxima that rise tile after tile (the reference moves every few
    tiles) or fall (only the first tile sets it)."""
    B, H, L, D = 1, 2, 1500, 128
    q = 0.1 * _normal((B, H, L, D), 601)
    k = 0.1 * _normal((B, H, L, D), 602)
    v = _normal((B, H, L, D), 603)
    q[..., 0] = 1.0
    ramp = np.arange(L, dtype=np.float32) * 0.4  # scores up to ~ 600 / sqrt(128) along the keys
    k[..., 0] = ramp if pattern == "rising" else ramp[::-1]
    vals = {"q": q, "k": k, "v": v}
    say(f"case reference moves {dtype} {pattern}")
    for causal in (False, True):
        _check(f"{pattern} {dtype} c{int(causal)}", vals, dtype, causal, 1.0 / np.sqrt(D))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_huge_scores_overflow_path(dtype):
    """Scale 40: scaled scores of thousands, so the first weights of a tile
    overflow to inf and the tile is redone from its maximum."""
    B, H, L, D = 1, 2, 400, 128
    vals = {t: _normal((B, H, L, D), 700 + i) for i, t in enumerate("qkv")}
    say(f"case huge scores {dtype}")
    for causal in (False, True):
        _check(f"huge {dtype} c{int(causal)}", vals, dtype, causal, 40.0)


@pytest.mark.parametrize("H,L,causal", [(257, 256, False), (37, 1024, True), (8, 512, True)])
def test_item_schedules(H, L, causal):
    """257 query tiles: more than one resident wave of workgroups, ranges of
    33 items with a short last one.  37 heads x 4 tiles: one item per
    workgroup, count not a multiple of 8.  8 x 2: one item per workgroup in
    per-XCD ranges."""
    B, D = 1, 128
    vals = {t: _normal((B, H, L, D), 800 + i + H) for i, t in enumerate("qkv")}
    say(f"case item schedule H{H} L{L} causal={causal}")
    _check(f"schedule H{H} L{L}", vals, "bf16", causal, 1.0 / np.sqrt(D))


@pytest.mark.parametrize("H,Lq,Lk,causal,dtype", [
    (130, 320, 320, False, "bf16"),  # 5 key tiles: the last V tile in buffer 0, so V_0 of the next item waits
    (130, 320, 320, True, "f16"),    # causal: items of 4 and 5 key tiles, a query tile with 64 live rows
    (300, 48, 48, False, "bf16"),    # one key tile per item (the first step is also the last)
    (300, 48, 48, True, "bf16"),
    (300, 100, 200, True, "bf16"),   # Lq < Lk: bottom-right causal, ragged tiles, persistent
])
def test_item_transitions(H, Lq, Lk, causal, dtype):
    """More items than resident workgroups, so each workgroup starts its next
    item inside the last step of the current one: the next item's Q, K_0,
    K_1 (and V_0 when the last V tile sits in the other buffer) load while
    the last value products run.  The shapes reach an odd key-tile count
    (V_0 issued after the last step), one-tile items, query tiles with rows
    past Lq and a rectangular causal problem."""
    B, D = 1, 128
    vals = {"q": _normal((B, H, Lq, D), 950 + H), "k": _normal((B, H, Lk, D), 951 + H),
            "v": _normal((B, H, Lk, D), 952 + H)}
    say(f"case item transitions H{H} Lq{Lq} Lk{Lk} causal={causal} {dtype}")
    _check(f"transitions H{H} {Lq}x{Lk} {dtype} c{int(causal)}", vals, dtype, causal, 1.0 / np.sqrt(D))


@pytest.mark.parametrize("B,H,Lq,Lk,D,dtype,causal", [
    (4, 8, 8192, 8192, 64, "f16", False),      # the fp16 sweep extended to L = 8192
    (1, 32, 512, 8192, 128, "bf16", True),     # chunked prefill: 512 new queries, 8192 cached keys
    (1, 32, 2048, 8192, 128, "bf16", True),
    (1, 1, 65536, 65536, 128, "bf16", True),   # one sequence, one head
])
def test_extended_shapes_sampled_rows(B, H, Lq, Lk, D, dtype, causal):
    """Shapes of the extended sweep, on 64 seeded rows per (b, h) (rows 0 and
    Lq-1 included)."""
    import torch
    from io_aware_softmax_amd import binding
    wl = inputs.custom(f"ext_{B}x{H}_{Lq}x{Lk}_D{D}", B, H, Lq, Lk, D, dtype, causal, seed=Lq + Lk + D)
    bits = inputs.generate(wl)
    q, k, v = (to_device(bits[t], dtype) for t in "qkv")
    O, L = binding.attn_fwd(q, k, v, causal=causal, scale=wl.scale)
    torch.cuda.synchronize()
    O, L = to_host_f64(O), to_host_f64(L)
    say(f"case extended shape B{B} H{H} Lq{Lq} Lk{Lk} D{D} {dtype} causal={causal}")
    for b in range(B):
        for h in range(H):
            rows = inputs.sample_rows(wl, h, 64)
            vals = {t: inputs.slab_values(wl, t, b, h)[None, None] for t in "qkv"}
            Or, Lr = oracle.attention(vals["q"], vals["k"], vals["v"], wl.scale, causal, rows=rows)
            compare(f"{wl.name} b{b} h{h}", dtype, O[b, h][rows][None, None], L[b, h][rows][None, None], Or, Lr)


# Causal needs Lq <= Lk, so the Lq > Lk shape runs non-causal only.
TWO_GROUP_D64 = [(B, H, Lq, Lk, causal) for (B, H, Lq, Lk) in [(1, 4, 700, 700), (2, 3, 300, 1000), (1, 2, 1000, 300)]
                 for causal in (False, True) if not (causal and Lq > Lk)]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("B,H,Lq,Lk,causal", TWO_GROUP_D64)
def test_two_group_d64(B, H, Lq, Lk, causal, dtype, monkeypatch):
    """The two-group kernel at D = 64 (ATTN_PREFILL_KERNEL=two): ragged query
    and key tails, Lq < Lk and Lq > Lk, against the oracle and against the
    single-group kernel on the same inputs."""
    D = 64
    vals = {"q": _normal((B, H, Lq, D), 900 + Lq), "k": _normal((B, H, Lk, D), 901 + Lk),
            "v": _normal((B, H, Lk, D), 902 + Lk)}
    scale = 1.0 / np.sqrt(D)
    say(f"case two-group D64 {B}x{H} {Lq}x{Lk} {dtype} causal={causal}")
    monkeypatch.setenv("ATTN_PREFILL_KERNEL", "two")
    _, O_two = _check(f"two-group D64 {Lq}x{Lk} {dtype} c{int(causal)}", vals, dtype, causal, scale)
    monkeypatch.setenv("ATTN_PREFILL_KERNEL", "single")
    _, O_one = _check(f"single-group D64 {Lq}x{Lk} {dtype} c{int(causal)}", vals, dtype, causal, scale)
    assert np.max(np.abs(O_two - O_one)) <= 2 * O_TOL[dtype]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_two_group_d64_reference_paths(dtype, monkeypatch):
    """D = 64 on the two-group kernel: rising row maxima (the reference
    moves every few tiles) and scale 40 (weights overflow to inf)."""
    B, H, L, D = 1, 2, 1500, 64
    q = 0.1 * _normal((B, H, L, D), 611)
    k = 0.1 * _normal((B, H, L, D), 612)
    v = _normal((B, H, L, D), 613)
    q[..., 0] = 1.0
    k[..., 0] = np.arange(L, dtype=np.float32) * 0.3
    monkeypatch.setenv("ATTN_PREFILL_KERNEL", "two")
    say(f"case two-group D64 reference paths {dtype}")
    for causal in (False, True):
        _check(f"rising D64 {dtype} c{int(causal)}", {"q": q, "k": k, "v": v}, dtype, causal, 1.0 / np.sqrt(D))
    vals = {t: _normal((1, 2, 400, D), 710 + i) for i, t in enumerate("qkv")}
    for causal in (False, True):
        _check(f"huge D64 {dtype} c{int(causal)}", vals, dtype, causal, 40.0)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
def test_single_group_reference_paths(dtype, D, monkeypatch):
    """The single-group kernel (the default at D = 64; ATTN_PREFILL_KERNEL=single
    at D = 128): row maxima that rise tile after tile (fp16: the weight-sum
    check fails and the tile is redone from its maximum; bf16: the
    look-ahead maximum moves the reference), that fall (only the first tile
    sets it), and scale 40 (weights overflow to inf)."""
    B, H, L = 1, 2, 1500
    if D == 128:
        monkeypatch.setenv("ATTN_PREFILL_KERNEL", "single")
    say(f"case single-group reference paths D{D} {dtype}")
    for pattern in ("rising", "falling"):
        q = 0.1 * _normal((B, H, L, D), 621 + D)
        k = 0.1 * _normal((B, H, L, D), 622 + D)
        v = _normal((B, H, L, D), 623 + D)
        q[..., 0] = 1.0
        ramp = np.arange(L, dtype=np.float32) * 0.3
        k[..., 0] = ramp if pattern == "rising" else ramp[::-1]
        for causal in (False, True):
            _check(f"single {pattern} D{D} {dtype} c{int(causal)}", {"q": q, "k": k, "v": v}, dtype, causal,
                   1.0 / np.sqrt(D))
    vals = {t: _normal((1, 2, 400, D), 720 + i + D) for i, t in enumerate("qkv")}
    for causal in (False, True):
        _check(f"single huge D{D} {dtype} c{int(causal)}", vals, dtype, causal, 40.0)
