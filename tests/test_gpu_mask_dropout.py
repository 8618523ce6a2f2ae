"""GPU parity of the fused general mask and dropout (``attn_fwd_ex``,
``attn_bwd_ex``) against the float64 oracle (``attention_ex``,
``attention_ex_bwd``) on the same rounded inputs.

Masks are seeded (boolean with some rows left without any key, additive
with -inf entries), broadcast over batch or heads; dropout uses Philox4x32-10
on both sides, and one case reads the keep pattern back bit for bit (V = I
makes O_ij = P_ij Z_ij / (1 - p), so the dropped weights are exact zeros).
Bounds: forward as for the plain forward (max |dO| 1e-2 fp16, 2e-2 bf16;
LSE within 1e-4 * max(1, |LSE_ref|); rows without keys exactly O = 0,
LSE = -inf); backward max |x - x_ref| <= 4 u max |x_ref| (u = 2^-8 bf16,
2^-11 fp16) as for the plain backward.
"""

import functools

import numpy as np
import pytest

import oracle
from io_aware_softmax_amd import inputs
from tests.gpu_common import O_TOL, compare, require_gpu, say, to_device, to_host_f64

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


def _mask_tensor(mask):
    import torch
    if mask is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(mask)).cuda()


def _case(name, B, H, Lq, Lk, D, dtype, causal, seed, mask=None, kind=None, p=0.0, dseed=0, offset=0,
          bwd=True):
    import torch
    from io_aware_softmax_amd import binding
    wl = inputs.custom(name, B, H, Lq, Lk, D, dtype, causal, seed=seed)
    bits = inputs.generate(wl, ("q", "k", "v", "do"))
    q, k, v, do = (to_device(bits[t], dtype) for t in ("q", "k", "v", "do"))
    mt = _mask_tensor(mask)
    say(f"case {name} B{B} H{H} Lq{Lq} Lk{Lk} D{D} {dtype} causal={causal} mask={kind} "
        f"{None if mask is None else mask.shape} p={p} seed={dseed} offset={offset}")
    O, L = binding.attn_fwd_ex(q, k, v, causal=causal, scale=wl.scale, mask=mt, dropout_p=p, seed=dseed,
                               offset=offset)
    torch.cuda.synchronize()
    vals = {t: inputs.to_float32(bits[t], dtype) for t in ("q", "k", "v", "do")}
    kw = dict(mask=mask, mask_kind=kind, dropout_p=p, seed=dseed, offset=offset)
    Or, Lr = oracle.attention_ex(vals["q"], vals["k"], vals["v"], wl.scale, causal, **kw)
    O, L = to_host_f64(O), to_host_f64(L)
    empty = np.isneginf(Lr)
    assert np.all(O[empty] == 0) and np.all(np.isneginf(L[empty])), "rows without keys"
    compare(name, dtype, O[~empty], L[~empty], Or[~empty], Lr[~empty])
    if not bwd:
        return
    O_t, L_t = binding.attn_fwd_ex(q, k, v, causal=causal, scale=wl.scale, mask=mt, dropout_p=p, seed=dseed,
                                   offset=offset)
    grads = binding.attn_bwd_ex(q, k, v, O_t, L_t, do, causal=causal, scale=wl.scale, mask=mt, dropout_p=p,
                                seed=dseed, offset=offset)
    torch.cuda.synchronize()
    ref = oracle.attention_ex_bwd(vals["q"], vals["k"], vals["v"], vals["do"], wl.scale, causal, **kw)
    for tname, g, r in zip(("dQ", "dK", "dV"), grads, ref):
        g = to_host_f64(g)
        assert np.all(np.isfinite(g)), f"{name}: non-finite {tname}"
        scale = float(np.max(np.abs(r)))
        rel = float(np.max(np.abs(g - r))) / scale if scale > 0 else float(np.max(np.abs(g)))
        say(f"  {name} {tname}: ratio {rel:.3e} (tol {TAU[dtype]:.2e})")
        assert rel <= TAU[dtype], f"{name}: {tname} {rel}"


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bool_mask(dtype, D, causal):
    B, H, Lq, Lk = 2, 2, 200, 333
    mask = inputs.bool_mask(10 + D, (1, H, Lq, Lk), keep=0.6, empty_rows=3)
    _case(f"bool_{dtype}_D{D}_c{int(causal)}", B, H, Lq, Lk, D, dtype, causal, seed=20 + D, mask=mask, kind="bool")


# Boolean masks without dropout at Lk % 8 == 0: the forward loads the mask
# bytes of a whole aligned tile one tile ahead, and the dQ kernel reads whole
# aligned blocks as vectors.  Lk 256 and 512 are whole key tiles; 264 is
# aligned with a ragged last tile (element loads there).
ALIGNED_BOOL = ([(512, D, dtype, causal) for D in (64, 128) for dtype in ("f16", "bf16") for causal in (False, True)]
                + [(Lk, D, "bf16", causal) for Lk in (256, 264) for D in (64, 128) for causal in (False, True)])


@pytest.mark.parametrize("Lk,D,dtype,causal", ALIGNED_BOOL)
def test_bool_mask_aligned_no_dropout(Lk, D, dtype, causal):
    B, H, Lq = 2, 2, 200
    mshape = (B, H, Lq, Lk) if Lk == 264 else (1, H, Lq, Lk)
    mask = inputs.bool_mask(Lk + D, mshape, keep=0.6, empty_rows=3)
    _case(f"bool_al_{Lk}_{dtype}_D{D}_c{int(causal)}", B, H, Lq, Lk, D, dtype, causal, seed=Lk + D + int(causal),
          mask=mask, kind="bool")


@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "f16")])
@pytest.mark.parametrize("causal", [False, True])
def test_additive_mask_aligned_no_dropout(D, dtype, causal):
    B, H, Lq, Lk = 2, 2, 200, 512
    mask = inputs.additive_mask(90 + D, (1, H, Lq, Lk), neg_inf=0.2)
    _case(f"add_al_{dtype}_D{D}_c{int(causal)}", B, H, Lq, Lk, D, dtype, causal, seed=91 + D, mask=mask,
          kind="add")


@pytest.mark.parametrize("Lq,Lk,D,dtype", [(520, 520, 128, "bf16"), (200, 584, 128, "bf16"), (520, 520, 64, "f16")])
@pytest.mark.parametrize("causal", [False, True])
def test_additive_mask_aligned_ragged_tail(Lq, Lk, D, dtype, causal):
    """Aligned rows (Lk % 8 == 0) whose last key tile is partial: the
    whole tiles take the terms loaded a tile ahead, the last one its own
    loads; with causal, waves stop at different tiles."""
    B, H = 1, 2
    mask = inputs.additive_mask(Lk + 3 * D, (1, H, Lq, Lk), neg_inf=0.15)
    _case(f"add_tail_{Lq}x{Lk}_{dtype}_D{D}_c{int(causal)}", B, H, Lq, Lk, D, dtype, causal, seed=Lq + Lk + D,
          mask=mask, kind="add")


@pytest.mark.parametrize("causal", [False, True])
def test_additive_mask_batch_broadcast(causal):
    B, H, Lq, Lk = 2, 3, 150, 260
    mask = inputs.additive_mask(31, (B, 1, Lq, Lk))
    _case(f"add_c{int(causal)}", B, H, Lq, Lk, 128, "bf16", causal, seed=31, mask=mask, kind="add")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout(dtype, p):
    _case(f"drop_{dtype}_{p}", 1, 3, 260, 260, 128, dtype, True, seed=40, p=p, dseed=0x1234_5678_9ABC_DEF0, offset=3)


def test_mask_and_dropout_together():
    mask = inputs.additive_mask(51, (1, 1, 130, 400), neg_inf=0.3)
    _case("add_drop", 2, 2, 130, 400, 64, "bf16", True, seed=51, mask=mask, kind="add", p=0.3, dseed=9, offset=77)


def test_all_ones_mask_matches_plain_forward():
    """The mask kernel with nothing masked against the plain kernels."""
    import torch
    from io_aware_softmax_amd import binding
    wl = inputs.custom("ones", 1, 4, 300, 300, 128, "bf16", True, seed=61)
    bits = inputs.generate(wl)
    q, k, v = (to_device(bits[t], "bf16") for t in "qkv")
    ones = torch.ones((1, 1, 300, 300), dtype=torch.uint8, device="cuda")
    O1, L1 = binding.attn_fwd_ex(q, k, v, causal=True, mask=ones)
    O2, L2 = binding.attn_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    say("case all-ones mask vs plain forward")
    assert (O1.float() - O2.float()).abs().max().item() <= 2 * O_TOL["bf16"]
    assert ((L1 - L2).abs() / L2.abs().clamp(min=1)).max().item() <= 2e-4


def test_dropout_keep_pattern_bit_exact():
    """V = I (Lk = D = 128): O_ij = P_ij Z_ij / (1 - p), so the zeros of O
    are exactly the dropped weights; compared with the oracle's Philox."""
    import torch
    from io_aware_softmax_amd import binding
    from oracle import philox
    B, H, Lq, Lk, D, p = 2, 2, 96, 128, 128, 0.3
    wl = inputs.custom("keep_bits", B, H, Lq, Lk, D, "bf16", False, seed=71)
    bits = inputs.generate(wl, ("q", "k"))
    q, k = (to_device(bits[t], "bf16") for t in "qk")
    v = torch.eye(D, dtype=torch.bfloat16, device="cuda").expand(B, H, Lk, D).contiguous()
    for seed, offset in ((5, 0), (2 ** 40 + 3, 12345)):
        O, _ = binding.attn_fwd_ex(q, k, v, dropout_p=p, seed=seed, offset=offset)
        torch.cuda.synchronize()
        got = (O.float().cpu().numpy() != 0)
        say(f"case keep pattern seed={seed} offset={offset}")
        for b in range(B):
            for h in range(H):
                ref = philox.keep_pattern(seed, offset, b * H + h, np.arange(Lq), Lk, p)
                assert np.array_equal(got[b, h], ref), (b, h)


def test_ex_deterministic_and_offset_sensitive():
    import torch
    from io_aware_softmax_amd import binding
    wl = inputs.custom("det_ex", 1, 4, 256, 256, 128, "bf16", True, seed=81)
    bits = inputs.generate(wl)
    q, k, v = (to_device(bits[t], "bf16") for t in "qkv")
    a, _ = binding.attn_fwd_ex(q, k, v, causal=True, dropout_p=0.2, seed=1, offset=0)
    b, _ = binding.attn_fwd_ex(q, k, v, causal=True, dropout_p=0.2, seed=1, offset=0)
    c, _ = binding.attn_fwd_ex(q, k, v, causal=True, dropout_p=0.2, seed=1, offset=1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert not torch.equal(a, c)


# Scores rising by about 60 (base 2) along every row of even heads and
# falling along odd heads: within a row the kernel's reference value has to
# move several times (rising), or one early key holds most of the weight
# (falling: the rounding of the dominant weight).
REF_MOVES = [  # dtype, D, mask kind, dropout p, Lq, Lk, causal
    ("bf16", 128, "bool", 0.0, 96, 640, False),
    ("bf16", 128, "add", 0.0, 320, 320, True),
    ("bf16", 64, None, 0.3, 96, 640, False),
    ("bf16", 128, "bool", 0.2, 320, 320, True),
    ("bf16", 64, "add", 0.0, 96, 640, False),
    ("f16", 64, "bool", 0.0, 96, 640, False),
    ("f16", 128, "add", 0.1, 320, 320, True),
    ("f16", 64, None, 0.3, 320, 320, True),
]


@pytest.mark.parametrize("dtype,D,kind,p,Lq,Lk,causal", REF_MOVES)
def test_ex_reference_moves(dtype, D, kind, p, Lq, Lk, causal):
    """Forward on ``inputs.rising_scores`` (B1 H2, scale 1/sqrt(D)).
    Boolean masks (70% kept) also hide keys [0, 150) from 16 rows in the
    middle of Lq, which then have no visible key for two or more tiles;
    additive masks are N(0, 15^2) with 10% -inf and every 7th key -1e4.

    Forward only: on rows where one key holds nearly all the weight, the
    backward's dP - Dv cancels, and Dv = sum_d dO O taken from the stored
    16-bit O (the output the backward is handed) then moves dQ by several
    percent of its largest entry, more than the random-input gradient bound
    allows; the exact-O oracle cannot tell that apart from a kernel error."""
    import torch
    from io_aware_softmax_amd import binding
    B, H = 1, 2
    scale = 1.0 / np.sqrt(D)
    seed = 31 * Lq + Lk + D
    q32, k32, v32 = inputs.rising_scores(seed, B, H, Lq, Lk, D, span=60.0 / (scale * np.log2(np.e)))
    bits = {t: inputs.round_to(x, dtype) for t, x in zip(("q", "k", "v"), (q32, k32, v32))}
    q, k, v = (to_device(bits[t], dtype) for t in ("q", "k", "v"))
    mask = None
    if kind == "bool":
        mask = inputs.bool_mask(seed, (B, H, Lq, Lk), keep=0.7)
        r0 = Lq // 2
        mask[:, :, r0:r0 + 16, :150] = 0
    elif kind == "add":
        mask = inputs.additive_mask(seed, (B, H, Lq, Lk), sigma=15.0, neg_inf=0.1)
        mask[..., ::7] = -1e4
    name = f"refmoves_{dtype}_D{D}_{kind}_p{p}_{Lq}x{Lk}_{'causal' if causal else 'full'}"
    say(f"case {name}")
    O, L = binding.attn_fwd_ex(q, k, v, causal=causal, scale=scale, mask=_mask_tensor(mask), dropout_p=p, seed=9)
    torch.cuda.synchronize()
    vals = {t: inputs.to_float32(bits[t], dtype) for t in ("q", "k", "v")}
    Or, Lr = oracle.attention_ex(vals["q"], vals["k"], vals["v"], scale, causal, mask=mask, mask_kind=kind,
                                 dropout_p=p, seed=9)
    O, L = to_host_f64(O), to_host_f64(L)
    empty = np.isneginf(Lr)
    assert np.all(O[empty] == 0) and np.all(np.isneginf(L[empty])), "rows without keys"
    compare(name, dtype, O[~empty], L[~empty], Or[~empty], Lr[~empty])


@pytest.mark.parametrize("B,H,Lq,Lk,D,dtype,causal,kind,mshape,p,scale", [
    (2, 3, 1, 1000, 128, "bf16", False, "bool", "full", 0.25, None),      # one query per (b, h)
    (2, 2, 77, 77, 64, "f16", True, "add", "full", 0.0, -0.3),            # negative scale, full mask
    (1, 2, 300, 130, 64, "f16", False, "add", "heads", 0.4, None),        # Lq > Lk
    (3, 2, 65, 129, 128, "bf16", True, "bool", "batch", 0.05, None),      # tile + 1 on both sides
    (1, 3, 200, 256, 128, "bf16", True, "bool", "shared", 0.0, None),     # odd B*H, one mask for all heads
    (3, 1, 130, 200, 64, "f16", False, "add", "shared", 0.1, None),       # odd B*H over batches
])
def test_ex_edge_shapes(B, H, Lq, Lk, D, dtype, causal, kind, mshape, p, scale):
    shape = {"full": (B, H, Lq, Lk), "heads": (1, H, Lq, Lk), "batch": (B, 1, Lq, Lk),
             "shared": (1, 1, Lq, Lk)}[mshape]
    if kind == "bool":
        mask = inputs.bool_mask(Lq + Lk, shape, keep=0.7, empty_rows=1)
    else:
        mask = inputs.additive_mask(Lq + Lk, shape, neg_inf=0.2)
    name = f"edge_{Lq}x{Lk}_D{D}_{dtype}_{kind}_{mshape}_p{p}"
    if scale is None:
        _case(name, B, H, Lq, Lk, D, dtype, causal, seed=Lq * 7 + Lk, mask=mask, kind=kind, p=p,
              dseed=(1 << 63) | 12345, offset=0xFFFFFFFF)
    else:
        _case_scaled(name, B, H, Lq, Lk, D, dtype, causal, Lq * 7 + Lk, mask, kind, p, scale)


def _case_scaled(name, B, H, Lq, Lk, D, dtype, causal, seed, mask, kind, p, scale):
    """As _case with an explicit scale (forward and backward)."""
    import torch
    from io_aware_softmax_amd import binding
    wl = inputs.custom(name, B, H, Lq, Lk, D, dtype, causal, seed=seed)
    bits = inputs.generate(wl, ("q", "k", "v", "do"))
    q, k, v, do = (to_device(bits[t], dtype) for t in ("q", "k", "v", "do"))
    mt = _mask_tensor(mask)
    say(f"case {name} scale={scale}")
    O, L = binding.attn_fwd_ex(q, k, v, causal=causal, scale=scale, mask=mt, dropout_p=p, seed=4)
    grads = binding.attn_bwd_ex(q, k, v, O, L, do, causal=causal, scale=scale, mask=mt, dropout_p=p, seed=4)
    torch.cuda.synchronize()
    vals = {t: inputs.to_float32(bits[t], dtype) for t in ("q", "k", "v", "do")}
    kw = dict(mask=mask, mask_kind=kind, dropout_p=p, seed=4)
    Or, Lr = oracle.attention_ex(vals["q"], vals["k"], vals["v"], scale, causal, **kw)
    O, L = to_host_f64(O), to_host_f64(L)
    empty = np.isneginf(Lr)
    assert np.all(O[empty] == 0) and np.all(np.isneginf(L[empty]))
    compare(name, dtype, O[~empty], L[~empty], Or[~empty], Lr[~empty])
    ref = oracle.attention_ex_bwd(vals["q"], vals["k"], vals["v"], vals["do"], scale, causal, **kw)
    for tname, g, r in zip(("dQ", "dK", "dV"), grads, ref):
        g = to_host_f64(g)
        rel = float(np.max(np.abs(g - r))) / max(float(np.max(np.abs(r))), 1e-30)
        say(f"  {name} {tname}: ratio {rel:.3e} (tol {TAU[dtype]:.2e})")
        assert rel <= TAU[dtype], f"{name}: {tname} {rel}"


# The causal bf16 8k workload (q x8 on heads 0-3) with the masks and dropout
# the masked-forward measurement times: a boolean mask keeping half the keys
# of every row (broadcast over batch and heads), an additive N(0, 4) mask,
# dropout 0.1, and the boolean mask with dropout 0.1.  Forward on seeded
# sampled rows of every head (the same rows in each head, plus the first
# rows and the tile and diagonal boundaries).
C3_EX_CASES = {
    "bool mask": ("bool", 0.0),
    "additive mask": ("add", 0.0),
    "dropout 0.1": (None, 0.1),
    "bool mask + dropout 0.1": ("bool", 0.1),
}


@functools.lru_cache(maxsize=1)
def _c3_inputs():
    wl = inputs.WORKLOADS["causal_bf16_8k"]
    return wl, inputs.generate(wl, ("q", "k", "v", "do"))


@functools.lru_cache(maxsize=2)
def _c3_mask(kind, L):
    """Drawn once per kind (about 15 s for 8192 x 8192 on the host)."""
    if kind == "bool":
        return inputs.bool_mask(5, (1, 1, L, L), keep=0.5)
    if kind == "add":
        return inputs.additive_mask(6, (1, 1, L, L), neg_inf=0.0)
    return None


@pytest.mark.parametrize("case", list(C3_EX_CASES))
def test_c3_shape_masked_forward_sampled_rows(case):
    import torch
    from io_aware_softmax_amd import binding
    kind, p = C3_EX_CASES[case]
    wl, bits = _c3_inputs()
    L = wl.Lq
    mask = _c3_mask(kind, L)
    q, k, v = (to_device(bits[t], "bf16") for t in "qkv")
    say(f"case c3 shape, {case}: B{wl.B} H{wl.H} L{L} D{wl.D} causal, 128 sampled rows per head")
    O, Lse = binding.attn_fwd_ex(q, k, v, causal=True, scale=wl.scale, mask=_mask_tensor(mask), dropout_p=p,
                                 seed=3)
    torch.cuda.synchronize()
    O, Lse = to_host_f64(O), to_host_f64(Lse)
    rows = np.unique(np.concatenate([inputs.sample_rows(wl, 0, 112),
                                     [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 4095, 4096, 8190, 8191]]))
    vals = {t: inputs.to_float32(bits[t], "bf16") for t in "qkv"}
    Or, Lr = oracle.attention_ex(vals["q"], vals["k"], vals["v"], wl.scale, True, mask=mask, mask_kind=kind,
                                 dropout_p=p, seed=3, offset=0, rows=rows)
    Og, Lg = O[:, :, rows], Lse[:, :, rows]
    empty = np.isneginf(Lr)
    assert np.all(Og[empty] == 0) and np.all(np.isneginf(Lg[empty])), "rows without keys"
    compare(f"c3 {case}", "bf16", Og[~empty], Lg[~empty], Or[~empty], Lr[~empty])
    del O, Lse, q, k, v
    torch.cuda.empty_cache()


def test_c3_shape_bool_mask_backward_full_heads():
    """attn_bwd_ex at the causal bf16 8k shape with the half-keep boolean
    mask: dQ, dK, dV of two whole heads (one with x8 queries) against the
    oracle's chain rule."""
    import torch
    from io_aware_softmax_amd import binding
    wl, bits = _c3_inputs()
    L = wl.Lq
    mask = _c3_mask("bool", L)
    mt = _mask_tensor(mask)
    q, k, v, do = (to_device(bits[t], "bf16") for t in ("q", "k", "v", "do"))
    say(f"case c3 shape, bool mask backward: B{wl.B} H{wl.H} L{L}, heads 1 and 17 in full")
    O, Lse = binding.attn_fwd_ex(q, k, v, causal=True, scale=wl.scale, mask=mt)
    grads = binding.attn_bwd_ex(q, k, v, O, Lse, do, causal=True, scale=wl.scale, mask=mt)
    torch.cuda.synchronize()
    grads = [to_host_f64(g) for g in grads]
    for h in (1, 17):
        vals = {t: inputs.to_float32(bits[t][:, h:h + 1], "bf16") for t in ("q", "k", "v", "do")}
        ref = oracle.attention_ex_bwd(vals["q"], vals["k"], vals["v"], vals["do"], wl.scale, True, mask=mask,
                                      mask_kind="bool")
        for tname, g, r in zip(("dQ", "dK", "dV"), grads, ref):
            gh = g[:, h:h + 1]
            assert np.all(np.isfinite(gh)), f"non-finite {tname}"
            rel = float(np.max(np.abs(gh - r))) / float(np.max(np.abs(r)))
            say(f"  c3 bool bwd h{h} {tname}: ratio {rel:.3e} (tol {TAU['bf16']:.2e})")
            assert rel <= TAU["bf16"], f"h{h} {tname} {rel}"
    del grads, q, k, v, do, O, Lse
    torch.cuda.empty_cache()
