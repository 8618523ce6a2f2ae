"""CPU tests of the C ABI: the library loads, exports what include/attn.h
declares, and rejects every bad argument before touching the GPU.

Validation calls use fake (never dereferenced) pointers; they return before
any HIP call, so they run in a container without a GPU.
"""

import re
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "attn.h"

binding = pytest.importorskip("io_aware_softmax_amd.binding")


def _declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def _header_enum(name):
    m = re.search(rf"\b{name}\s*=\s*(-?\d+)", HEADER.read_text())
    return int(m.group(1))


@pytest.fixture(scope="module")
def lib():
    if not binding.LIB_PATH.exists():
        pytest.fail("libattn.so is not built; run __graft_entry__.build()")
    return binding.load()


def test_exports_every_declared_function(lib):
    declared = _declared_functions()
    assert set(declared) == set(binding.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", str(binding.LIB_PATH)],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_[a-z_]+)\b", out))
    assert set(declared) <= exported, set(declared) - exported
    for name in declared:
        assert hasattr(lib, name)
    # Nothing beyond the declared API is exported under the attn_ prefix.
    assert exported == set(declared)


def test_noalloc_validation_errors(lib):
    """attn_decode_fwd_noalloc: the forward's checks, the split range, and
    ATTN_ERR_WORKSPACE when the partials would not fit the fixed scratch,
    all before any HIP call."""
    e = {n: _header_enum(n) for n in ("ATTN_ERR_NULL", "ATTN_ERR_DIM", "ATTN_ERR_SPLITS", "ATTN_ERR_WORKSPACE",
                                       "ATTN_ERR_ALIAS", "ATTN_ERR_UNSUPPORTED_D")}
    n = lib.attn_decode_fwd_noalloc
    cap = int(re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", HEADER.read_text()).group(1)) << 20
    assert cap == binding.ATTN_NOALLOC_SCRATCH_BYTES
    assert n(0, 2 * G, 3 * G, 4 * G, 5 * G, 2, 3, 100, 64, 0.1, 4, None, 2) == e["ATTN_ERR_NULL"]
    assert n(G, 2 * G, 3 * G, 4 * G, 5 * G, 2, 3, 100, 64, 0.1, 257, None, 2) == e["ATTN_ERR_SPLITS"]
    assert n(G, 2 * G, 3 * G, 4 * G, 5 * G, 2, 3, 100, 48, 0.1, 4, None, 2) == e["ATTN_ERR_UNSUPPORTED_D"]
    assert n(G, 2 * G, 3 * G, G, 5 * G, 2, 3, 100, 64, 0.1, 4, None, 2) == e["ATTN_ERR_ALIAS"]
    # partials of (D + 2) * 4 bytes per (b, h, split): the largest B * H * splits that fits, and one more
    for D in (64, 128):
        fit = cap // ((D + 2) * 4)
        H = fit // 256  # with 256 splits
        assert n(G, 2 * G, 3 * G, 4 * G, 5 * G, 1, H + 1, 1 << 16, D, 0.1, 256, None, 2) == e["ATTN_ERR_WORKSPACE"]
    assert n(G, 2 * G, 3 * G, 4 * G, 5 * G, 16, 32, 32768, 128, 0.1, 256, None, 2) == e["ATTN_ERR_WORKSPACE"]


def test_header_constants_match_binding():
    assert _header_enum("ATTN_F32") == binding.ATTN_F32
    assert _header_enum("ATTN_F16") == binding.ATTN_F16
    assert _header_enum("ATTN_BF16") == binding.ATTN_BF16
    assert int(re.search(r"#define ATTN_MAX_SPLITS (\d+)", HEADER.read_text()).group(1)) == binding.ATTN_MAX_SPLITS


G = 1 << 40  # fake, far-apart, 16-byte aligned device addresses


def _fwd(lib, q=G, k=2 * G, v=3 * G, o=4 * G, lse=5 * G, B=2, H=3, Lq=16, Lk=16, D=64,
         causal=0, scale=0.125, dtype=2):
    return lib.attn_fwd(q, k, v, o, lse, B, H, Lq, Lk, D, causal, scale, None, dtype)


def test_validation_errors(lib):
    e = {n: _header_enum(n) for n in ("ATTN_ERR_NULL", "ATTN_ERR_DIM", "ATTN_ERR_UNSUPPORTED_D",
                                       "ATTN_ERR_DTYPE", "ATTN_ERR_SCALE", "ATTN_ERR_CAUSAL_SHAPE",
                                       "ATTN_ERR_SPLITS", "ATTN_ERR_ALIAS", "ATTN_ERR_ALIGN")}
    for kw in ("q", "k", "v", "o", "lse"):
        assert _fwd(lib, **{kw: 0}) == e["ATTN_ERR_NULL"]
    for kw in ("B", "H", "Lq", "Lk", "D"):
        assert _fwd(lib, **{kw: 0}) == e["ATTN_ERR_DIM"]
        assert _fwd(lib, **{kw: -5}) == e["ATTN_ERR_DIM"]
    for d in (32, 96, 256, 65, 127):
        assert _fwd(lib, D=d) == e["ATTN_ERR_UNSUPPORTED_D"]
    assert _fwd(lib, Lq=(1 << 31) // 64 + 1) == e["ATTN_ERR_DIM"]
    assert _fwd(lib, Lk=(1 << 30), D=128) == e["ATTN_ERR_DIM"]
    assert _fwd(lib, B=1 << 16, H=1 << 16) == e["ATTN_ERR_DIM"]
    for dt in (-1, 3, 99):
        assert _fwd(lib, dtype=dt) == e["ATTN_ERR_DTYPE"]
    for s in (float("nan"), float("inf"), float("-inf")):
        assert _fwd(lib, scale=s) == e["ATTN_ERR_SCALE"]
    assert _fwd(lib, causal=1, Lq=17, Lk=16) == e["ATTN_ERR_CAUSAL_SHAPE"]
    assert _fwd(lib, o=G) == e["ATTN_ERR_ALIAS"]              # o == q
    assert _fwd(lib, o=2 * G + 64) == e["ATTN_ERR_ALIAS"]     # o inside k
    assert _fwd(lib, lse=3 * G + 128) == e["ATTN_ERR_ALIAS"]  # lse inside v
    assert _fwd(lib, lse=4 * G + 16) == e["ATTN_ERR_ALIAS"]   # lse inside o
    for kw in ("q", "k", "v", "o"):
        assert _fwd(lib, **{kw: {"q": G, "k": 2 * G, "v": 3 * G, "o": 4 * G}[kw] + 8}) == e["ATTN_ERR_ALIGN"]
    assert _fwd(lib, lse=5 * G + 2) == e["ATTN_ERR_ALIGN"]
    # decode entry point
    d = lib.attn_decode_fwd
    assert d(G, 2 * G, 3 * G, 4 * G, 5 * G, 2, 3, 100, 64, 0.1, -1, None, 2) == e["ATTN_ERR_SPLITS"]
    assert d(G, 2 * G, 3 * G, 4 * G, 5 * G, 2, 3, 100, 64, 0.1, 257, None, 2) == e["ATTN_ERR_SPLITS"]
    assert d(G, 2 * G, 3 * G, 4 * G, 5 * G, 2, 3, 100, 48, 0.1, 4, None, 2) == e["ATTN_ERR_UNSUPPORTED_D"]
    assert d(G, 0, 3 * G, 4 * G, 5 * G, 2, 3, 100, 64, 0.1, 4, None, 2) == e["ATTN_ERR_NULL"]
    assert d(G, 2 * G, 3 * G, 4 * G, 5 * G, 2, 3, 0, 64, 0.1, 4, None, 2) == e["ATTN_ERR_DIM"]
    # ragged-length decode entry point (seqlens at 6 G)
    r = lib.attn_decode_varlen_fwd
    assert r(G, 2 * G, 3 * G, 4 * G, 5 * G, 0, 2, 3, 100, 64, 0.1, 0, None, 2) == e["ATTN_ERR_NULL"]
    assert r(G, 2 * G, 3 * G, 4 * G, 5 * G, 6 * G + 2, 2, 3, 100, 64, 0.1, 0, None, 2) == e["ATTN_ERR_ALIGN"]
    assert r(G, 2 * G, 3 * G, 4 * G, 5 * G, 6 * G, 2, 3, 100, 64, 0.1, 300, None, 2) == e["ATTN_ERR_SPLITS"]
    assert r(G, 2 * G, 3 * G, 4 * G, 5 * G, 6 * G, 2, 3, 0, 64, 0.1, 0, None, 2) == e["ATTN_ERR_DIM"]
    assert r(G, 2 * G, 3 * G, 4 * G, 5 * G, 4 * G + 8, 2, 3, 100, 64, 0.1, 0, None, 2) == e["ATTN_ERR_ALIAS"]
    assert r(G, 2 * G, 3 * G, 4 * G, 5 * G, 5 * G, 2, 3, 100, 64, 0.1, 0, None, 2) == e["ATTN_ERR_ALIAS"]


def _bwd(lib, q=G, k=2 * G, v=3 * G, o=4 * G, do=5 * G, lse=6 * G, dq=7 * G, dk=8 * G, dv=9 * G,
         B=2, H=3, Lq=16, Lk=16, D=64, causal=0, scale=0.125, dtype=2):
    return lib.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, Lq, Lk, D, causal, scale, None, dtype)


def test_backward_validation_errors(lib):
    e = {n: _header_enum(n) for n in ("ATTN_ERR_NULL", "ATTN_ERR_DIM", "ATTN_ERR_UNSUPPORTED_D",
                                       "ATTN_ERR_DTYPE", "ATTN_ERR_SCALE", "ATTN_ERR_CAUSAL_SHAPE",
                                       "ATTN_ERR_ALIAS", "ATTN_ERR_ALIGN")}
    for kw in ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv"):
        assert _bwd(lib, **{kw: 0}) == e["ATTN_ERR_NULL"]
    for kw in ("B", "H", "Lq", "Lk", "D"):
        assert _bwd(lib, **{kw: 0}) == e["ATTN_ERR_DIM"]
    assert _bwd(lib, D=96) == e["ATTN_ERR_UNSUPPORTED_D"]
    for dt in (0, -1, 3):  # fp32 has no backward
        assert _bwd(lib, dtype=dt) == e["ATTN_ERR_DTYPE"]
    assert _bwd(lib, scale=float("nan")) == e["ATTN_ERR_SCALE"]
    assert _bwd(lib, causal=1, Lq=20, Lk=16) == e["ATTN_ERR_CAUSAL_SHAPE"]
    base = {"q": G, "k": 2 * G, "v": 3 * G, "o": 4 * G, "do": 5 * G, "lse": 6 * G}
    for out in ("dq", "dk", "dv"):
        for name, addr in base.items():
            assert _bwd(lib, **{out: addr + 64}) == e["ATTN_ERR_ALIAS"], (out, name)
    assert _bwd(lib, dk=7 * G + 32) == e["ATTN_ERR_ALIAS"]   # dk inside dq
    assert _bwd(lib, dv=8 * G) == e["ATTN_ERR_ALIAS"]        # dv == dk
    for kw in ("do", "dq", "dk", "dv"):
        assert _bwd(lib, **{kw: {"do": 5 * G, "dq": 7 * G, "dk": 8 * G, "dv": 9 * G}[kw] + 8}) == e["ATTN_ERR_ALIGN"]


def test_ex_validation_errors(lib):
    e = {n: _header_enum(n) for n in ("ATTN_ERR_NULL", "ATTN_ERR_DTYPE", "ATTN_ERR_MASK", "ATTN_ERR_DROPOUT",
                                       "ATTN_ERR_ALIAS", "ATTN_ERR_ALIGN", "ATTN_ERR_DIM")}

    def fwd(mask=10 * G, kind=1, mb=1, mh=3, p=0.0, dtype=2, o=4 * G, Lq=16):
        return lib.attn_fwd_ex(G, 2 * G, 3 * G, o, 5 * G, 2, 3, Lq, 16, 64, 0, 0.125, mask, kind, mb, mh, p, 7, 0,
                               None, dtype)

    def bwd(mask=10 * G, kind=2, mb=2, mh=1, p=0.0, dq=7 * G):
        return lib.attn_bwd_ex(G, 2 * G, 3 * G, 4 * G, 5 * G, 6 * G, dq, 8 * G, 9 * G, 2, 3, 16, 16, 64, 0, 0.125,
                               mask, kind, mb, mh, p, 7, 0, None, 2)
    assert fwd(mask=0) == e["ATTN_ERR_NULL"]
    assert fwd(kind=3) == e["ATTN_ERR_MASK"] and fwd(kind=-1) == e["ATTN_ERR_MASK"]
    assert fwd(mb=3) == e["ATTN_ERR_MASK"] and fwd(mh=2) == e["ATTN_ERR_MASK"]
    assert fwd(mask=10 * G + 8) == e["ATTN_ERR_ALIGN"]
    for p in (-0.1, 1.0, 1.5, float("nan"), float("inf")):
        assert fwd(p=p) == e["ATTN_ERR_DROPOUT"]
    assert fwd(dtype=0) == e["ATTN_ERR_DTYPE"]
    assert fwd(o=10 * G + 256) == e["ATTN_ERR_ALIAS"]        # o inside the mask
    assert fwd(Lq=0) == e["ATTN_ERR_DIM"]
    assert bwd(dq=10 * G + 64) == e["ATTN_ERR_ALIAS"]        # dq inside the additive mask
    assert bwd(kind=5) == e["ATTN_ERR_MASK"]
    assert bwd(p=2.0) == e["ATTN_ERR_DROPOUT"]
    assert bwd(mask=0) == e["ATTN_ERR_NULL"]


def test_strerror_and_auto_splits(lib):
    for code in range(-13, 1):
        msg = binding.attn_strerror(code)
        assert msg and msg != "unknown status"
    assert binding.attn_strerror(-14) == "unknown status"
    assert binding.attn_strerror(-10).startswith("HIP error")
    s = binding.attn_decode_auto_splits(16, 32, 32768, 128)
    assert 1 <= s <= binding.ATTN_MAX_SPLITS
    assert binding.attn_decode_auto_splits(1, 1, 4, 64) == 1
    assert lib.attn_decode_auto_splits(1, 1, 4, 48) == _header_enum("ATTN_ERR_UNSUPPORTED_D")
    assert lib.attn_decode_auto_splits(0, 1, 4, 64) == _header_enum("ATTN_ERR_DIM")


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        binding.attn_fwd(x, x, x)


def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.bfloat16)


def _expect_value_error(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_binding_rejects_mismatched_shapes():
    """Every size the C ABI takes from q.shape and k.shape is checked against
    the other tensors before any pointer is passed on: a shorter v, or a k
    with another B, H or D, would make the kernels read past the end of a
    buffer, and a wrong out / lse would make them write past it.  The checks
    run before the device check, so CPU tensors reach them here."""
    import torch
    q, k, v = _cpu(2, 3, 16, 64), _cpu(2, 3, 20, 64), _cpu(2, 3, 20, 64)
    f = binding.attn_fwd
    _expect_value_error(lambda: f(q, k, _cpu(2, 3, 19, 64)), "v must have the shape of k")
    _expect_value_error(lambda: f(q, _cpu(2, 3, 20, 32), _cpu(2, 3, 20, 32)), "k must be")
    _expect_value_error(lambda: f(q, _cpu(1, 3, 20, 64), _cpu(1, 3, 20, 64)), "k must be")
    _expect_value_error(lambda: f(q, _cpu(2, 2, 20, 64), _cpu(2, 2, 20, 64)), "k must be")
    _expect_value_error(lambda: f(q, k, v, out=_cpu(2, 3, 15, 64)), "out must be")
    _expect_value_error(lambda: f(q, k, v, out=_cpu(2, 3, 16, 64, dtype=torch.float16)), "out must be")
    _expect_value_error(lambda: f(q, k, v, lse=_cpu(2, 3, 17, dtype=torch.float32)), "lse must be")
    _expect_value_error(lambda: f(q, k, v, lse=_cpu(2, 3, 16)), "lse must be")
    _expect_value_error(lambda: f(q, k.half(), v), "share one of")
    _expect_value_error(lambda: f(q[:, :, :, :3], k, v), "q must be")
    _expect_value_error(lambda: f(q.transpose(2, 3), k, v), "contiguous")
    _expect_value_error(lambda: f(q, k, v), "GPU tensor")  # everything consistent: only the device is wrong
    # decode entry points
    q1 = _cpu(2, 3, 1, 64)
    _expect_value_error(lambda: binding.attn_decode_fwd(q1, k, _cpu(2, 3, 21, 64)), "v must have the shape of k")
    _expect_value_error(lambda: binding.attn_decode_fwd(q, k, v), "one query")
    sl = torch.zeros(2, dtype=torch.int32)
    _expect_value_error(lambda: binding.attn_decode_varlen_fwd(q1, k, v, torch.zeros(3, dtype=torch.int32)),
                        "seqlens")
    _expect_value_error(lambda: binding.attn_decode_varlen_fwd(q1, k, _cpu(2, 3, 20, 128), sl), "v must have")
    _expect_value_error(lambda: binding.attn_decode_varlen_fwd(q1, k, v, sl), "GPU tensor")


def test_binding_backward_checks():
    """attn_bwd and attn_bwd_ex apply the same checks: out / dout like q, lse
    [B, H, Lq] float32, caller gradients like their inputs."""
    import torch
    q, k, v = _cpu(2, 3, 16, 64), _cpu(2, 3, 20, 64), _cpu(2, 3, 20, 64)
    o, do, lse = _cpu(2, 3, 16, 64), _cpu(2, 3, 16, 64), _cpu(2, 3, 16, dtype=torch.float32)
    for fn in (binding.attn_bwd, binding.attn_bwd_ex):
        _expect_value_error(lambda: fn(q, k, _cpu(2, 3, 19, 64), o, lse, do), "v must have the shape of k")
        _expect_value_error(lambda: fn(q, k, v, _cpu(2, 3, 15, 64), lse, do), "out must be")
        _expect_value_error(lambda: fn(q, k, v, o, _cpu(2, 3, 15, dtype=torch.float32), do), "lse must be")
        _expect_value_error(lambda: fn(q, k, v, o, lse, _cpu(2, 3, 16, 32)), "dout must be")
        _expect_value_error(lambda: fn(q, k, v, o, lse, do, dq=_cpu(2, 3, 20, 64)), "dq must be")
        _expect_value_error(lambda: fn(q, k, v, o, lse, do, dk=_cpu(2, 3, 16, 64)), "dk must be")
        _expect_value_error(lambda: fn(q, k, v, o, lse, do, dv=_cpu(2, 3, 20, 64, dtype=torch.float16)), "dv must be")
        _expect_value_error(lambda: fn(q, k, v, o, None, do), "required")
        _expect_value_error(lambda: fn(q, k, v, o, lse, do), "GPU tensor")


def test_binding_mask_checks():
    import torch
    q, k, v = _cpu(2, 3, 16, 64), _cpu(2, 3, 20, 64), _cpu(2, 3, 20, 64)
    f = binding.attn_fwd_ex
    _expect_value_error(lambda: f(q, k, v, mask=torch.ones(2, 3, 16, 19, dtype=torch.bool)), "mask must be")
    _expect_value_error(lambda: f(q, k, v, mask=torch.ones(3, 1, 16, 20, dtype=torch.bool)), "mask must be")
    _expect_value_error(lambda: f(q, k, v, mask=torch.ones(1, 2, 16, 20, dtype=torch.bool)), "mask must be")
    _expect_value_error(lambda: f(q, k, v, mask=torch.ones(1, 1, 16, 20, dtype=torch.float16)), "mask dtype")
    _expect_value_error(lambda: f(q, k, v, mask=torch.ones(1, 1, 16, 20, dtype=torch.bool)), "GPU tensor")
