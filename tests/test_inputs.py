"""CPU tests of the seeded input generator (no attention arithmetic here)."""

import numpy as np
import pytest
import torch

from io_aware_softmax_amd import inputs


def test_same_seed_same_bytes_and_slabs_differ():
    wl = inputs.custom("t", 2, 3, 17, 17, 64, "bf16", False, seed=1)
    a = inputs.generate(wl, threads=4)
    b = inputs.generate(wl, threads=1)
    for t in "qkv":
        assert a[t].tobytes() == b[t].tobytes()
    assert not np.array_equal(a["q"][0, 0], a["q"][0, 1])
    assert not np.array_equal(a["q"][0, 0], a["k"][0, 0])
    assert not np.array_equal(a["q"][0, 0], a["q"][1, 0])
    np.testing.assert_array_equal(inputs.slab_values(wl, "k", 1, 2), inputs.to_float32(a["k"][1, 2], "bf16"))


@pytest.mark.parametrize("dtype,tdt", [("bf16", torch.bfloat16), ("f16", torch.float16)])
def test_rounding_matches_torch(dtype, tdt):
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 8,
                        np.array([1.00390625, 1.01171875, -2.0078125, 0.0, -0.0, 1e-30], np.float32)])
    bits = inputs.round_to(x, dtype)
    ref = torch.from_numpy(x).to(tdt).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = inputs.to_float32(bits, dtype)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(tdt).float().numpy())


def test_power_of_two_head_multiplier_is_exact():
    wl = inputs.WORKLOADS["causal_bf16_8k"]
    x1 = inputs.slab(wl.seed_words, "q", 0, 0, 64, 128, "bf16", 1.0)
    x8 = inputs.slab(wl.seed_words, "q", 0, 0, 64, 128, "bf16", 8.0)
    np.testing.assert_array_equal(inputs.to_float32(x8, "bf16"), 8 * inputs.to_float32(x1, "bf16"))
    assert wl.q_mult(3) == 8.0 and wl.q_mult(4) == 1.0
    with pytest.raises(ValueError):
        inputs.slab(wl.seed_words, "q", 0, 0, 4, 4, "bf16", 3.0)


def test_sample_rows():
    wl = inputs.WORKLOADS["long_causal_bf16_64k"]
    r = inputs.sample_rows(wl, 3)
    assert r.shape == (256,) and r[0] == 0 and r[-1] == 65535
    assert np.all(np.diff(r) > 0)
    np.testing.assert_array_equal(r, inputs.sample_rows(wl, 3))
    assert not np.array_equal(r, inputs.sample_rows(wl, 4))


def test_named_workloads():
    w = inputs.WORKLOADS
    assert (w["check_f32"].B, w["check_f32"].H, w["check_f32"].Lq, w["check_f32"].D) == (4, 8, 256, 64)
    assert w["causal_bf16_8k"].flops() == pytest.approx(5.4976e11, rel=1e-4)
    assert w["decode_bf16_32k"].kv_bytes() == 8589934592
    assert w["long_causal_bf16_64k"].flops() == pytest.approx(8.796e12, rel=1e-3)
    assert w["check_f32"].scale == 0.125


def test_upstream_gradient_draws():
    """dO has the queries' shape, its own stream (tensor id 3) and regenerates
    slab by slab."""
    wl = inputs.custom("do_draw", 2, 3, 17, 29, 64, "bf16", True, seed=5)
    a = inputs.generate(wl, ("q", "do"))
    assert a["do"].shape == (2, 3, 17, 64)
    assert not np.array_equal(a["do"], a["q"])
    b = inputs.generate(wl, ("do",))
    np.testing.assert_array_equal(a["do"], b["do"])
    np.testing.assert_array_equal(a["do"][1, 2], inputs.slab(wl.seed_words, "do", 1, 2, 17, 64, "bf16"))


def test_mask_generators():
    m = inputs.bool_mask(3, (2, 1, 50, 70), keep=0.6, empty_rows=4)
    assert m.dtype == np.uint8 and m.shape == (2, 1, 50, 70)
    assert np.all(m[0, 0, :4] == 0)
    assert abs(m[:, :, 4:].mean() - 0.6) < 0.03
    np.testing.assert_array_equal(m, inputs.bool_mask(3, (2, 1, 50, 70), keep=0.6, empty_rows=4))
    a = inputs.additive_mask(4, (1, 2, 40, 60), sigma=2.0, neg_inf=0.1)
    assert a.dtype == np.float32
    frac = np.isneginf(a).mean()
    assert 0.05 < frac < 0.15
    fin = a[np.isfinite(a)]
    assert abs(fin.std() - 2.0) < 0.15
    np.testing.assert_array_equal(a, inputs.additive_mask(4, (1, 2, 40, 60), sigma=2.0, neg_inf=0.1))
