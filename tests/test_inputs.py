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
