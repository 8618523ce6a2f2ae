"""Pins of the float64 backward oracle (``oracle.attention_bwd``).

All on the CPU.  The pins do not reuse the oracle's backward arithmetic:

* central finite differences of the forward oracle's loss sum(dO * O), entry
  by entry, on tiny causal and non-causal problems;
* torch.autograd in float64 through a softmax attention written here with
  its own causal mask;
* closed forms: a single key (weights 1: dV is the sum of dO, dQ = dK = 0),
  zero queries (uniform weights: dV_j is the mean of dO, dK = 0 and
  dQ_i = (scale / Lk) sum_j (dO_i . v_j)(k_j - mean k));
* invariants: the key gradients of one row sum to zero (shifting every key
  by one vector leaves the softmax unchanged), linearity in dO;
* row subsets equal the matching rows of the full result;
* planted mistakes in the oracle (a dropped term, a wrong sign, swapped or
  transposed operands, a missing scale) fail the finite-difference pin.
"""

import sys

import numpy as np
import pytest
import torch

import oracle

# The package re-exports the function ``attention`` under the submodule's name.
oa = sys.modules["oracle.attention"]


def _rand(seed, B, H, Lq, Lk, D):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, Lq, D)), rng.standard_normal((B, H, Lk, D)),
            rng.standard_normal((B, H, Lk, D)), rng.standard_normal((B, H, Lq, D)))


def _fd_grads(q, k, v, do, scale, causal, eps=1e-6):
    """Central differences of sum(do * attention(q, k, v)) entry by entry."""
    def loss(**a):
        return float((oracle.attention(a["q"], a["k"], a["v"], scale, causal, check=False)[0] * do).sum())
    base = {"q": q, "k": k, "v": v}
    out = {}
    for name, x in base.items():
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            g[idx] = (loss(**{**base, name: xp}) - loss(**{**base, name: xm})) / (2 * eps)
        out[name] = g
    return out["q"], out["k"], out["v"]


def _check_fd(Lq, Lk, causal, seed=1, scale=0.7):
    q, k, v, do = _rand(seed, 1, 2, Lq, Lk, 3)
    got = oracle.attention_bwd(q, k, v, do, scale, causal)
    ref = _fd_grads(q, k, v, do, scale, causal)
    for name, g, r in zip("qkv", got, ref):
        err = np.max(np.abs(g - r))
        assert err <= 1e-7 * max(1.0, np.max(np.abs(r))), f"d{name}: {err}"


@pytest.mark.parametrize("Lq,Lk,causal", [(5, 7, False), (7, 4, False), (5, 7, True), (6, 6, True), (1, 5, True)])
def test_finite_differences(Lq, Lk, causal):
    _check_fd(Lq, Lk, causal)


def _torch_grads(q, k, v, do, scale, causal):
    """float64 autograd through softmax(scale q k^T + mask) v; the mask is
    built here from the bottom-right rule, key j visible to query i iff
    j - i <= Lk - Lq."""
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    Lq, Lk = q.shape[2], k.shape[2]
    a = scale * torch.matmul(t[0], t[1].transpose(-1, -2))
    if causal:
        i = torch.arange(Lq)[:, None]
        j = torch.arange(Lk)[None, :]
        a = a.masked_fill(j - i > Lk - Lq, float("-inf"))
    o = torch.matmul(torch.softmax(a, dim=-1), t[2])
    o.backward(torch.tensor(do, dtype=torch.float64))
    return [x.grad.numpy() for x in t]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lq,Lk", [(33, 40), (64, 64), (17, 100)])
def test_torch_autograd(Lq, Lk, causal):
    q, k, v, do = _rand(Lq + Lk, 2, 3, Lq, Lk, 8)
    got = oracle.attention_bwd(q, k, v, do, 0.35, causal)
    ref = _torch_grads(q, k, v, do, 0.35, causal)
    for name, g, r in zip("qkv", got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12, err_msg=f"d{name}")


def test_one_key():
    q, k, v, do = _rand(3, 2, 2, 9, 1, 5)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 1.3, False)
    np.testing.assert_allclose(dv[:, :, 0], do.sum(axis=2), rtol=1e-14, atol=1e-14)
    assert np.max(np.abs(dq)) < 1e-14 and np.max(np.abs(dk)) < 1e-14


def test_uniform_weights_closed_form():
    _, k, v, do = _rand(4, 1, 2, 6, 11, 4)
    q = np.zeros((1, 2, 6, 4))
    scale = 0.9
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, False)
    Lk = k.shape[2]
    np.testing.assert_allclose(dv, np.broadcast_to(do.sum(axis=2, keepdims=True) / Lk, dv.shape), rtol=1e-13)
    assert np.max(np.abs(dk)) < 1e-14
    for h in range(2):
        kc = k[0, h] - k[0, h].mean(axis=0)
        ref = np.array([(scale / Lk) * sum((do[0, h, i] @ v[0, h, j]) * kc[j] for j in range(Lk))
                        for i in range(6)])
        np.testing.assert_allclose(dq[0, h], ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(causal):
    q, k, v, do = _rand(5, 2, 2, 20, 30, 6)
    _, dk, _ = oracle.attention_bwd(q, k, v, do, 0.6, causal)
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-12 * max(1.0, np.max(np.abs(dk)))


def test_linear_in_upstream_gradient():
    q, k, v, do = _rand(6, 1, 2, 12, 12, 4)
    do2 = np.random.default_rng(60).standard_normal(do.shape)
    g1 = oracle.attention_bwd(q, k, v, do, 0.5, True)
    g2 = oracle.attention_bwd(q, k, v, do2, 0.5, True)
    g3 = oracle.attention_bwd(q, k, v, 2.0 * do - 3.0 * do2, 0.5, True)
    for a, b, c in zip(g1, g2, g3):
        np.testing.assert_allclose(c, 2.0 * a - 3.0 * b, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_row_subsets(causal):
    q, k, v, do = _rand(7, 1, 2, 50, 70, 8)
    full = oracle.attention_bwd(q, k, v, do, 0.4, causal, row_block=16)
    qr = np.array([49, 0, 17, 33])
    kr = np.array([69, 3, 0, 40])
    dq, _, _ = oracle.attention_bwd(q, k, v, do, 0.4, causal, q_rows=qr, k_rows=[], row_block=3)
    _, dk, dv = oracle.attention_bwd(q, k, v, do, 0.4, causal, q_rows=qr, k_rows=kr, row_block=7)
    np.testing.assert_allclose(dq, full[0][:, :, qr], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dk, full[1][:, :, kr], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(dv, full[2][:, :, kr], rtol=1e-13, atol=1e-15)


def _vjp_dropped_term(p, dp):
    return p * dp


def _vjp_wrong_sign(p, dp):
    return p * (dp + (p * dp).sum(axis=1, keepdims=True))


def _grads_keys_from_upstream(p, da, qq, kk, g, scale):
    return p.T @ g, scale * (da.T @ g), scale * (da @ kk)


def _grads_values_from_vjp(p, da, qq, kk, g, scale):
    return da.T @ g, scale * (da.T @ qq), scale * (da @ kk)


def _grads_missing_scale(p, da, qq, kk, g, scale):
    return p.T @ g, da.T @ qq, scale * (da @ kk)


def _mask_one_short(rows, Lq, Lk, causal):
    j = np.arange(Lk)[None, :]
    if not causal:
        return np.ones((rows.shape[0], Lk), dtype=bool)
    return j < (rows[:, None] + (Lk - Lq))


@pytest.mark.parametrize("name,mutant", [
    ("_softmax_vjp", _vjp_dropped_term),
    ("_softmax_vjp", _vjp_wrong_sign),
    ("_score_grads", _grads_keys_from_upstream),
    ("_score_grads", _grads_values_from_vjp),
    ("_score_grads", _grads_missing_scale),
])
def test_planted_mistakes_fail_finite_differences(name, mutant, monkeypatch):
    monkeypatch.setattr(oa, name, mutant)
    with pytest.raises(AssertionError):
        _check_fd(5, 7, True)


def test_planted_mask_mistake_fails_autograd(monkeypatch):
    """An off-by-one causal mask would move forward and backward together
    (finite differences agree with it); the autograd pin builds its own mask."""
    monkeypatch.setattr(oa, "_allowed_keys", _mask_one_short)
    with pytest.raises(AssertionError):
        test_torch_autograd(33, 40, True)
