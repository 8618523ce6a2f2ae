"""Pins of the float64 CPU oracle against facts it does not compute itself.

Every test here runs on the CPU.  The pins are: the two-block worked example
of the comfyai.app chapter (values from closed forms, tests/golden), closed
forms and invariants of attention, SciPy's softmax/logsumexp on explicitly
built score matrices, brute force over every chunk partition for L <= 8
across the pages' recurrences, and a few planted mistakes that must fail.
"""

import itertools
import math
from pathlib import Path

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle

GOLDEN = Path(__file__).parent / "golden" / "worked_example_1234.txt"


def _golden():
    vals = {}
    for line in GOLDEN.read_text().splitlines():
        if line.startswith("#") or not line.strip():
            continue
        name, rest = line.split(":", 1)
        vals[name.strip()] = np.array([float(x) for x in rest.split()])
    return vals


def _attn1(a, vals=None):
    """Scores a as one attention query: q = [1], k_j = [a_j], scale 1."""
    a = np.asarray(a, dtype=np.float64)
    L = a.shape[0]
    q = np.ones((1, 1, 1, 1))
    k = a.reshape(1, 1, L, 1)
    if vals is None:
        vals = np.eye(L)
    D = vals.shape[1]
    # D must match for q and k; pad them with zero columns (no score change).
    qq = np.zeros((1, 1, 1, D)); qq[..., 0] = 1.0
    kk = np.zeros((1, 1, L, D)); kk[..., 0] = a
    return oracle.attention(qq, kk, vals.reshape(1, 1, L, D), 1.0)


# --------------------------------------------------------------------------
# Worked example: [1, 2, 3, 4] split as [1, 2] | [3, 4]
# --------------------------------------------------------------------------

def test_worked_example_materialised():
    g = _golden()
    O, L = _attn1([1, 2, 3, 4])
    np.testing.assert_allclose(O[0, 0, 0], g["O2"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(L[0, 0, 0], g["LSE"][0], rtol=1e-15)
    Os, _ = _attn1([1, 2, 3, 4], np.array([[1.0], [2.0], [3.0], [4.0]]))
    np.testing.assert_allclose(Os[0, 0, 0, 0], g["O_scalar_v"][0], rtol=1e-15)


def test_worked_example_recurrences():
    g = _golden()
    a = np.array([1.0, 2.0, 3.0, 4.0])
    # After the first chunk only.
    O1, d1, s1 = oracle.one_pass_chunked(a[:2], np.eye(4)[:2], [0, 2])
    assert d1 == g["d1"][0]
    np.testing.assert_allclose(s1, g["s1"][0], rtol=1e-15)
    np.testing.assert_allclose(O1, g["O1"], atol=1e-15)
    # Both chunks.
    O2, d2, s2 = oracle.one_pass_chunked(a, np.eye(4), [0, 2, 4])
    assert d2 == g["d2"][0]
    np.testing.assert_allclose(s2, g["s2"][0], rtol=1e-15)
    np.testing.assert_allclose(O2, g["O2"], atol=1e-15)
    np.testing.assert_allclose((s1 / s2) * math.exp(d1 - d2), g["correction"][0], rtol=1e-15)
    w, d, s = oracle.two_pass_chunked(a, [0, 2, 4])
    np.testing.assert_allclose(w, g["O2"], atol=1e-15)
    np.testing.assert_allclose(s, g["s2"][0], rtol=1e-15)
    sm, m, l, blocks = oracle.decoupled_softmax(a, [0, 2, 4])
    np.testing.assert_allclose(sm, g["O2"], atol=1e-15)
    np.testing.assert_allclose([b[0] for b in blocks], g["block_m"], rtol=0)
    np.testing.assert_allclose([b[1] for b in blocks], g["block_l"], rtol=1e-15)
    np.testing.assert_allclose(l, g["l_new"][0], rtol=1e-15)


# --------------------------------------------------------------------------
# Library cross-check: SciPy softmax / logsumexp on explicit score matrices
# --------------------------------------------------------------------------

@pytest.mark.parametrize("Lq,Lk,D,causal", [
    (1, 1, 4, False), (5, 7, 3, False), (7, 7, 8, True), (3, 9, 5, True),
    (16, 33, 16, False), (33, 33, 8, True), (1, 50, 6, True)])
def test_matches_scipy(Lq, Lk, D, causal):
    rng = np.random.default_rng(Lq * 1000 + Lk * 10 + D)
    B, H = 2, 3
    q = rng.standard_normal((B, H, Lq, D)) * 2
    k = rng.standard_normal((B, H, Lk, D))
    v = rng.standard_normal((B, H, Lk, D))
    scale = 0.7
    O, LSE = oracle.attention(q, k, v, scale, causal)
    for b in range(B):
        for h in range(H):
            a = np.empty((Lq, Lk))
            for i in range(Lq):
                for j in range(Lk):
                    a[i, j] = scale * sum(q[b, h, i, d] * k[b, h, j, d] for d in range(D))
                    if causal and j > i + (Lk - Lq):
                        a[i, j] = -np.inf
            np.testing.assert_allclose(O[b, h], softmax(a, axis=1) @ v[b, h], atol=1e-13)
            np.testing.assert_allclose(LSE[b, h], logsumexp(a, axis=1), atol=1e-13)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 2, 40, 8)) for _ in range(3))
    O, L = oracle.attention(q, k, v, 0.4, True)
    rows = np.array([0, 7, 39, 12])
    Os, Ls = oracle.attention(q, k, v, 0.4, True, rows=rows, row_block=3)
    np.testing.assert_allclose(Os, O[:, :, rows], atol=1e-15)
    np.testing.assert_allclose(Ls, L[:, :, rows], atol=1e-14)


# --------------------------------------------------------------------------
# Closed forms and invariants
# --------------------------------------------------------------------------

def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(4)
    L, D = 12, 6
    q = rng.standard_normal((1, 1, L, D))
    krow = rng.standard_normal(D)
    k = np.tile(krow, (1, 1, L, 1))
    v = rng.standard_normal((1, 1, L, D))
    O, LSE = oracle.attention(q, k, v, 0.3, False)
    np.testing.assert_allclose(O[0, 0], np.tile(v[0, 0].mean(axis=0), (L, 1)), atol=1e-14)
    a = 0.3 * q[0, 0] @ krow
    np.testing.assert_allclose(LSE[0, 0], a + math.log(L), atol=1e-13)
    # Causal: prefix means, LSE = a + ln(i + 1).
    Oc, Lc = oracle.attention(q, k, v, 0.3, True)
    pref = np.cumsum(v[0, 0], axis=0) / np.arange(1, L + 1)[:, None]
    np.testing.assert_allclose(Oc[0, 0], pref, atol=1e-14)
    np.testing.assert_allclose(Lc[0, 0], a + np.log(np.arange(1, L + 1)), atol=1e-13)


def test_permuting_keys_and_values_together():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 2, 9, 5))
    k = rng.standard_normal((2, 2, 14, 5))
    v = rng.standard_normal((2, 2, 14, 5))
    perm = rng.permutation(14)
    O, L = oracle.attention(q, k, v, 0.5)
    Op, Lp = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.5)
    np.testing.assert_allclose(Op, O, atol=1e-14)
    np.testing.assert_allclose(Lp, L, atol=1e-13)
    # Permuting only V must change the output (the weights pair with keys).
    Ox, _ = oracle.attention(q, k, v[:, :, perm], 0.5)
    assert np.max(np.abs(Ox - O)) > 1e-3


def test_constant_values_zero_scale_single_key():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, 2, 6, 4))
    k = rng.standard_normal((1, 2, 10, 4))
    v = np.full((1, 2, 10, 4), 2.5)
    O, _ = oracle.attention(q, k, v, 0.9, True)
    np.testing.assert_allclose(O, 2.5, atol=1e-14)
    v = rng.standard_normal((1, 2, 10, 4))
    O0, L0 = oracle.attention(q, k, v, 0.0, False)
    np.testing.assert_allclose(O0[0, 0], np.tile(v[0, 0].mean(axis=0), (6, 1)), atol=1e-14)
    np.testing.assert_allclose(L0, math.log(10), atol=1e-14)
    O1, L1 = oracle.attention(q, k[:, :, :1], v[:, :, :1], 0.9, False)
    np.testing.assert_allclose(O1, np.broadcast_to(v[:, :, :1], O1.shape), atol=1e-15)
    np.testing.assert_allclose(L1, 0.9 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0]), atol=1e-14)


def test_causal_rows():
    rng = np.random.default_rng(7)
    for Lq, Lk in [(11, 11), (5, 13)]:
        q = rng.standard_normal((1, 1, Lq, 4))
        k = rng.standard_normal((1, 1, Lk, 4))
        v = rng.standard_normal((1, 1, Lk, 4))
        O, L = oracle.attention(q, k, v, 0.8, True)
        off = Lk - Lq
        if off == 0:
            np.testing.assert_array_equal(O[0, 0, 0], v[0, 0, 0])
        for i in range(Lq):
            n = i + off + 1
            Oi, Li = oracle.attention(q[:, :, i:i + 1], k[:, :, :n], v[:, :, :n], 0.8, False)
            np.testing.assert_allclose(O[0, 0, i], Oi[0, 0, 0], atol=1e-14)
            np.testing.assert_allclose(L[0, 0, i], Li[0, 0, 0], atol=1e-13)
        # The last row sees every key: equals non-causal.
        On, Ln = oracle.attention(q, k, v, 0.8, False)
        np.testing.assert_allclose(O[0, 0, -1], On[0, 0, -1], atol=1e-14)


def test_key_shift_moves_lse_only():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 1, 7, 5))
    k = rng.standard_normal((1, 1, 9, 5))
    v = rng.standard_normal((1, 1, 9, 5))
    u = rng.standard_normal(5)
    O, L = oracle.attention(q, k, v, 0.6)
    O2, L2 = oracle.attention(q, k + u, v, 0.6)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(L2[0, 0], L[0, 0] + 0.6 * q[0, 0] @ u, atol=1e-13)


def test_identity_values_expose_weights():
    rng = np.random.default_rng(9)
    Lq, Lk = 6, 8
    q = rng.standard_normal((1, 1, Lq, Lk))
    k = rng.standard_normal((1, 1, Lk, Lk))
    v = np.eye(Lk).reshape(1, 1, Lk, Lk)
    O, _ = oracle.attention(q, k, v, 0.5, True)
    a = 0.5 * q[0, 0] @ k[0, 0].T
    a[np.arange(Lk)[None, :] > np.arange(Lq)[:, None] + 2] = -np.inf
    np.testing.assert_allclose(O[0, 0], softmax(a, axis=1), atol=1e-15)


def test_large_scores_do_not_overflow():
    # Scaled scores far above ln(FLT_MAX) ~ 88.7: safe softmax keeps them finite.
    q = np.zeros((1, 1, 1, 2)); q[..., 0] = 1.0
    k = np.zeros((1, 1, 3, 2)); k[0, 0, :, 0] = [500.0, 800.0, 799.0]
    v = np.arange(6, dtype=np.float64).reshape(1, 1, 3, 2)
    O, L = oracle.attention(q, k, v, 1.0)
    w = np.array([0.0, 1.0, math.exp(-1.0)]) / (1 + math.exp(-1.0))
    np.testing.assert_allclose(O[0, 0, 0], w @ v[0, 0], atol=1e-14)
    np.testing.assert_allclose(L[0, 0, 0], 800 + math.log(1 + math.exp(-1)), rtol=1e-15)


# --------------------------------------------------------------------------
# Brute force over every chunk partition, L <= 8
# --------------------------------------------------------------------------

def _compositions(L):
    for cuts in itertools.product([0, 1], repeat=L - 1):
        b = [0] + [i + 1 for i, c in enumerate(cuts) if c] + [L]
        yield b


def _patterns(L, rng):
    yield rng.standard_normal(L) * 3
    yield np.arange(L, dtype=np.float64)          # max jumps every chunk
    yield -np.arange(L, dtype=np.float64)         # max fixed by the first
    yield np.full(L, 0.25)                        # all equal
    x = rng.standard_normal(L); x[rng.integers(L)] = 60.0; yield x
    x = rng.standard_normal(L); x[rng.integers(L)] = -60.0; yield x


@pytest.mark.parametrize("L", range(1, 9))
def test_all_chunk_partitions_agree(L):
    rng = np.random.default_rng(100 + L)
    vals = rng.standard_normal((L, 3))
    for a in _patterns(L, rng):
        O_ref, LSE_ref = _attn1(a, vals)
        w_ref, _ = _attn1(a)
        O_ref, w_ref = O_ref[0, 0, 0], w_ref[0, 0, 0]
        for bounds in _compositions(L):
            w, d, s = oracle.two_pass_chunked(a, bounds)
            np.testing.assert_allclose(w, w_ref, rtol=1e-14, atol=1e-300)
            assert d == a.max()
            np.testing.assert_allclose(d + math.log(s), LSE_ref[0, 0, 0], rtol=1e-14, atol=1e-14)
            O, d1, s1 = oracle.one_pass_chunked(a, vals, bounds)
            np.testing.assert_allclose(O, O_ref, rtol=1e-13, atol=1e-14)
            sm, m, l, _ = oracle.decoupled_softmax(a, bounds)
            np.testing.assert_allclose(sm, w_ref, rtol=1e-14, atol=1e-300)
            np.testing.assert_allclose(l, s, rtol=1e-14)


def test_partitions_with_masked_entries():
    # A fully masked first chunk must not produce (-inf) - (-inf).
    a = np.array([-np.inf, -np.inf, 1.0, 3.0, -np.inf, 2.0])
    vals = np.arange(12, dtype=np.float64).reshape(6, 2)
    finite = np.isfinite(a)
    ref = softmax(a[finite])
    for bounds in _compositions(6):
        w, _, _ = oracle.two_pass_chunked(a, bounds)
        np.testing.assert_allclose(w[finite], ref, rtol=1e-14)
        assert np.all(w[~finite] == 0)
        O, _, _ = oracle.one_pass_chunked(a, vals, bounds)
        np.testing.assert_allclose(O, ref @ vals[finite], rtol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("br,bc", [(1, 1), (2, 3), (4, 4), (5, 2), (64, 64)])
def test_tiled_outer_kv_order(causal, br, bc):
    rng = np.random.default_rng(br * 10 + bc)
    Lq, Lk, D = (9, 13, 6) if not causal else (10, 13, 6)
    q = rng.standard_normal((Lq, D)) * 2
    k = rng.standard_normal((Lk, D))
    v = rng.standard_normal((Lk, D))
    O, L = oracle.tiled_outer_kv(q, k, v, 0.45, causal, br, bc)
    Or, Lr = oracle.attention(q[None, None], k[None, None], v[None, None], 0.45, causal)
    np.testing.assert_allclose(O, Or[0, 0], atol=1e-14)
    np.testing.assert_allclose(L, Lr[0, 0], atol=1e-13)


# --------------------------------------------------------------------------
# Planted mistakes: each must be caught by one of the pins above
# --------------------------------------------------------------------------

def _mutant_strict_mask(rows, Lq, Lk, causal):
    j = np.arange(Lk)[None, :]
    if not causal:
        return np.ones((rows.shape[0], Lk), dtype=bool)
    return j < (rows[:, None] + (Lk - Lq))  # off by one: the diagonal is dropped


def _mutant_top_left_mask(rows, Lq, Lk, causal):
    j = np.arange(Lk)[None, :]
    if not causal:
        return np.ones((rows.shape[0], Lk), dtype=bool)
    return j <= rows[:, None]  # top-left alignment


def test_planted_mask_mistakes_are_caught(monkeypatch):
    import sys
    mod = sys.modules["oracle.attention"]
    for mutant in (_mutant_strict_mask, _mutant_top_left_mask):
        monkeypatch.setattr(mod, "_allowed_keys", mutant)
        with pytest.raises((AssertionError, FloatingPointError, ValueError)):
            with np.errstate(invalid="ignore", divide="ignore"):
                test_causal_rows()
                test_matches_scipy(3, 9, 5, True)
        monkeypatch.undo()
    test_causal_rows()


def test_planted_transpose_is_caught():
    # Swapping the roles of q and k (a transposed operand) changes the result
    # of a non-square problem; the SciPy pin would see it.
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 1, 6, 4))
    k = rng.standard_normal((1, 1, 6, 4))
    v = rng.standard_normal((1, 1, 6, 4))
    O, _ = oracle.attention(q, k, v, 0.5)
    Ot, _ = oracle.attention(k, q, v, 0.5)
    assert np.max(np.abs(O - Ot)) > 1e-3


# --------------------------------------------------------------------------
# Decode over caches with per-sequence lengths
# --------------------------------------------------------------------------

def test_decode_varlen_full_lengths_equal_attention():
    rng = np.random.default_rng(91)
    q = rng.standard_normal((3, 2, 1, 16))
    k = rng.standard_normal((3, 2, 40, 16))
    v = rng.standard_normal((3, 2, 40, 16))
    O, L = oracle.decode_varlen(q, k, v, [40, 40, 40], 0.3)
    Or, Lr = oracle.attention(q, k, v, 0.3)
    np.testing.assert_array_equal(O, Or)
    np.testing.assert_array_equal(L, Lr)


def test_decode_varlen_ignores_rows_past_length():
    """Rows past a sequence's length (here NaN and huge) change nothing, and
    a sequence equals plain attention over its own keys (SciPy on the
    explicit score row)."""
    rng = np.random.default_rng(92)
    B, H, Lk, D = 4, 2, 50, 8
    q = rng.standard_normal((B, H, 1, D))
    k = rng.standard_normal((B, H, Lk, D))
    v = rng.standard_normal((B, H, Lk, D))
    lens = [1, 17, 50, 33]
    k2, v2 = k.copy(), v.copy()
    for b, n in enumerate(lens):
        k2[b, :, n:] = np.nan
        v2[b, :, n:] = 1e30
    O, L = oracle.decode_varlen(q, k2, v2, lens, 0.5)
    for b, n in enumerate(lens):
        for h in range(H):
            a = 0.5 * (k[b, h, :n] @ q[b, h, 0])
            np.testing.assert_allclose(O[b, h, 0], softmax(a) @ v[b, h, :n], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(L[b, h, 0], logsumexp(a), rtol=1e-13)
    # length 1: the only value row, the only score
    np.testing.assert_allclose(O[0, :, 0], v[0, :, 0], rtol=1e-15)
    np.testing.assert_allclose(L[0, :, 0], 0.5 * np.einsum("hd,hd->h", q[0, :, 0], k[0, :, 0]), rtol=1e-14)


def test_decode_varlen_empty_and_clamped_lengths():
    rng = np.random.default_rng(93)
    q = rng.standard_normal((3, 1, 1, 8))
    k = rng.standard_normal((3, 1, 10, 8))
    v = rng.standard_normal((3, 1, 10, 8))
    O, L = oracle.decode_varlen(q, k, v, [0, -4, 99], 1.0)
    assert np.all(O[:2] == 0) and np.all(np.isneginf(L[:2]))
    Or, Lr = oracle.attention(q[2:], k[2:], v[2:], 1.0)
    np.testing.assert_array_equal(O[2:], Or)
    np.testing.assert_array_equal(L[2:], Lr)
