"""Pins of the masked / dropout oracle (``attention_ex``, ``attention_ex_bwd``)
and of its counter-based generator (``oracle/philox.py``).  CPU only.

* Philox: the 32-bit instance equals the published Philox4x32-10
  known-answer vectors (``tests/golden/philox4x32_10_kat.txt``); the round
  structure and key schedule, run at 64-bit width, equal NumPy's
  Philox4x64-10 bit generator block for block; the vectorised
  32-bit evaluation equals the scalar one; the 32-bit words are uniform
  (mean, per-bit frequencies) and a one-bit change of the counter flips
  about half of the output bits.
* Keep pattern: rate 1 - p within binomial bounds, p = 0 keeps everything,
  rows are independent of which other rows are asked for, offsets and
  seeds change the pattern.
* Forward: no mask and p = 0 is ``attention``; a boolean mask equals plain
  attention over the kept keys (SciPy softmax on the explicit scores); an
  additive mask equals SciPy's softmax of the biased scores; a per-row
  constant bias changes nothing; -inf equals a false boolean; rows with no
  key give O = 0 and LSE = -inf; dropout equals (P o Z) V / (1 - p) with P
  from SciPy.
* Backward: central finite differences of the forward (mask and dropout
  fixed), float64 autograd through an explicit masked, dropped-out softmax,
  and the plain backward when nothing is masked or dropped.
"""

import sys
from pathlib import Path

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle
from oracle import philox as ph

oa = sys.modules["oracle.attention"]
_KEEP = ph.keep_pattern  # the pins use this reference, never a patched one


# ---------------------------------------------------------------- Philox --

KAT = Path(__file__).parent / "golden" / "philox4x32_10_kat.txt"


def _kat_rows():
    rows = []
    for line in KAT.read_text().splitlines():
        if line.startswith("#") or not line.strip():
            continue
        lhs, rhs = line.split(":")
        rows.append(([int(w, 16) for w in lhs.split()], [int(w, 16) for w in rhs.split()]))
    return rows


def test_philox32_known_answers():
    """The 32-bit instance (multipliers, Weyl constants, round structure)
    against the published Philox4x32-10 known-answer vectors, through both
    the scalar and the vectorised form."""
    rows = _kat_rows()
    assert len(rows) == 3
    for words, expect in rows:
        ctr, key = words[:4], words[4:]
        assert [int(x) for x in ph.philox4x32(*ctr, *key)] == expect, words
        assert ph.philox(ctr, key, 32, ph.M4x32, ph.W4x32) == expect, words


def test_keep_pattern_reads_the_known_answer_words():
    """keep_pattern takes, for key j, the 16-bit half (j mod 2; low half
    first) of word ((j mod 8) / 2) of the block with counter
    (j / 8, i, bh, offset) and key (seed low, seed high): with the all-zero
    KAT counter and key (block 0 of row 0, bh 0, offset 0, seed 0) keys
    0 .. 7 see exactly the halves of that vector's four words, in order."""
    words, expect = _kat_rows()[0]
    assert words == [0] * 6
    halves = [h for w in expect for h in (w & 0xFFFF, w >> 16)]
    assert len(halves) == 8
    for x in halves:
        # p just above x / 2^16: halves <= x are dropped, larger ones kept.
        p = float(np.nextafter(np.float32((x + 0.5) / 2.0 ** 16), np.float32(1.0)))
        thr = ph.dropout_threshold(p)
        assert thr == x
        keep = ph.keep_pattern(0, 0, 0, [0], 8, p)[0]
        assert list(keep) == [y >= thr for y in halves]
        assert keep[halves.index(x)]  # a half equal to the threshold is kept
    # the eight thresholds keep eight different numbers of keys: every case
    # tells the halves apart
    assert len({sum(y >= x for y in halves) for x in halves}) == len(set(halves)) == 8


@pytest.mark.parametrize("key", [(1, 2), (0, 0), (0xDEADBEEFCAFEF00D, 0x0123456789ABCDEF)])
def test_philox64_matches_numpy(key):
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array([7, 0, 0, 0], dtype=np.uint64))
    raw = bg.random_raw(4 * 5)
    for blk in range(5):
        # NumPy increments the counter before producing a block.
        ours = ph.philox4x64([8 + blk, 0, 0, 0], key)
        assert [int(x) for x in raw[4 * blk:4 * blk + 4]] == ours


def test_philox64_high_counter_words_match_numpy():
    ctr = [0xFFFFFFFFFFFFFFFE, 5, 9, 11]
    bg = np.random.Philox(key=np.array([3, 4], dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
    raw = bg.random_raw(8)
    assert [int(x) for x in raw[:4]] == ph.philox4x64([0xFFFFFFFFFFFFFFFF, 5, 9, 11], (3, 4))
    # carry into the second word
    assert [int(x) for x in raw[4:]] == ph.philox4x64([0, 6, 9, 11], (3, 4))


def test_philox32_vector_equals_scalar():
    rng = np.random.default_rng(5)
    for _ in range(20):
        c = [int(x) for x in rng.integers(0, 2 ** 32, 4)]
        k = [int(x) for x in rng.integers(0, 2 ** 32, 2)]
        vec = ph.philox4x32(*c, *k)
        assert [int(x) for x in vec] == ph.philox(c, k, 32, ph.M4x32, ph.W4x32)


def test_philox32_statistics():
    n = 1 << 16
    c0 = np.arange(n, dtype=np.uint64)
    words = np.concatenate(ph.philox4x32(c0, 3, 17, 0, 12345, 678))
    u = words.astype(np.float64) / 2 ** 32
    assert abs(u.mean() - 0.5) < 4 * np.sqrt(1 / 12 / u.size)
    bits = (words[:, None] >> np.arange(32, dtype=np.uint64)[None, :]) & np.uint64(1)
    freq = bits.mean(axis=0)
    assert np.all(np.abs(freq - 0.5) < 5 * 0.5 / np.sqrt(words.size))
    # avalanche: flipping bit b of counter word 1 flips about half the bits
    base = ph.philox4x32(c0[:4096], 3, 17, 0, 12345, 678)
    for b in (0, 13, 31):
        flip = ph.philox4x32(c0[:4096], 3 ^ (1 << b), 17, 0, 12345, 678)
        d = np.concatenate([x ^ y for x, y in zip(base, flip)])
        pop = np.unpackbits(d.astype(np.uint32).view(np.uint8)).mean()
        assert abs(pop - 0.5) < 0.01


def test_philox32_rounds_matter():
    a = ph.philox4x32(1, 2, 3, 4, 5, 6)
    b = ph.philox4x32(1, 2, 3, 4, 5, 6, rounds=9)
    assert any(int(x) != int(y) for x, y in zip(a, b))


# ---------------------------------------------------------- keep pattern --

@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_rate(p):
    z = ph.keep_pattern(77, 3, 5, np.arange(512), 512, p)
    n = z.size
    assert abs(z.mean() - (1 - p)) < 5 * np.sqrt(p * (1 - p) / n)


def test_keep_pattern_properties():
    full = ph.keep_pattern(1, 0, 2, np.arange(100), 333, 0.3)
    rows = np.array([99, 0, 41])
    np.testing.assert_array_equal(ph.keep_pattern(1, 0, 2, rows, 333, 0.3), full[rows])
    assert ph.keep_pattern(1, 0, 2, np.arange(100), 333, 0.0).all()
    other = [ph.keep_pattern(1, 1, 2, np.arange(100), 333, 0.3), ph.keep_pattern(2, 0, 2, np.arange(100), 333, 0.3),
             ph.keep_pattern(1, 0, 3, np.arange(100), 333, 0.3)]
    for o in other:
        assert (o != full).mean() > 0.3
    assert ph.dropout_threshold(0.5) == 2 ** 15
    assert ph.dropout_threshold(0.0) == 0
    assert ph.dropout_threshold(float(np.nextafter(np.float32(1.0), np.float32(0.0)))) == 0xFFFF
    with pytest.raises(ValueError):
        ph.dropout_threshold(1.0)


# --------------------------------------------------------------- forward --

def _qkv(seed, B, H, Lq, Lk, D):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, Lq, D)), rng.standard_normal((B, H, Lk, D)),
            rng.standard_normal((B, H, Lk, D)), rng)


@pytest.mark.parametrize("causal", [False, True])
def test_no_mask_no_dropout_is_attention(causal):
    q, k, v, _ = _qkv(1, 2, 3, 20, 30, 8)
    O, L = oracle.attention_ex(q, k, v, 0.4, causal)
    Or, Lr = oracle.attention(q, k, v, 0.4, causal)
    np.testing.assert_allclose(O, Or, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(L, Lr, rtol=1e-14)


def test_bool_mask_is_attention_over_kept_keys():
    q, k, v, rng = _qkv(2, 2, 3, 12, 25, 8)
    mask = rng.random((2, 1, 12, 25)) < 0.6
    mask[0, 0, 3] = False  # a row with no key
    O, L = oracle.attention_ex(q, k, v, 0.7, False, mask.astype(np.uint8), "bool")
    for b in range(2):
        for h in range(3):
            for i in range(12):
                sel = mask[b, 0, i]
                if not sel.any():
                    assert np.all(O[b, h, i] == 0) and np.isneginf(L[b, h, i])
                    continue
                a = 0.7 * (k[b, h, sel] @ q[b, h, i])
                np.testing.assert_allclose(O[b, h, i], softmax(a) @ v[b, h, sel], rtol=1e-12, atol=1e-14)
                np.testing.assert_allclose(L[b, h, i], logsumexp(a), rtol=1e-13)


def test_additive_mask_is_softmax_of_biased_scores():
    q, k, v, rng = _qkv(3, 1, 4, 9, 17, 8)
    add = rng.standard_normal((1, 4, 9, 17)).astype(np.float32) * 3
    add[0, 1, :, 5] = -np.inf
    O, L = oracle.attention_ex(q, k, v, 0.5, True, add, "add")
    off = 17 - 9
    for h in range(4):
        for i in range(9):
            a = 0.5 * (k[0, h] @ q[0, h, i]) + add[0, h, i].astype(np.float64)
            a[np.arange(17) > i + off] = -np.inf
            np.testing.assert_allclose(O[0, h, i], softmax(a) @ v[0, h], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(L[0, h, i], logsumexp(a), rtol=1e-13)


def test_additive_mask_invariances():
    q, k, v, rng = _qkv(4, 2, 2, 10, 14, 4)
    row_const = np.broadcast_to(rng.standard_normal((2, 2, 10, 1)), (2, 2, 10, 14))
    O, L = oracle.attention_ex(q, k, v, 0.3, False, row_const, "add")
    Or, Lr = oracle.attention(q, k, v, 0.3)
    np.testing.assert_allclose(O, Or, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L - Lr, row_const[..., 0], rtol=1e-12, atol=1e-12)
    keep = rng.random((1, 1, 10, 14)) < 0.5
    keep[..., 0] = True
    Ob, Lb = oracle.attention_ex(q, k, v, 0.3, False, keep.astype(np.uint8), "bool")
    Oa, La = oracle.attention_ex(q, k, v, 0.3, False, np.where(keep, 0.0, -np.inf), "add")
    np.testing.assert_allclose(Ob, Oa, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(Lb, La, rtol=1e-14)


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout_forward_formula(p):
    q, k, v, rng = _qkv(5, 2, 2, 16, 21, 8)
    O, L = oracle.attention_ex(q, k, v, 0.6, True, dropout_p=p, seed=99, offset=4)
    Or, Lr = oracle.attention(q, k, v, 0.6, True)
    np.testing.assert_allclose(L, Lr, rtol=1e-14)  # LSE ignores dropout
    off = 21 - 16
    for b in range(2):
        for h in range(2):
            z = _KEEP(99, 4, b * 2 + h, np.arange(16), 21, p)
            a = 0.6 * (q[b, h] @ k[b, h].T)
            a[np.arange(21)[None, :] > np.arange(16)[:, None] + off] = -np.inf
            P = softmax(a, axis=1)
            np.testing.assert_allclose(O[b, h], (P * z / (1 - float(np.float32(p)))) @ v[b, h], rtol=1e-12, atol=1e-14)


# -------------------------------------------------------------- backward --

def _fd(f, x, eps=1e-6):
    g = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += eps
        xm[idx] -= eps
        g[idx] = (f(xp) - f(xm)) / (2 * eps)
    return g


@pytest.mark.parametrize("kind,p,causal", [("bool", 0.0, False), ("add", 0.0, True), (None, 0.4, True),
                                           ("bool", 0.3, True), ("add", 0.5, False)])
def test_backward_finite_differences(kind, p, causal):
    q, k, v, rng = _qkv(6, 1, 2, 5, 7, 3)
    do = rng.standard_normal(q.shape)
    mask = None
    if kind == "bool":
        mask = (rng.random((1, 2, 5, 7)) < 0.7).astype(np.uint8)
        mask[..., 0] = 1
    elif kind == "add":
        mask = rng.standard_normal((1, 1, 5, 7))
    kw = dict(mask=mask, mask_kind=kind, dropout_p=p, seed=3, offset=1)
    got = oracle.attention_ex_bwd(q, k, v, do, 0.8, causal, **kw)

    def loss(qq, kk, vv):
        return float((oracle.attention_ex(qq, kk, vv, 0.8, causal, **kw)[0] * do).sum())
    ref = (_fd(lambda x: loss(x, k, v), q), _fd(lambda x: loss(q, x, v), k), _fd(lambda x: loss(q, k, x), v))
    for name, g, r in zip("qkv", got, ref):
        assert np.max(np.abs(g - r)) <= 1e-7 * max(1.0, np.max(np.abs(r))), name


def test_backward_autograd_explicit():
    q, k, v, rng = _qkv(7, 2, 2, 24, 30, 8)
    do = rng.standard_normal(q.shape)
    add = rng.standard_normal((2, 1, 24, 30))
    add[0, 0, :, 3] = -np.inf
    p = 0.25
    got = oracle.attention_ex_bwd(q, k, v, do, 0.45, True, add, "add", p, 11, 2)
    t = [torch.tensor(x, requires_grad=True) for x in (q, k, v)]
    a = 0.45 * t[0] @ t[1].transpose(-1, -2) + torch.tensor(add)
    i = torch.arange(24)[:, None]
    j = torch.arange(30)[None, :]
    a = a.masked_fill(j - i > 30 - 24, float("-inf"))
    P = torch.softmax(a, dim=-1)
    Z = torch.tensor(np.stack([np.stack([_KEEP(11, 2, b * 2 + h, np.arange(24), 30, p) for h in range(2)])
                               for b in range(2)]).astype(np.float64))
    O = (P * Z / (1 - float(np.float32(p)))) @ t[2]
    O.backward(torch.tensor(do))
    for name, g, tt in zip("qkv", got, t):
        np.testing.assert_allclose(g, tt.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_backward_plain_case_is_attention_bwd():
    q, k, v, rng = _qkv(8, 1, 2, 13, 19, 4)
    do = rng.standard_normal(q.shape)
    a = oracle.attention_ex_bwd(q, k, v, do, 0.5, True)
    b = oracle.attention_bwd(q, k, v, do, 0.5, True)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)


def test_planted_dropout_scale_mistake(monkeypatch):
    """The forward formula pin notices a keep pattern used without 1/(1-p)."""
    real = ph.keep_pattern
    monkeypatch.setattr(ph, "keep_pattern", lambda *a: real(*a) * (1 - float(np.float32(a[-1]))))
    with pytest.raises(AssertionError):
        test_dropout_forward_formula(0.5)
