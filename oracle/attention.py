"""Float64 host implementations of attention and of the pages' softmax recurrences.

Test infrastructure only (see the package docstring): nothing on the product
path may import this module.

``attention`` is the oracle proper.  The pages state that the tiled one-pass
method reaches exactly the result of standard attention ("identical" /
"exactly the same" in the quidproquo.cc guide's TL;DR and "The scene"
section; "mathematically equivalent" in the comfyai.app chapter's
introduction), so the oracle is that plain definition written out: it
materialises every score, subtracts the row maximum, exponentiates, sums,
divides and only then takes the weighted sum of the values.

The other functions are independent evaluations of the same quantities that
follow the pages' recurrences step by step.  They exist to pin ``attention``
and each other in the CPU test tier; none of them shares arithmetic with the
GPU kernels.

Conventions (readings of points the pages leave open):

* scores are ``a_ij = scale * (q_i . k_j)``; the guide writes the plain dot
  product (slides 3-4) and the comfyai chapter names a "scale" step of the
  fused tile without a surviving formula;
* causal masking is aligned to the bottom-right corner: query ``i`` of ``Lq``
  may see key ``j`` of ``Lk`` iff ``j <= i + (Lk - Lq)``; masked scores are
  minus infinity, so they drop out of both the maximum and the sum;
* the log-sum-exp returned per row is ``m + ln(s)`` in natural-log units of
  the scaled scores, where ``m`` is the row maximum and ``s`` the
  denominator.
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

__all__ = [
    "attention",
    "attention_bwd",
    "attention_ex",
    "attention_ex_bwd",
    "decode_varlen",
    "two_pass_chunked",
    "one_pass_chunked",
    "decoupled_softmax",
    "tiled_outer_kv",
]


def _allowed_keys(rows: np.ndarray, Lq: int, Lk: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), Lk] mask of the keys each query row may attend to."""
    j = np.arange(Lk)[None, :]
    if not causal:
        return np.ones((rows.shape[0], Lk), dtype=bool)
    return j <= (rows[:, None] + (Lk - Lq))


def attention(q, k, v, scale: float, causal: bool = False, rows=None,
              row_block: int = 1024, check: bool = True):
    """Exact attention forward, materialised, in float64.

    Follows standard attention as both pages describe it: the guide's
    self-attention review (slides 3-4: dot products ``a_i``, softmax to
    ``a^_i``, weighted sum of ``v_i``) with the "subtract Amax before taking
    the exponential" step of its naive multi-pass walk-through (slides 11-17),
    which the comfyai chapter calls safe softmax (section 6.3.2).

    Args:
      q: [B, H, Lq, D] array of any real float dtype (upcast exactly).
      k, v: [B, H, Lk, D].
      scale: multiplier applied to every dot product before the softmax.
      causal: bottom-right aligned causal mask (requires Lq <= Lk).
      rows: optional 1-D integer array of query rows to evaluate; the result
        then has ``len(rows)`` rows in that order.
      row_block: rows per materialised score block (bounds host memory).
      check: run the internal consistency checks listed below.

    Returns:
      (O, LSE): O is [B, H, R, D] float64 and LSE is [B, H, R] float64,
      with R = Lq or len(rows).

    Internal checks (``check=True``): every weight row sums to one within
    1e-13; ``m <= LSE <= m + ln(#allowed keys)``; each output element lies in
    the range of the value column it averages (a convex combination).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, L, D]")
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    if k.shape != (B, H, Lk, D) or v.shape != (B, H, Lk, D):
        raise ValueError("k and v must be [B, H, Lk, D] matching q")
    if causal and Lq > Lk:
        raise ValueError("causal attention needs Lq <= Lk")
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    O = np.zeros((B, H, R, D), dtype=np.float64)
    LSE = np.zeros((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kk = k[b, h].astype(np.float64)
            vv = v[b, h].astype(np.float64)
            for r0 in range(0, R, row_block):
                rr = rows[r0:r0 + row_block]
                qq = q[b, h, rr].astype(np.float64)
                # Scores a_ij = scale * q_i . k_j for every key.
                a = scale * (qq @ kk.T)
                allowed = _allowed_keys(rr, Lq, Lk, causal)
                a = np.where(allowed, a, -np.inf)
                # Pass 1: the row maximum Amax.
                m = a.max(axis=1)
                # Pass 2: exp(a_i - Amax) (masked entries become exactly 0).
                e = np.exp(a - m[:, None])
                # Pass 3: the denominator.
                s = e.sum(axis=1)
                # Pass 4: the weights a^_i.
                p = e / s[:, None]
                # Pass 5: the weighted sum of the values.
                o = p @ vv
                O[b, h, r0:r0 + len(rr)] = o
                LSE[b, h, r0:r0 + len(rr)] = m + np.log(s)
                if check:
                    _check_block(p, o, m, m + np.log(s), allowed, vv)
    return O, LSE


def decode_varlen(q, k, v, seqlens, scale: float):
    """Single-query attention over caches with per-sequence lengths, float64.

    The decode step of the guide's prefill/decode split (slide 5) over a key
    cache: query ``q[b, h, 0]`` attends to the first ``seqlens[b]`` keys of
    ``k[b, h]`` and nothing else.  Each sequence is the plain definition
    (``attention`` on the sliced keys).  Readings of the interface: a length
    is clamped to ``[0, Lk]``; a sequence with no key gets O = 0 and
    LSE = -inf (the empty sum).

    Args:
      q: [B, H, 1, D]; k, v: [B, H, Lk, D]; seqlens: B integers.
    Returns:
      (O [B, H, 1, D], LSE [B, H, 1]) in float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, Lq, D = q.shape
    if Lq != 1:
        raise ValueError("decode_varlen takes one query per (batch, head)")
    Lk = k.shape[2]
    lens = np.clip(np.asarray(seqlens, dtype=np.int64).reshape(B), 0, Lk)
    O = np.zeros((B, H, 1, D), dtype=np.float64)
    LSE = np.full((B, H, 1), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        O[b:b + 1], LSE[b:b + 1] = attention(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], scale)
    return O, LSE


def attention_bwd(q, k, v, do, scale: float, causal: bool = False, q_rows=None, k_rows=None,
                  row_block: int = 1024):
    """Gradients of exact attention with respect to q, k and v, in float64.

    The comfyai.app chapter "6.3 FlashAttention" states (after its "A simple
    implementation w/ C++" part, and again in "Computation and GPU Memory")
    that the training backward pass keeps no score or weight matrix from the
    forward and recomputes what it needs instead, at a cost of the same
    order as the forward.  The pages give no backward formulas, so this is
    the plain derivative of the forward's definition (``attention``) for an
    upstream gradient ``do`` of O, written out with every matrix
    materialised:

      a  = scale * q k^T, masked entries -inf     (the forward's scores)
      P  = softmax of each row of a               (the forward's weights)
      dV = P^T dO
      dP = dO V^T
      dA_ij = P_ij (dP_ij - sum_l P_il dP_il)      (Jacobian of the softmax)
      dQ = scale * dA K,    dK = scale * dA^T Q

    Masked entries have P = 0 and so contribute nothing.  No gradient flows
    into LSE (it is treated as an output nobody differentiates).

    Args:
      q, do: [B, H, Lq, D]; k, v: [B, H, Lk, D]; any real float dtypes.
      scale, causal: as for ``attention``.
      q_rows: optional query rows whose dQ is returned (all keys are used).
      k_rows: optional key rows whose dK, dV are returned (all queries are
        used; every row of the weights is still computed in full).
      row_block: query rows per materialised block.

    Returns:
      (dQ [B, H, Rq, D], dK [B, H, Rk, D], dV [B, H, Rk, D]) in float64.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    if do.shape != q.shape or k.shape != (B, H, Lk, D) or v.shape != (B, H, Lk, D):
        raise ValueError("q, do must be [B, H, Lq, D]; k, v [B, H, Lk, D]")
    if causal and Lq > Lk:
        raise ValueError("causal attention needs Lq <= Lk")
    q_rows = np.arange(Lq) if q_rows is None else np.asarray(q_rows, dtype=np.int64)
    k_rows = np.arange(Lk) if k_rows is None else np.asarray(k_rows, dtype=np.int64)
    dQ = np.zeros((B, H, len(q_rows), D), dtype=np.float64)
    dK = np.zeros((B, H, len(k_rows), D), dtype=np.float64)
    dV = np.zeros((B, H, len(k_rows), D), dtype=np.float64)
    # Query blocks: every row when key gradients are wanted, else the rows asked for.
    need_all = len(k_rows) > 0
    for b in range(B):
        for h in range(H):
            kk = k[b, h].astype(np.float64)
            vv = v[b, h].astype(np.float64)
            blocks = range(0, Lq, row_block) if need_all else range(0, len(q_rows), row_block)
            for r0 in blocks:
                rr = np.arange(r0, min(r0 + row_block, Lq)) if need_all else q_rows[r0:r0 + row_block]
                qq = q[b, h, rr].astype(np.float64)
                g = do[b, h, rr].astype(np.float64)
                a = scale * (qq @ kk.T)
                a = np.where(_allowed_keys(rr, Lq, Lk, causal), a, -np.inf)
                e = np.exp(a - a.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)
                da = _softmax_vjp(p, g @ vv.T)
                dv, dk, dq = _score_grads(p, da, qq, kk, g, scale)
                dV[b, h] += dv[k_rows]
                dK[b, h] += dk[k_rows]
                if need_all:
                    # Rows of this block that were asked for, in the caller's order.
                    pos = np.nonzero((q_rows >= rr[0]) & (q_rows <= rr[-1]))[0]
                    if len(pos):
                        dQ[b, h, pos] = dq[q_rows[pos] - rr[0]]
                else:
                    dQ[b, h, r0:r0 + len(rr)] = dq
    return dQ, dK, dV


def _mask_block(mask, mask_kind, b, h, rr, Lk):
    """Rows rr of the (b, h) slab of a [Bm, Hm, Lq, Lk] mask broadcast over
    batch and heads of size 1: (allowed bool block, additive float64 block)."""
    mb = mask[b if mask.shape[0] > 1 else 0, h if mask.shape[1] > 1 else 0][rr]
    if mask_kind == "bool":
        return mb != 0, np.zeros((len(rr), Lk))
    if mask_kind == "add":
        add = mb.astype(np.float64)
        return ~np.isneginf(add), np.where(np.isneginf(add), 0.0, add)
    raise ValueError("mask_kind is 'bool' or 'add'")


def attention_ex(q, k, v, scale: float, causal: bool = False, mask=None, mask_kind=None,
                 dropout_p: float = 0.0, seed: int = 0, offset: int = 0, rows=None, row_block: int = 1024):
    """Attention with a general mask and dropout on the weights, float64.

    The fused tile of the comfyai.app chapter "6.3 FlashAttention"
    (section 6.3.3, "Kernel Fusion") runs scores, scale, mask, softmax,
    dropout and the value product in one place.  Written out plainly:

      a_ij = scale q_i . k_j (+ mask_ij for an additive mask)
      keys with a false boolean mask, an additive -inf or (causal) past the
      bottom-right diagonal are excluded: they drop out of the maximum and
      the sum;
      P = softmax of each row over the remaining keys; LSE = m + ln(s) as
      for ``attention`` (dropout does not change it);
      O = (P o Z / (1 - p)) V with Z the keep pattern of
      ``philox.keep_pattern`` (all ones when p = 0).
    A row with no remaining key has O = 0 and LSE = -inf.

    Args:
      mask: None, or [Bm, Hm, Lq, Lk] with Bm in {1, B}, Hm in {1, H}
        (size-1 axes broadcast); mask_kind "bool" (nonzero = attend) or
        "add" (float values added to the scaled scores, -inf = excluded).
      dropout_p, seed, offset: dropout probability (float32 value used) and
        the generator's key and counter word.
      rows, row_block: as for ``attention``.
    Returns:
      (O [B, H, R, D], LSE [B, H, R]) in float64.
    """
    from .philox import keep_pattern
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    if causal and Lq > Lk:
        raise ValueError("causal attention needs Lq <= Lk")
    if mask is not None:
        mask = np.asarray(mask)
        if mask.ndim != 4 or mask.shape[2:] != (Lq, Lk) or mask.shape[0] not in (1, B) or mask.shape[1] not in (1, H):
            raise ValueError("mask must be [1 or B, 1 or H, Lq, Lk]")
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    rp = 1.0 / (1.0 - float(np.float32(dropout_p)))
    O = np.zeros((B, H, R, D), dtype=np.float64)
    LSE = np.full((B, H, R), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            kk = k[b, h].astype(np.float64)
            vv = v[b, h].astype(np.float64)
            for r0 in range(0, R, row_block):
                rr = rows[r0:r0 + row_block]
                a = scale * (q[b, h, rr].astype(np.float64) @ kk.T)
                allowed = _allowed_keys(rr, Lq, Lk, causal)
                if mask is not None:
                    ok, add = _mask_block(mask, mask_kind, b, h, rr, Lk)
                    allowed = allowed & ok
                    a = a + add
                a = np.where(allowed, a, -np.inf)
                live = allowed.any(axis=1)
                m = np.where(live, a.max(axis=1), 0.0)
                e = np.where(allowed, np.exp(a - m[:, None]), 0.0)
                s = e.sum(axis=1)
                p = np.where(live[:, None], e / np.where(live, s, 1.0)[:, None], 0.0)
                if dropout_p:
                    p = p * keep_pattern(seed, offset, b * H + h, rr, Lk, dropout_p) * rp
                O[b, h, r0:r0 + len(rr)] = p @ vv
                LSE[b, h, r0:r0 + len(rr)] = np.where(live, m + np.log(np.where(live, s, 1.0)), -np.inf)
    return O, LSE


def attention_ex_bwd(q, k, v, do, scale: float, causal: bool = False, mask=None, mask_kind=None,
                     dropout_p: float = 0.0, seed: int = 0, offset: int = 0, row_block: int = 1024):
    """Gradients of ``attention_ex``'s O with respect to q, k and v, float64.

    The chain rule of O = (P o Z / (1 - p)) V with P the masked softmax of
    a = scale q k^T (+ additive mask): with dP~ = (Z / (1 - p)) o (dO V^T),
      dV = (P o Z / (1 - p))^T dO,
      dA_ij = P_ij (dP~_ij - sum_l P_il dP~_il),
      dQ = scale dA K,  dK = scale dA^T Q.
    No gradient is returned for the mask.  Returns (dQ, dK, dV).
    """
    from .philox import keep_pattern
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    do = np.asarray(do)
    B, H, Lq, D = q.shape
    Lk = k.shape[2]
    if mask is not None:
        mask = np.asarray(mask)
    rp = 1.0 / (1.0 - float(np.float32(dropout_p)))
    dQ = np.zeros((B, H, Lq, D))
    dK = np.zeros((B, H, Lk, D))
    dV = np.zeros((B, H, Lk, D))
    for b in range(B):
        for h in range(H):
            kk = k[b, h].astype(np.float64)
            vv = v[b, h].astype(np.float64)
            for r0 in range(0, Lq, row_block):
                rr = np.arange(r0, min(r0 + row_block, Lq))
                qq = q[b, h, rr].astype(np.float64)
                g = do[b, h, rr].astype(np.float64)
                a = scale * (qq @ kk.T)
                allowed = _allowed_keys(rr, Lq, Lk, causal)
                if mask is not None:
                    ok, add = _mask_block(mask, mask_kind, b, h, rr, Lk)
                    allowed = allowed & ok
                    a = a + add
                a = np.where(allowed, a, -np.inf)
                live = allowed.any(axis=1)
                m = np.where(live, a.max(axis=1), 0.0)
                e = np.where(allowed, np.exp(a - m[:, None]), 0.0)
                s = e.sum(axis=1)
                p = np.where(live[:, None], e / np.where(live, s, 1.0)[:, None], 0.0)
                z = keep_pattern(seed, offset, b * H + h, rr, Lk, dropout_p) * rp if dropout_p else 1.0
                da = _softmax_vjp(p, z * (g @ vv.T))
                dv, dk, dq = _score_grads(p * z, da, qq, kk, g, scale)
                dV[b, h] += dv
                dK[b, h] += dk
                dQ[b, h, rr] = dq
    return dQ, dK, dV


def _softmax_vjp(p, dp):
    """dA_ij = P_ij (dP_ij - sum_l P_il dP_il): the upstream gradient dP of
    the weights pulled back through each row's softmax."""
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def _score_grads(p, da, qq, kk, g, scale):
    """Products of one query block: P^T dO (values), scale dA^T Q (keys) and
    scale dA K (queries), the last two from a = scale q k^T."""
    return p.T @ g, scale * (da.T @ qq), scale * (da @ kk)


def _check_block(p, o, m, lse, allowed, vv):
    n_allowed = allowed.sum(axis=1)
    if np.max(np.abs(p.sum(axis=1) - 1.0)) > 1e-13:
        raise AssertionError("oracle: weight rows do not sum to one")
    tol = 1e-12 * np.maximum(1.0, np.abs(m))
    if np.any(lse < m - tol) or np.any(lse > m + np.log(n_allowed) + tol):
        raise AssertionError("oracle: LSE outside [m, m + ln(#keys)]")
    # Convex combination: O[i, d] lies within the range of v[:, d] over the
    # keys row i may see.  Small blocks check per row; large blocks check
    # against the range over all keys (cheaper, still a valid bound).
    if o.shape[0] * vv.shape[0] <= (1 << 16):
        sel = allowed[:, :, None]
        lo = np.where(sel, vv[None, :, :], np.inf).min(axis=1)
        hi = np.where(sel, vv[None, :, :], -np.inf).max(axis=1)
    else:
        lo = vv.min(axis=0)[None, :]
        hi = vv.max(axis=0)[None, :]
    slack = 1e-12 * np.maximum(1.0, np.abs(lo) + np.abs(hi))
    if np.any(o < lo - slack) or np.any(o > hi + slack):
        raise AssertionError("oracle: output outside the range of V")


def _chunks(n: int, bounds: Sequence[int]) -> Iterable[slice]:
    """Slices for chunk boundaries ``0 = b0 < b1 < ... < bK = n``."""
    b = list(bounds)
    if b[0] != 0 or b[-1] != n or any(x >= y for x, y in zip(b, b[1:])):
        raise ValueError("bounds must increase strictly from 0 to n")
    for x, y in zip(b, b[1:]):
        yield slice(x, y)


def two_pass_chunked(a, bounds):
    """Softmax of one score row in two reads, chunk by chunk.

    The guide's simplified mechanism (slides 18-24): the first read keeps a
    running maximum ``d_k`` and a running denominator ``s_k``, with
    ``d_k = max(d_{k-1}, max of chunk k)`` and
    ``s_k = s_{k-1} exp(d_{k-1} - d_k) + sum_{i in chunk k} exp(a_i - d_k)``;
    the second read forms ``a^_i = exp(a_i - d_B) / s_B``.

    A chunk whose scores are all minus infinity (fully masked) contributes
    nothing and is skipped while no finite maximum exists yet, so that
    ``(-inf) - (-inf)`` never occurs.

    Returns (weights, d_B, s_B).
    """
    a = np.asarray(a, dtype=np.float64)
    d = -math.inf
    s = 0.0
    for c in _chunks(a.shape[0], bounds):
        chunk_max = float(np.max(a[c]))
        d_new = max(d, chunk_max)
        if d_new == -math.inf:
            continue
        rescale = math.exp(d - d_new) if d != -math.inf else 0.0
        s = s * rescale + float(np.sum(np.exp(a[c] - d_new)))
        d = d_new
    w = np.exp(a - d) / s
    return w, d, s


def one_pass_chunked(a, vals, bounds):
    """Weighted sum of value rows in one read, with the output correction.

    The guide's full mechanism (slides 25-27): after each chunk ``k`` the
    running output is normalised with the chunk's ``d_k`` and ``s_k``:
    ``O_k = O_{k-1} (s_{k-1} / s_k) exp(d_{k-1} - d_k)
            + sum_{i in chunk k} exp(a_i - d_k) / s_k * v_i``,
    starting from ``O_0 = 0``, ``s_0 = 0``, ``d_0 = -inf``; after the last
    chunk ``O_B = sum_i a^_i v_i``.

    Args:
      a: [L] scores.
      vals: [L, Dv] value rows.
      bounds: chunk boundaries from 0 to L.

    Returns (O_B, d_B, s_B).
    """
    a = np.asarray(a, dtype=np.float64)
    vals = np.asarray(vals, dtype=np.float64)
    if vals.ndim == 1:
        vals = vals[:, None]
    O = np.zeros(vals.shape[1], dtype=np.float64)
    d = -math.inf
    s = 0.0
    for c in _chunks(a.shape[0], bounds):
        d_new = max(d, float(np.max(a[c])))
        if d_new == -math.inf:
            continue
        e = np.exp(a[c] - d_new)
        first = d == -math.inf
        s_new = (0.0 if first else s * math.exp(d - d_new)) + float(e.sum())
        carried = np.zeros_like(O) if first else O * (s / s_new) * math.exp(d - d_new)
        O = carried + (e / s_new) @ vals[c]
        d, s = d_new, s_new
    return O, d, s


def decoupled_softmax(x, bounds):
    """Softmax over blocks with per-block statistics, merged afterwards.

    The comfyai chapter's "Decoupled Softmax" and its "A Simple Example"
    (section 6.3.3): each block ``j`` keeps its own maximum ``m~_j`` and sum
    ``l~_j = sum exp(x - m~_j)``; blocks merge by
    ``m_new = max(m, m~_j)`` and
    ``l_new = exp(m - m_new) l + exp(m~_j - m_new) l~_j``,
    and each block's numerators are rescaled by ``exp(m~_j - m_final)``.

    Returns (softmax, m_final, l_final, per_block) where ``per_block`` lists
    (m~_j, l~_j) in block order.
    """
    x = np.asarray(x, dtype=np.float64)
    m = -math.inf
    l = 0.0
    per_block = []
    for c in _chunks(x.shape[0], bounds):
        m_blk = float(np.max(x[c]))
        l_blk = float(np.sum(np.exp(x[c] - m_blk)))
        per_block.append((m_blk, l_blk))
        m_new = max(m, m_blk)
        l = (math.exp(m - m_new) * l if m != -math.inf else 0.0) + math.exp(m_blk - m_new) * l_blk
        m = m_new
    out = np.empty_like(x)
    for c, (m_blk, _) in zip(_chunks(x.shape[0], bounds), per_block):
        out[c] = np.exp(x[c] - m_blk) * math.exp(m_blk - m) / l
    return out, m, l, per_block


def tiled_outer_kv(q, k, v, scale: float, causal: bool = False,
                   block_r: int = 4, block_c: int = 4):
    """One head of attention in the comfyai chapter's tile order.

    Follows the "Full Forward Process" of section 6.3.3: O, l and m are
    initialised (to 0, 0 and minus infinity) in "HBM" (here host arrays);
    the outer loop walks the key/value blocks K_j, V_j of ``block_c`` rows;
    the inner loop walks the query blocks Q_i of ``block_r`` rows, reads back
    O_i, l_i, m_i, computes the block scores S_ij = scale Q_i K_j^T, the
    block statistics m~_ij (row max), P~_ij = exp(S_ij - m~_ij) and
    l~_ij (row sum), merges them into m_new = max(m_i, m~_ij) and
    l_new = exp(m_i - m_new) l_i + exp(m~_ij - m_new) l~_ij, updates
    O_i <- (l_i exp(m_i - m_new) O_i + exp(m~_ij - m_new) P~_ij V_j) / l_new
    and writes O_i, l_i, m_i back.

    Rows of a block with no allowed key in K_j (causal) keep their state.

    Args:
      q: [Lq, D]; k, v: [Lk, D].

    Returns (O [Lq, D], LSE [Lq]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, Lk = q.shape[0], k.shape[0]
    O = np.zeros((Lq, v.shape[1]))
    l = np.zeros(Lq)
    m = np.full(Lq, -np.inf)
    for j0 in range(0, Lk, block_c):
        Kj = k[j0:j0 + block_c]
        Vj = v[j0:j0 + block_c]
        cols = np.arange(j0, j0 + Kj.shape[0])
        for i0 in range(0, Lq, block_r):
            rows = np.arange(i0, min(i0 + block_r, Lq))
            S = scale * (q[rows] @ Kj.T)
            if causal:
                S = np.where(cols[None, :] <= rows[:, None] + (Lk - Lq), S, -np.inf)
            live = np.isfinite(S).any(axis=1)
            if not live.any():
                continue
            r = rows[live]
            S = S[live]
            m_t = S.max(axis=1)
            P_t = np.exp(S - m_t[:, None])
            l_t = P_t.sum(axis=1)
            m_old = m[r]
            m_new = np.maximum(m_old, m_t)
            a_old = np.where(np.isfinite(m_old), np.exp(m_old - m_new), 0.0)
            a_new = np.exp(m_t - m_new)
            l_new = a_old * l[r] + a_new * l_t
            O[r] = ((l[r] * a_old)[:, None] * O[r] + a_new[:, None] * (P_t @ Vj)) / l_new[:, None]
            l[r] = l_new
            m[r] = m_new
    return O, m + np.log(l)
