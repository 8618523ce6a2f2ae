"""Philox4x32-10 and the dropout keep pattern, written from the published
definition (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
as 1, 2, 3", SC 2011, section 3.2 and table 2).

Test infrastructure only: nothing on the product path imports this module,
and it imports nothing from it.  The GPU kernels carry their own
implementation of the same generator; the two are compared bit for bit.

Philox4xW-R maps a 4-word counter and a 2-word key to 4 words through R
rounds.  One round multiplies words 0 and 2 by the constants M0, M1 (full
2W-bit products split into high and low halves), then outputs

    (hi(M1 x2) ^ x1 ^ k0,  lo(M1 x2),  hi(M0 x0) ^ x3 ^ k1,  lo(M0 x0))

and the key is bumped by the Weyl constants (W0, W1) between rounds.  The
function is generic in the word width: the 64-bit instance is pinned against
NumPy's own Philox bit generator (same round structure and key schedule);
the 32-bit instance, the one dropout uses, is pinned to the published
Philox4x32-10 known-answer vectors of the Random123 library that accompanies
the paper.

Dropout reading (the comfyai.app chapter "6.3 FlashAttention" lists dropout
between the softmax and the value product of the fused tile, section 6.3.3,
"Kernel Fusion", without fixing a generator or the width of the uniform):
the weight P_ij of (b, h, i, j) is kept iff the 16-bit half (j mod 2: 0 the
low half, 1 the high half) of word ((j mod 8) / 2) of

    Philox4x32-10(counter = (j / 8, i, b H + h, offset),
                  key = (seed mod 2^32, seed / 2^32))

is >= floor(p 2^16), with p the float32 dropout probability; kept weights
are scaled by 1 / (1 - p).  One block thus serves 8 consecutive keys; the
keep rate is 1 - floor(p 2^16) / 2^16, within 2^-16 of 1 - p.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["philox", "philox4x32", "philox4x64", "dropout_threshold", "keep_pattern"]

M4x32 = (0xD2511F53, 0xCD9E8D57)
W4x32 = (0x9E3779B9, 0xBB67AE85)
M4x64 = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
W4x64 = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)


def philox(ctr, key, bits, M, W, rounds=10):
    """Philox4x{bits}-{rounds} on Python integers (one block).

    ctr: 4 words, key: 2 words, each < 2^bits.  Returns 4 words.
    """
    mask = (1 << bits) - 1
    x = [int(c) & mask for c in ctr]
    k = [int(c) & mask for c in key]
    for r in range(rounds):
        if r:
            k = [(k[0] + W[0]) & mask, (k[1] + W[1]) & mask]
        p0 = M[0] * x[0]
        p1 = M[1] * x[2]
        x = [(p1 >> bits) ^ x[1] ^ k[0], p1 & mask, (p0 >> bits) ^ x[3] ^ k[1], p0 & mask]
    return x


def philox4x64(ctr, key):
    return philox(ctr, key, 64, M4x64, W4x64)


def philox4x32(c0, c1, c2, c3, k0, k1, rounds=10):
    """Vectorised Philox4x32: counter words and key words are broadcastable
    integer arrays (values < 2^32); returns four uint64 arrays of 32-bit
    words.  Same rounds as ``philox`` with bits = 32."""
    m = np.uint64(0xFFFFFFFF)
    x = [np.asarray(c, dtype=np.uint64) & m for c in (c0, c1, c2, c3)]
    k = [np.asarray(k0, dtype=np.uint64) & m, np.asarray(k1, dtype=np.uint64) & m]
    M0, M1 = np.uint64(M4x32[0]), np.uint64(M4x32[1])
    for r in range(rounds):
        if r:
            k = [(k[0] + np.uint64(W4x32[0])) & m, (k[1] + np.uint64(W4x32[1])) & m]
        p0 = M0 * x[0]  # < 2^64: exact in uint64
        p1 = M1 * x[2]
        x = [(p1 >> np.uint64(32)) ^ x[1] ^ k[0], p1 & m, (p0 >> np.uint64(32)) ^ x[3] ^ k[1], p0 & m]
    return x


def dropout_threshold(p: float) -> int:
    """floor(p 2^16) for the float32 value of p, p in [0, 1)."""
    p32 = float(np.float32(p))
    if not 0.0 <= p32 < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return min(int(math.floor(p32 * 65536.0)), 0xFFFF)


def keep_pattern(seed: int, offset: int, bh: int, rows, Lk: int, p: float) -> np.ndarray:
    """Boolean [len(rows), Lk]: which weights of (b H + h = bh) survive dropout."""
    rows = np.asarray(rows, dtype=np.uint64)[:, None]
    j = np.arange(Lk, dtype=np.uint64)[None, :]
    words = philox4x32(j >> np.uint64(3), rows, np.uint64(bh), np.uint64(offset & 0xFFFFFFFF),
                       np.uint64(seed & 0xFFFFFFFF), np.uint64((seed >> 32) & 0xFFFFFFFF))
    sel = ((j >> np.uint64(1)) & np.uint64(3)).astype(np.int64)
    w = np.choose(np.broadcast_to(sel, (rows.shape[0], Lk)), [np.broadcast_to(x, (rows.shape[0], Lk)) for x in words])
    half = (w >> (np.uint64(16) * (j & np.uint64(1)))) & np.uint64(0xFFFF)
    return half >= np.uint64(dropout_threshold(p))
