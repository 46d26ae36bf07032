"""Philox4x32-10 counter-based generator and the dropout decisions built on
it — TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Philox4x32-R (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
as 1, 2, 3", SC 2011): a 4-word counter and a 2-word key; each of R rounds
multiplies counter words 0 and 2 by two fixed 32-bit constants into 64-bit
products, and the new counter is (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2),
hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key is bumped by two Weyl constants
between rounds.  R = 10 is the recommended round count.  Written here from
that description, vectorised with NumPy 64-bit integers.

The pages only name dropout among the operations fused into the attention
kernel; the decision rule below is this repository's reading (stated where
it is used): element (i, j) of head bh is kept iff byte j % 4 of word i % 4
of Philox4x32-10((i // 4, j // 4, bh, offset), (seed_lo, seed_hi)) is at
least t = floor(256 p + 0.5).
"""
from __future__ import annotations

import math

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32(ctr, key, rounds: int = 10):
    """ctr: four arrays (or ints) broadcastable together; key: (k0, k1).
    Returns four uint32 arrays."""
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & _MASK for x in ctr)
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0, k1 = np.uint64(key[0]) & _MASK, np.uint64(key[1]) & _MASK
    m0, m1 = np.uint64(M0), np.uint64(M1)
    for r in range(rounds):
        if r:
            k0 = (k0 + np.uint64(W0)) & _MASK
            k1 = (k1 + np.uint64(W1)) & _MASK
        p0 = m0 * c0          # < 2^64: exact in uint64
        p1 = m1 * c2
        c0, c1, c2, c3 = (((p1 >> np.uint64(32)) ^ c1 ^ k0) & _MASK, p1 & _MASK,
                          ((p0 >> np.uint64(32)) ^ c3 ^ k1) & _MASK, p0 & _MASK)
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def drop_threshold(p: float) -> int:
    """t = floor(256 p + 0.5) for the float32 value of p; p' = t / 256."""
    pf = float(np.float32(p))
    if not (0.0 <= pf < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    t = math.floor(pf * 256.0 + 0.5)
    if t > 255:
        raise ValueError("dropout probability rounds to 256/256")
    return t


def keep_matrix(n_q: int, n_k: int, head: int, seed: int, offset: int, thr: int) -> np.ndarray:
    """Boolean [n_q, n_k]: the dropout keep decisions of one head."""
    bq, bk = (n_q + 3) // 4, (n_k + 3) // 4
    ib = np.arange(bq, dtype=np.uint64)[:, None]
    jb = np.arange(bk, dtype=np.uint64)[None, :]
    words = philox4x32((ib, jb, head, offset), (seed & 0xFFFFFFFF, seed >> 32))
    W = np.stack(words)                                   # [row r, ib, jb]
    shifts = (8 * np.arange(4, dtype=np.uint32))[None, None, None, :]
    B = (W[..., None] >> shifts) & 0xFF                   # [r, ib, jb, byte c]
    M = B.transpose(1, 0, 2, 3).reshape(4 * bq, 4 * bk)   # row 4 ib + r, column 4 jb + c
    return M[:n_q, :n_k] >= thr
