"""The pages' blocked online-softmax recurrences, in float64 — TEST ONLY.

These are not a second oracle: they exist so the tests can show that the
plain definition in ``oracle.attention`` equals what the tiled algorithms on
the pages compute (Theorem 1 on the FlashAttention paper summary at
zhaifeiyue.github.io/papers/2205.14135), and can replay the three-tile worked
example of the wmrh.cn explainer.  Only ``tests/`` use them.

Functions
---------
``online_stats``        running (m, l) over consecutive score tiles of one row
                        (FlashAttention-2 notes, eqs. (5)-(6); languisher.top
                        notes, "Online Softmax", incremental normaliser).
``merge_states``        merge two partial softmax states (m, l, O) into one
                        (languisher.top notes, merging two vectors' softmax
                        statistics; paper summary, Technique 1).
``fa1_forward``         K/V-outer loop, output renormalised on every step and
                        written back (walkthrough on bluuewhale.github.io,
                        "Algorithm"; languisher.top, "Online Softmax in
                        FlashAttention", the Phi + Delta update).
``fa2_forward``         Q-outer loop, unnormalised accumulator rescaled by
                        exp(m_old - m_new), one division at the end, and
                        L = m + ln(l) (FlashAttention-2 notes, Algorithm 1 and
                        eqs. (10)-(15)).  The notes print the rescale factor
                        as diag(exp(m_old - m_new)) with an inverse; the
                        two-block check of eq. (13) and the wmrh.cn pseudocode
                        both multiply by exp(m_old - m_new), which is the
                        reading taken here (the inverse breaks eq. (14)).
"""
from __future__ import annotations

import numpy as np


def _exp_shift(a, b):
    """exp(a - b) with the convention exp(-inf - (-inf)) = 0 (empty state)."""
    a, b = np.broadcast_arrays(np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64))
    out = np.zeros(a.shape)
    ok = np.isfinite(a) & np.isfinite(b)
    out[ok] = np.exp(a[ok] - b[ok])
    return out if out.ndim else float(out)


def online_stats(tiles):
    """Running (m, l) of one score row seen tile by tile.

    Starts from m = -inf, l = 0 (languisher.top notes, initialisation) and
    after each tile applies m' = max(m, max(tile)), l' = exp(m - m') l +
    sum(exp(tile - m')).  Returns the list of (m, l) after every tile.
    """
    m, l = -np.inf, 0.0
    hist = []
    for t in tiles:
        t = np.asarray(t, dtype=np.float64)
        m_new = max(m, float(t.max()))
        l = _exp_shift(m, m_new) * l + float(np.exp(t - m_new).sum())
        m = m_new
        hist.append((m, l))
    return hist


def merge_states(s1, s2):
    """Merge (m1, l1, O1) and (m2, l2, O2), each O normalised by its own l.

    m = max(m1, m2); l = exp(m1 - m) l1 + exp(m2 - m) l2;
    O = (exp(m1 - m) l1 O1 + exp(m2 - m) l2 O2) / l.  Row-wise on arrays.
    """
    m1, l1, o1 = s1
    m2, l2, o2 = s2
    m = np.maximum(m1, m2)
    a1 = _exp_shift(m1, m) * l1
    a2 = _exp_shift(m2, m) * l2
    l = a1 + a2
    safe = np.where(l > 0, l, 1.0)
    o = (np.asarray(a1)[..., None] * o1 + np.asarray(a2)[..., None] * o2) / np.asarray(safe)[..., None]
    return m, l, o


def _tile_scores(q, k, scale, r0, r1, c0, c1, causal):
    S = scale * (q[r0:r1] @ k[c0:c1].T)
    if causal:
        i = np.arange(r0, r1)[:, None]
        j = np.arange(c0, c1)[None, :]
        S = np.where(j <= i, S, -np.inf)
    return S


def fa1_forward(q, k, v, scale, br, bc, causal=False, trace=None):
    """K/V-outer blocked forward with the output renormalised every step.

    State O, l, m lives in full-length arrays that each inner step reads and
    rewrites (the HBM round trip of the first FlashAttention).  If ``trace``
    is a list, (j, m.copy(), l.copy(), O.copy()) is appended after every
    outer step j so the Theorem 1 invariants can be checked.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n = q.shape[0]
    nk, dv = v.shape
    O = np.zeros((n, dv))
    l = np.zeros(n)
    m = np.full(n, -np.inf)
    for c0 in range(0, nk, bc):
        c1 = min(nk, c0 + bc)
        for r0 in range(0, n, br):
            r1 = min(n, r0 + br)
            S = _tile_scores(q, k, scale, r0, r1, c0, c1, causal)
            mt = S.max(axis=1)                              # tile row max
            Pt = _exp_shift(S, mt[:, None])                 # tile numerators
            lt = Pt.sum(axis=1)
            mi, li, oi = m[r0:r1], l[r0:r1], O[r0:r1]
            m_new = np.maximum(mi, mt)
            a_old = _exp_shift(mi, m_new) * li              # diag(l) e^{m - m_new}
            a_new = _exp_shift(mt, m_new)                   # e^{m_tile - m_new}
            l_new = a_old + a_new * lt
            num = a_old[:, None] * oi + a_new[:, None] * (Pt @ v[c0:c1])
            O[r0:r1] = num / np.where(l_new > 0, l_new, 1.0)[:, None]
            l[r0:r1] = l_new
            m[r0:r1] = m_new
        if trace is not None:
            trace.append((c1, m.copy(), l.copy(), O.copy()))
    return O, m, l


def fa2_forward(q, k, v, scale, br, bc, causal=False, inverse_rescale=False):
    """Q-outer blocked forward with deferred normalisation; returns (O, L).

    ``inverse_rescale=True`` applies the rescale factor with the inverse as
    printed in the notes' eq. (10); it exists only so a test can show that
    reading is wrong.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    n = q.shape[0]
    nk, dv = v.shape
    O = np.zeros((n, dv))
    L = np.zeros(n)
    for r0 in range(0, n, br):
        r1 = min(n, r0 + br)
        acc = np.zeros((r1 - r0, dv))                        # unnormalised O~
        l = np.zeros(r1 - r0)
        m = np.full(r1 - r0, -np.inf)
        for c0 in range(0, nk, bc):
            c1 = min(nk, c0 + bc)
            S = _tile_scores(q, k, scale, r0, r1, c0, c1, causal)
            m_new = np.maximum(m, S.max(axis=1))
            Pt = _exp_shift(S, m_new[:, None])
            alpha = _exp_shift(m, m_new)
            if inverse_rescale:
                alpha = np.where(alpha > 0, 1.0 / np.where(alpha > 0, alpha, 1.0), 0.0)
            l = alpha * l + Pt.sum(axis=1)
            acc = alpha[:, None] * acc + Pt @ v[c0:c1]
            m = m_new
        has = l > 0
        O[r0:r1] = acc / np.where(has, l, 1.0)[:, None]
        L[r0:r1] = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return O, L
