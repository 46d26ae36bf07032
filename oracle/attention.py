"""Plain float64 definition of exact attention and its gradient (CPU oracle).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the GPU library.

What is computed, per (batch, head), with Q, K, V, dO in R^{N x d} taken as the
exact values the GPU received (dtype-rounded, then widened to float64):

* scores S = scale * Q K^T, the scaled form on the FlashAttention walkthrough
  (bluuewhale.github.io, "How Attention Is Computed");
* entries that the causal rule (key j <= query i, FlashAttention-2 notes,
  "Causal mask optimisation") or the block mask (walkthrough,
  "Block-Sparse FlashAttention": one 0/1 entry per score tile) forbid are set
  to -inf before the softmax;
* P = row softmax of S with the row maximum subtracted first (safe softmax,
  Flash Attention v1 notes on languisher.top, "Naive Attention");
* O = P V and the row log-sum-exp LSE_i = m_i + ln(sum_j exp(S_ij - m_i))
  (FlashAttention-2 notes, eq. (15));
* the backward pass by the chain rule (FlashAttention-2 notes, eqs. (27)-(30)):
  dV = P^T dO, dP = dO V^T, dS = P o (dP - <p, dp>), dQ = scale dS K,
  dK = scale dS^T Q.  The row term <p, dp> is summed from P and dP directly,
  not from rowsum(dO o O), so the D identity used by the GPU backward is
  checked independently rather than assumed.

S and P are materialised in full (no tiling, no online softmax); rows may be
processed in chunks only to bound host memory, which changes no arithmetic
beyond the summation order of dK and dV across chunks.

Rows with no allowed key (unreachable for causal or diagonal-kept masks) follow
a stated convention: O = 0, LSE = -inf, zero gradient contributions.
"""
from __future__ import annotations

import numpy as np

MASK_BLOCK = 128  # tokens per block-mask entry


def allowed(n_q: int, n_k: int, causal: bool, block_mask=None,
            mask_block: int = MASK_BLOCK, rows=None) -> np.ndarray:
    """Boolean matrix [len(rows), n_k]: True where query row i may see key j.

    causal: j <= i + (n_k - n_q).  With equal lengths this is j <= i (query
    and key positions share one index space).  With fewer queries than keys
    (a KV cache) the queries are the last n_q positions of the sequence, so
    query i sits at position n_k - n_q + i: the last query sees every key,
    and a query with n_k - n_q + i < 0 sees none.
    block_mask: 0/1 array [ceil(n_q/mask_block), ceil(n_k/mask_block)]; entry
    (i // mask_block, j // mask_block) must be 1.
    """
    i = np.arange(n_q) if rows is None else np.asarray(rows)
    j = np.arange(n_k)
    ok = np.ones((i.shape[0], n_k), dtype=bool)
    if causal:
        ok &= j[None, :] <= i[:, None] + (n_k - n_q)
    if block_mask is not None:
        bm = np.asarray(block_mask).astype(bool)
        ok &= bm[i[:, None] // mask_block, j[None, :] // mask_block]
    return ok


def _softmax_rows(S: np.ndarray):
    """Safe row softmax of S (entries may be -inf). Returns P, m, LSE."""
    m = S.max(axis=1)
    has = np.isfinite(m)
    m0 = np.where(has, m, 0.0)
    E = np.exp(S - m0[:, None])          # exp(-inf) = 0 for masked entries
    l = E.sum(axis=1)
    l1 = np.where(has, l, 1.0)
    P = E / l1[:, None]
    lse = np.where(has, m0 + np.log(l1), -np.inf)
    return P, m, lse


def scores(q, k, scale, causal=False, block_mask=None, mask_block=MASK_BLOCK, rows=None):
    """S = scale * Q K^T with forbidden entries set to -inf (rows subset optional)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    r = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    S = scale * (q[r] @ k.T)
    ok = allowed(q.shape[0], k.shape[0], causal, block_mask, mask_block, rows=r)
    return np.where(ok, S, -np.inf)


def forward_head(q, k, v, scale, causal=False, block_mask=None,
                 mask_block=MASK_BLOCK, rows=None):
    """One head: returns (O [R, d], LSE [R]) for the selected query rows."""
    S = scores(q, k, scale, causal, block_mask, mask_block, rows)
    P, _, lse = _softmax_rows(S)
    O = P @ np.asarray(v, dtype=np.float64)
    return O, lse


def probs_head(q, k, scale, causal=False, block_mask=None, mask_block=MASK_BLOCK, rows=None):
    """One head: the full probability rows P [R, N] (for invariant tests)."""
    P, _, _ = _softmax_rows(scores(q, k, scale, causal, block_mask, mask_block, rows))
    return P


def _row_chunk(n: int) -> int:
    # keep one fp64 chunk of S/P/dP near 64 MiB
    return max(1, min(n, (1 << 23) // max(n, 1)))


def backward_head(q, k, v, do, scale, causal=False, block_mask=None,
                  mask_block=MASK_BLOCK, chunk=None):
    """One head: (dQ, dK, dV) of loss sum(O o dO) by the chain rule.

    Every row's P and dP are materialised; ``chunk`` only bounds memory.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n = q.shape[0]
    c = chunk or _row_chunk(k.shape[0])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, n, c):
        rows = np.arange(r0, min(n, r0 + c))
        P = probs_head(q, k, scale, causal, block_mask, mask_block, rows)
        dv += P.T @ do[rows]                       # dV = P^T dO
        dP = do[rows] @ v.T                        # dP = dO V^T
        rowdot = (P * dP).sum(axis=1)              # <p, dp> per row, eq. (30)
        dS = P * (dP - rowdot[:, None])            # softmax Jacobian, eq. (29)
        dq[rows] = scale * (dS @ k)                # S = scale Q K^T
        dk += scale * (dS.T @ q[rows])
    return dq, dk, dv


def _heads(B, H, heads):
    return [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)


def forward(q, k, v, scale, causal=False, block_mask=None, mask_block=MASK_BLOCK, heads=None):
    """Batched [B, H, N, d] float64 inputs -> dict {(b, h): (O, LSE)}."""
    B, H = q.shape[:2]
    return {(b, h): forward_head(q[b, h], k[b, h], v[b, h], scale, causal, block_mask, mask_block)
            for (b, h) in _heads(B, H, heads)}


def backward(q, k, v, do, scale, causal=False, block_mask=None, mask_block=MASK_BLOCK, heads=None):
    """Batched [B, H, N, d] float64 inputs -> dict {(b, h): (dQ, dK, dV)}."""
    B, H = q.shape[:2]
    return {(b, h): backward_head(q[b, h], k[b, h], v[b, h], do[b, h], scale, causal,
                                  block_mask, mask_block)
            for (b, h) in _heads(B, H, heads)}


def grad_q_rows(q, k, v, do, scale, causal=False, block_mask=None, mask_block=MASK_BLOCK, rows=None):
    """dQ for the selected query rows only: each row of dQ depends on its own
    row of P and dP (and on all of K and V), so large problems can be checked
    row by row."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    r = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    P = probs_head(q, k, scale, causal, block_mask, mask_block, r)
    dP = do[r] @ v.T
    rowdot = (P * dP).sum(axis=1)
    dS = P * (dP - rowdot[:, None])
    return scale * (dS @ k)


# ---------------------------------------------------------------- grouped K/V heads
# FlashAttention-2 notes, "MQA and GQA support": query heads are split into
# groups that each read one shared K/V head (one group: multi-query
# attention; one head per group: ordinary multi-head attention).  The notes
# give the group of query head i as a floor division of i by the group
# parameter; read with H / Hkv query heads per group, head i belongs to group
# i // (H / Hkv), i.e. runs of consecutive heads share a K/V head.

def kv_head_of(h: int, H: int, Hkv: int) -> int:
    """K/V head read by query head h when Hkv K/V heads serve H query heads."""
    if Hkv <= 0 or H % Hkv:
        raise ValueError(f"H={H} query heads cannot share Hkv={Hkv} K/V heads evenly")
    return h // (H // Hkv)


def forward_gqa(q, k, v, scale, causal=False, heads=None):
    """q [B, H, N, d], k, v [B, Hkv, N, d] -> {(b, h): (O, LSE)}: each query
    head attends over its group's K/V head."""
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    return {(b, h): forward_head(q[b, h], k[b, kv_head_of(h, H, Hkv)], v[b, kv_head_of(h, H, Hkv)],
                                 scale, causal)
            for (b, h) in _heads(B, H, heads)}


def backward_gqa(q, k, v, do, scale, causal=False):
    """Gradients of sum(O o dO) with grouped K/V heads.

    Returns (dq {(b, h)}, dk {(b, hk)}, dv {(b, hk)}).  A shared K/V head
    enters the loss once per query head of its group, so its gradient is the
    sum of those heads' per-head gradients (the notes' backward reduction over
    the group)."""
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    dq = {}
    dk = {(b, g): np.zeros(k.shape[2:], dtype=np.float64) for b in range(B) for g in range(Hkv)}
    dv = {(b, g): np.zeros(v.shape[2:], dtype=np.float64) for b in range(B) for g in range(Hkv)}
    for b in range(B):
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            gq, gk, gv = backward_head(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal)
            dq[(b, h)] = gq
            dk[(b, g)] += gk
            dv[(b, g)] += gv
    return dq, dk, dv


# ---------------------------------------------------------------- packed variable-length batches
# Several sequences of different lengths packed along one token axis: each
# sequence is its own attention problem (its keys only; the causal rule
# counts positions from its own start).  q [T, H, d], k, v [T, Hkv, d],
# cu [B + 1] with sequence b on rows cu[b] .. cu[b+1]-1; LSE is [H, T].

def forward_varlen(q, k, v, cu, scale, causal=False):
    q = np.asarray(q, dtype=np.float64)
    T, H, _ = q.shape
    Hkv = k.shape[1]
    O = np.zeros(q.shape)
    L = np.full((H, T), -np.inf)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        if e <= s:
            continue
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            O[s:e, h], L[h, s:e] = forward_head(q[s:e, h], k[s:e, g], v[s:e, g], scale, causal)
    return O, L


def backward_varlen(q, k, v, do, cu, scale, causal=False):
    """(dQ [T, H, d], dK, dV [T, Hkv, d]) of sum(O o dO) for a packed batch."""
    q = np.asarray(q, dtype=np.float64)
    T, H, _ = q.shape
    Hkv = k.shape[1]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(len(cu) - 1):
        s, e = int(cu[b]), int(cu[b + 1])
        if e <= s:
            continue
        for h in range(H):
            g = kv_head_of(h, H, Hkv)
            gq, gk, gv = backward_head(q[s:e, h], k[s:e, g], v[s:e, g], do[s:e, h], scale, causal)
            dq[s:e, h] = gq
            dk[s:e, g] += gk
            dv[s:e, g] += gv
    return dq, dk, dv


# ---------------------------------------------------------------- dropout
# The pages name dropout among the operations fused into the attention
# kernel (FlashAttention paper summary) without fixing it further; read
# here as inverted dropout on the probabilities: with keep decisions Z and
# drop probability p', O = (P o Z) V / (1 - p'), LSE unchanged.  The
# gradient is the chain rule through the same Z.

def forward_head_dropout(q, k, v, scale, causal, keep, p_drop):
    """(O, LSE) with the probabilities P o keep / (1 - p_drop)."""
    S = scores(q, k, scale, causal)
    P, _, lse = _softmax_rows(S)
    Pd = P * keep / (1.0 - p_drop)
    return Pd @ np.asarray(v, dtype=np.float64), lse


def backward_head_dropout(q, k, v, do, scale, causal, keep, p_drop):
    """(dQ, dK, dV) of sum(O o dO) for the dropout forward above."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    P = probs_head(q, k, scale, causal)
    zs = keep / (1.0 - p_drop)
    dv = (P * zs).T @ do                      # O = (P zs) V
    dP = (do @ v.T) * zs                      # gradient reaching P
    rowdot = (P * dP).sum(axis=1)             # <p, dp> per row, eq. (30)
    dS = P * (dP - rowdot[:, None])
    return scale * (dS @ k), scale * (dS.T @ q), dv


# ---------------------------------------------------------------- KV cache: fewer queries than keys
# FlashAttention-2 notes, "impact on the KV cache" (MQA/GQA shrink the
# cache that decoding reads): at a decoding step a few new queries (often
# one) attend to every cached key of their sequence.  q [B, H, Nq, d];
# k, v [B, Hkv, Nk, d] hold Nk cache slots, of which the first L_b are
# valid for sequence b (cache_lens, default all Nk).  The queries are the
# last Nq positions of a sequence of L_b tokens: under the causal rule,
# query i sees key j iff j <= i + L_b - Nq (``allowed`` above).

def forward_kvcache(q, k, v, scale, causal=False, cache_lens=None, heads=None):
    """-> {(b, h): (O [Nq, d], LSE [Nq])}; each query head attends over its
    group's K/V head, keys 0 .. L_b - 1."""
    B, H, Nq = q.shape[:3]
    Hkv, Nk = k.shape[1], k.shape[2]
    out = {}
    for (b, h) in _heads(B, H, heads):
        L = Nk if cache_lens is None else int(cache_lens[b])
        g = kv_head_of(h, H, Hkv)
        if L == 0:
            out[(b, h)] = (np.zeros((Nq, q.shape[3])), np.full(Nq, -np.inf))
            continue
        out[(b, h)] = forward_head(q[b, h], k[b, g, :L], v[b, g, :L], scale, causal)
    return out
