"""Pins of the CPU oracle against what the pages and mathematics fix.

Nothing here compares the oracle with itself: every check is a worked
example printed on a page, a closed form, a finite-difference gradient, a
pure-Python brute force on tiny inputs, or an invariant that follows from
the definition.  Runs on the CPU (no ``gpu`` marker).
"""
import json
import math
import os
import re

import numpy as np
import pytest

from oracle import attention as A
from oracle import online as OL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- brute force
def brute_attention(q, k, v, scale, ok):
    """Pure-Python loops with math.exp / math.fsum; independent of numpy code."""
    n, d = len(q), len(q[0])
    nk = len(k)
    O, L = [], []
    for i in range(n):
        s = []
        for j in range(nk):
            if ok(i, j):
                s.append((j, scale * math.fsum(q[i][t] * k[j][t] for t in range(d))))
        if not s:
            O.append([0.0] * d)
            L.append(-math.inf)
            continue
        mx = max(x for _, x in s)
        e = [(j, math.exp(x - mx)) for j, x in s]
        tot = math.fsum(w for _, w in e)
        O.append([math.fsum(w * v[j][t] for j, w in e) / tot for t in range(len(v[0]))])
        L.append(mx + math.log(tot))
    return np.array(O), np.array(L)


# ------------------------------------------------------- P1 worked example
def test_worked_example_three_tiles():
    g = json.load(open(os.path.join(GOLDEN, "online_softmax_worked_example.json")))
    tiles = g["tiles"]
    hist = OL.online_stats(tiles)
    ms = [m for m, _ in hist]
    ls = [l for _, l in hist]
    assert ms == g["printed_m"]
    assert round(ls[0], 2) == pytest.approx(g["printed_l"][0], abs=1e-12)
    # l_1, l_2 from the recurrence's closed forms (the page's printed 1.88 /
    # 3.03 do not follow from its own formulas; see the fixture's note)
    l0 = 1.0 + math.exp(-1.0)
    l1 = l0 * math.exp(-1.0) + 1.0 + math.exp(-2.5)
    l2 = l1 + math.exp(-1.5) + math.exp(-0.5)
    assert ls[0] == pytest.approx(l0, rel=1e-15)
    assert ls[1] == pytest.approx(l1, rel=1e-15)
    assert ls[2] == pytest.approx(l2, rel=1e-15)
    assert ls[1] == pytest.approx(1.58530, abs=1e-5)
    assert ls[2] == pytest.approx(2.41496, abs=1e-5)
    assert abs(ls[1] - g["printed_l"][1]) > 0.2 and abs(ls[2] - g["printed_l"][2]) > 0.5

    # the same six scores through the plain oracle: q = [1], k_j = score_j
    flat = [x for t in tiles for x in t]
    q = np.array([[1.0]])
    k = np.array([[x] for x in flat])
    v = _rng(1).standard_normal((6, 3))
    O, L = A.forward_head(q, k, v, 1.0)
    assert L[0] == pytest.approx(3.881683, abs=1e-6)
    assert L[0] == pytest.approx(ms[-1] + math.log(ls[-1]), rel=1e-15)
    P = A.probs_head(q, k, 1.0)[0]
    expect = [0.15233, 0.05604, 0.41409, 0.03399, 0.09239, 0.25116]
    np.testing.assert_allclose(P, expect, atol=5e-6)
    # output through the deferred-normalisation recurrence, tile width 2
    O2, L2 = OL.fa2_forward(q, k, v, 1.0, br=1, bc=2)
    np.testing.assert_allclose(O2, O, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(O[0], P @ v, rtol=1e-14)


# ------------------------------------------------------- P2 Theorem 1
@pytest.mark.parametrize("n,nk_eq,br,bc,causal", [
    (37, True, 8, 5, False), (37, True, 7, 16, True), (64, True, 16, 16, True),
    (50, True, 50, 3, False), (1, True, 1, 1, False), (29, True, 1, 29, True),
])
def test_theorem1_blocked_equals_plain(n, nk_eq, br, bc, causal):
    r = _rng(n * 131 + br)
    d = 6
    q, k, v = (r.standard_normal((n, d)) * 1.5 for _ in range(3))
    s = 0.37
    O, L = A.forward_head(q, k, v, s, causal)
    O1, m1, l1 = OL.fa1_forward(q, k, v, s, br, bc, causal)
    O2, L2 = OL.fa2_forward(q, k, v, s, br, bc, causal)
    np.testing.assert_allclose(O1, O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(O2, O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(m1 + np.log(l1), L, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L2, L, rtol=1e-12, atol=1e-13)


def test_theorem1_invariants_after_each_outer_step():
    """After outer step j: m = rowmax S[:, :j], l = rowsum exp(S[:, :j] - m),
    O = softmax(S[:, :j]) V[:j]  (paper summary, Theorem 1 proof sketch)."""
    r = _rng(7)
    n, d = 23, 4
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    s = 0.8
    trace = []
    OL.fa1_forward(q, k, v, s, br=6, bc=5, trace=trace)
    S = s * q @ k.T
    for c1, m, l, O in trace:
        sub = S[:, :c1]
        mref = sub.max(axis=1)
        np.testing.assert_allclose(m, mref, rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(l, np.exp(sub - mref[:, None]).sum(axis=1), rtol=1e-13)
        Pref = np.exp(sub - mref[:, None]) / np.exp(sub - mref[:, None]).sum(axis=1, keepdims=True)
        np.testing.assert_allclose(O, Pref @ v[:c1], rtol=1e-12, atol=1e-14)


def test_two_block_proof_eq14():
    """The two-block derivation: e^{m1-m} O~1 + e^{S2-m} V2 over l equals the
    softmax of the concatenated scores times stacked V (FA2 notes, eq. (14))."""
    r = _rng(3)
    S1, S2 = r.standard_normal((4, 3)) * 3, r.standard_normal((4, 5)) * 3
    V1, V2 = r.standard_normal((3, 2)), r.standard_normal((5, 2))
    m1 = S1.max(1)
    m = np.maximum(m1, S2.max(1))
    O1 = np.exp(S1 - m1[:, None]) @ V1
    O2 = np.exp(m1 - m)[:, None] * O1 + np.exp(S2 - m[:, None]) @ V2
    l2 = np.exp(S1 - m[:, None]).sum(1) + np.exp(S2 - m[:, None]).sum(1)
    S = np.concatenate([S1, S2], 1)
    ref = (np.exp(S) / np.exp(S).sum(1, keepdims=True)) @ np.concatenate([V1, V2])
    np.testing.assert_allclose(O2 / l2[:, None], ref, rtol=1e-13)


def test_inverse_rescale_reading_is_wrong():
    """The notes print the per-step factor as diag(e^{m_old-m_new})^{-1};
    taken literally that breaks Theorem 1, so the multiply reading is used."""
    r = _rng(11)
    q, k, v = (r.standard_normal((32, 8)) * 2 for _ in range(3))
    O, _ = A.forward_head(q, k, v, 0.5)
    Obad, _ = OL.fa2_forward(q, k, v, 0.5, 8, 4, inverse_rescale=True)
    assert np.abs(Obad - O).max() > 1e-3


def test_state_merge_of_two_halves():
    """Merging the softmax states of two key halves gives the full result
    (languisher.top notes, merging two vectors' statistics)."""
    r = _rng(5)
    q, k, v = (r.standard_normal((9, 3)) for _ in range(3))
    k2, v2 = r.standard_normal((7, 3)), r.standard_normal((7, 3))
    s = 0.9
    O1, L1 = A.forward_head(q, k, v, s)
    O2, L2 = A.forward_head(q, k2, v2, s)
    m, l, O = OL.merge_states((L1, np.ones(9), O1), (L2, np.ones(9), O2))
    Of, Lf = brute_attention(q.tolist(), np.vstack([k, k2]).tolist(), np.vstack([v, v2]).tolist(),
                             s, lambda i, j: True)
    np.testing.assert_allclose(O, Of, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(m + np.log(l), Lf, rtol=1e-13)


# ------------------------------------------------------- brute force (P8 part)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_plain_matches_pure_python_bruteforce(causal, masked):
    r = _rng(17 + causal + 2 * masked)
    n, d, mb = 11, 3, 3
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    T = (n + mb - 1) // mb
    bm = (r.random((T, T)) < 0.5).astype(np.uint8) if masked else None
    if masked:
        np.fill_diagonal(bm, 1)
    s = 0.6

    def ok(i, j):
        if causal and j > i:
            return False
        if bm is not None and not bm[i // mb][j // mb]:
            return False
        return True

    O, L = A.forward_head(q, k, v, s, causal, bm, mask_block=mb)
    Ob, Lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), s, ok)
    np.testing.assert_allclose(O, Ob, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(L, Lb, rtol=1e-13, atol=1e-15)


# ------------------------------------------------------- P3 / P4
@pytest.mark.parametrize("causal", [False, True])
def test_rows_are_distributions_and_lse_bounds(causal):
    r = _rng(23)
    n, d = 40, 8
    q, k = r.standard_normal((n, d)) * 3, r.standard_normal((n, d)) * 3
    bm = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    for mask in (None, bm):
        ok = A.allowed(n, n, causal, mask, mask_block=16)
        P = A.probs_head(q, k, 0.4, causal, mask, mask_block=16)
        np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-14)
        assert (P[ok] > 0).all() and (P[ok] <= 1).all() and (P[~ok] == 0).all()
        S = A.scores(q, k, 0.4, causal, mask, mask_block=16)
        _, L = A.forward_head(q, k, np.eye(n, d), 0.4, causal, mask, mask_block=16)
        m = S.max(1)
        nrow = ok.sum(1)
        assert (m <= L + 1e-12).all() and (L <= m + np.log(nrow) + 1e-12).all()
        # P = exp(S - L) in (0, 1] (FA2 notes, eq. (16) and eq. (24))
        np.testing.assert_allclose(np.exp(S - L[:, None]), P, rtol=1e-13, atol=1e-300)


# ------------------------------------------------------- P5 finite differences
def _loss(q, k, v, do, s, causal, bm, mb):
    O, _ = A.forward_head(q, k, v, s, causal, bm, mb)
    return float((O * do).sum())


@pytest.mark.parametrize("n,d", [(1, 1), (2, 2), (3, 4), (5, 2), (8, 4)])
@pytest.mark.parametrize("mode", ["dense", "causal", "mask"])
def test_gradients_by_central_differences(n, d, mode):
    r = _rng(n * 10 + d + len(mode))
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    s = 0.7
    causal = mode == "causal"
    mb = 2
    bm = None
    if mode == "mask":
        T = (n + mb - 1) // mb
        bm = (r.random((T, T)) < 0.6).astype(np.uint8)
        np.fill_diagonal(bm, 1)
    dq, dk, dv = A.backward_head(q, k, v, do, s, causal, bm, mb)
    h = 1e-6
    for X, G in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            old = X[idx]
            X[idx] = old + h
            fp = _loss(q, k, v, do, s, causal, bm, mb)
            X[idx] = old - h
            fm = _loss(q, k, v, do, s, causal, bm, mb)
            X[idx] = old
            num[idx] = (fp - fm) / (2 * h)
        scale = max(1.0, np.abs(G).max())
        assert np.abs(num - G).max() <= 1e-6 * scale


# ------------------------------------------------------- P6 D identity
@pytest.mark.parametrize("causal", [False, True])
def test_D_identity(causal):
    """rowsum(dO o O) = <P_i, dP_i>  (paper summary, Technique 2; FA2 notes,
    backward precompute)."""
    r = _rng(29)
    n, d = 33, 5
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    O, _ = A.forward_head(q, k, v, 0.5, causal)
    P = A.probs_head(q, k, 0.5, causal)
    dP = do @ v.T
    np.testing.assert_allclose((do * O).sum(1), (P * dP).sum(1), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------- P7 closed forms
def test_closed_forms():
    r = _rng(31)
    d = 4
    # N = 1: O = V, LSE = s q.k
    q, k, v = (r.standard_normal((1, d)) for _ in range(3))
    O, L = A.forward_head(q, k, v, 0.3)
    np.testing.assert_allclose(O, v, rtol=1e-15)
    assert L[0] == pytest.approx(0.3 * float(q[0] @ k[0]), rel=1e-14)
    # all keys equal: uniform P over allowed keys
    n = 9
    q = r.standard_normal((n, d))
    k = np.tile(r.standard_normal((1, d)), (n, 1))
    v = r.standard_normal((n, d))
    for causal in (False, True):
        O, L = A.forward_head(q, k, v, 0.3, causal)
        for i in range(n):
            cnt = i + 1 if causal else n
            np.testing.assert_allclose(O[i], v[:cnt].mean(0), rtol=1e-13, atol=1e-15)
            assert L[i] == pytest.approx(0.3 * float(q[i] @ k[0]) + math.log(cnt), rel=1e-13)
    # causal row 0 sees only key 0
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    O, L = A.forward_head(q, k, v, 0.3, True)
    np.testing.assert_allclose(O[0], v[0], rtol=1e-15)
    assert L[0] == pytest.approx(0.3 * float(q[0] @ k[0]), rel=1e-14)


# ------------------------------------------------------- P8 masks
def test_mask_special_cases():
    r = _rng(37)
    n, d, mb = 12, 3, 4
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    T = n // mb
    ones = np.ones((T, T), np.uint8)
    O0, L0 = A.forward_head(q, k, v, 0.5)
    O1, L1 = A.forward_head(q, k, v, 0.5, False, ones, mb)
    np.testing.assert_array_equal(O0, O1)
    np.testing.assert_array_equal(L0, L1)
    g0 = A.backward_head(q, k, v, do, 0.5)
    g1 = A.backward_head(q, k, v, do, 0.5, False, ones, mb)
    for a, b in zip(g0, g1):
        np.testing.assert_array_equal(a, b)
    # diagonal-only mask: each block attends only within itself
    diag = np.eye(T, dtype=np.uint8)
    O, L = A.forward_head(q, k, v, 0.5, False, diag, mb)
    for t in range(T):
        sl = slice(t * mb, (t + 1) * mb)
        Ob, Lb = brute_attention(q[sl].tolist(), k[sl].tolist(), v[sl].tolist(), 0.5, lambda i, j: True)
        np.testing.assert_allclose(O[sl], Ob, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(L[sl], Lb, rtol=1e-13)


def test_fully_masked_rows_convention():
    """A row with no allowed key gives O = 0, LSE = -inf and no NaN anywhere."""
    r = _rng(41)
    n, d, mb = 8, 3, 4
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    bm = np.array([[0, 0], [1, 1]], np.uint8)   # rows 0..3 see nothing
    O, L = A.forward_head(q, k, v, 0.5, False, bm, mb)
    assert (O[:4] == 0).all() and np.isneginf(L[:4]).all() and np.isfinite(L[4:]).all()
    dq, dk, dv = A.backward_head(q, k, v, do, 0.5, False, bm, mb)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    assert (dq[:4] == 0).all()


# ------------------------------------------------------- P9 gradient invariants
@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(causal):
    r = _rng(43)
    n, d = 30, 6
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    dq, dk, dv = A.backward_head(q, k, v, do, 0.45, causal)
    np.testing.assert_allclose(dk.sum(0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(0), do.sum(0), rtol=1e-12, atol=1e-12)


def test_row_chunking_changes_nothing():
    r = _rng(47)
    n, d = 40, 4
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    a = A.backward_head(q, k, v, do, 0.5, True, chunk=n)
    b = A.backward_head(q, k, v, do, 0.5, True, chunk=7)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)


def test_oracle_is_independent_of_gpu_package():
    here = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle")
    for f in os.listdir(here):
        if f.endswith(".py"):
            src = open(os.path.join(here, f)).read()
            assert not re.search(r"^\s*(import|from)\s+io_aware_exact_flash_amd", src, re.M)
            assert "ctypes" not in src and "torch" not in src


# ------------------------------------------------------- the pins have teeth
def _planted_backward(q, k, v, do, s, causal, bug):
    """Chain rule with one plausible mistake planted (CPU only)."""
    P = A.probs_head(q, k, s, causal)
    dP = do @ v.T
    rowdot = (P * dP).sum(1)
    if bug == "drop_D":
        rowdot = 0 * rowdot
    dS = P * (dP - rowdot[:, None])
    if bug == "sign":
        dS = -dS
    dq = s * dS @ k
    dk = s * dS.T @ q
    dv = P.T @ do if bug != "transpose" else P @ do
    if bug == "no_scale":
        dq, dk = dq / s, dk / s
    return dq, dk, dv


@pytest.mark.parametrize("bug", ["drop_D", "sign", "transpose", "no_scale"])
def test_finite_differences_catch_planted_mistakes(bug):
    r = _rng(53)
    n, d = 5, 3
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    s = 0.7
    good = A.backward_head(q, k, v, do, s, True)
    bad = _planted_backward(q, k, v, do, s, True, bug)
    h = 1e-6
    worst = 0.0
    for X, Gg, Gb in zip((q, k, v), good, bad):
        for idx in np.ndindex(*X.shape):
            old = X[idx]
            X[idx] = old + h
            fp = _loss(q, k, v, do, s, True, None, 128)
            X[idx] = old - h
            fm = _loss(q, k, v, do, s, True, None, 128)
            X[idx] = old
            num = (fp - fm) / (2 * h)
            assert abs(num - Gg[idx]) <= 1e-6 * max(1.0, np.abs(Gg).max())
            worst = max(worst, abs(num - Gb[idx]))
    assert worst > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_row_restricted_dq_by_finite_differences(causal):
    """grad_q_rows on a subset of rows against central differences."""
    r = _rng(59)
    n, d = 6, 3
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    rows = [0, 3, 5]
    g = A.grad_q_rows(q, k, v, do, 0.6, causal, rows=rows)
    h = 1e-6
    for a, i in enumerate(rows):
        for t in range(d):
            old = q[i, t]
            q[i, t] = old + h
            fp = _loss(q, k, v, do, 0.6, causal, None, 128)
            q[i, t] = old - h
            fm = _loss(q, k, v, do, 0.6, causal, None, 128)
            q[i, t] = old
            assert abs((fp - fm) / (2 * h) - g[a, t]) <= 1e-6 * max(1.0, np.abs(g).max())


# ------------------------------------------------------- P9 grouped K/V heads
def test_gqa_group_map():
    """FA2 notes, "MQA and GQA support": a single K/V head serves every query
    head (MQA); one K/V head per query head is plain multi-head attention;
    otherwise runs of H / Hkv consecutive query heads share one K/V head."""
    assert [A.kv_head_of(h, 8, 1) for h in range(8)] == [0] * 8
    assert [A.kv_head_of(h, 8, 8) for h in range(8)] == list(range(8))
    assert [A.kv_head_of(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [A.kv_head_of(h, 6, 3) for h in range(6)] == [0, 0, 1, 1, 2, 2]
    for H, Hkv in ((6, 4), (4, 0), (3, -1)):
        with pytest.raises(ValueError):
            A.kv_head_of(0, H, Hkv)


@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (3, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_gqa_forward_against_broadcast_bruteforce(H, Hkv, causal):
    """Grouped forward equals pure-Python attention over K/V heads broadcast
    to every query head (the copy the notes say the kernels avoid)."""
    r = _rng(100 + 10 * H + Hkv + causal)
    B, n, d = 2, 5, 3
    q = r.standard_normal((B, H, n, d))
    k = r.standard_normal((B, Hkv, n, d))
    v = r.standard_normal((B, Hkv, n, d))
    krep = np.repeat(k, H // Hkv, axis=1)  # [B, H, n, d]
    vrep = np.repeat(v, H // Hkv, axis=1)
    got = A.forward_gqa(q, k, v, 0.6, causal)
    ok = (lambda i, j: j <= i) if causal else (lambda i, j: True)
    for b in range(B):
        for h in range(H):
            O, L = brute_attention(q[b, h].tolist(), krep[b, h].tolist(), vrep[b, h].tolist(), 0.6, ok)
            np.testing.assert_allclose(got[(b, h)][0], O, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(got[(b, h)][1], L, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("H,Hkv,causal", [(4, 2, False), (3, 1, True), (2, 2, True)])
def test_gqa_gradients_by_central_differences(H, Hkv, causal):
    """dK, dV of a shared head sum over its group: checked against central
    differences of the total loss sum_h sum(O_h o dO_h)."""
    r = _rng(7 * H + Hkv)
    B, n, d, s = 1, 4, 2, 0.8
    q = r.standard_normal((B, H, n, d))
    k = r.standard_normal((B, Hkv, n, d))
    v = r.standard_normal((B, Hkv, n, d))
    do = r.standard_normal((B, H, n, d))

    def loss():
        out = A.forward_gqa(q, k, v, s, causal)
        return float(sum((out[(0, h)][0] * do[0, h]).sum() for h in range(H)))

    dq, dk, dv = A.backward_gqa(q, k, v, do, s, causal)
    G = {"q": np.stack([dq[(0, h)] for h in range(H)])[None],
         "k": np.stack([dk[(0, g)] for g in range(Hkv)])[None],
         "v": np.stack([dv[(0, g)] for g in range(Hkv)])[None]}
    eps = 1e-6
    for name, X in (("q", q), ("k", k), ("v", v)):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            old = X[idx]
            X[idx] = old + eps
            fp = loss()
            X[idx] = old - eps
            fm = loss()
            X[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        assert np.abs(num - G[name]).max() <= 1e-6 * max(1.0, np.abs(G[name]).max()), name


# ------------------------------------------------------- P10 packed variable-length batches
def test_varlen_each_sequence_is_its_own_problem():
    """Packed sequences against pure-Python attention on each sequence alone
    (causal positions counted from the sequence start), with grouped heads;
    an empty sequence contributes nothing."""
    r = _rng(41)
    lens, H, Hkv, d, s = [3, 0, 5, 1], 4, 2, 3, 0.7
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = r.standard_normal((T, H, d))
    k = r.standard_normal((T, Hkv, d))
    v = r.standard_normal((T, Hkv, d))
    for causal in (False, True):
        O, L = A.forward_varlen(q, k, v, cu, s, causal)
        ok = (lambda i, j: j <= i) if causal else (lambda i, j: True)
        for b in range(len(lens)):
            a, e = cu[b], cu[b + 1]
            for h in range(H):
                g = h // (H // Hkv)
                if e == a:
                    continue
                Ob, Lb = brute_attention(q[a:e, h].tolist(), k[a:e, g].tolist(), v[a:e, g].tolist(), s, ok)
                np.testing.assert_allclose(O[a:e, h], Ob, rtol=1e-12, atol=1e-13)
                np.testing.assert_allclose(L[h, a:e], Lb, rtol=1e-12, atol=1e-13)
        # changing the tokens of one sequence leaves the others untouched
        q2 = q.copy()
        q2[cu[2]:cu[3]] += 1.0
        O2, _ = A.forward_varlen(q2, k, v, cu, s, causal)
        np.testing.assert_array_equal(O2[:cu[2]], O[:cu[2]])
        np.testing.assert_array_equal(O2[cu[3]:], O[cu[3]:])


def test_varlen_gradients_by_central_differences():
    r = _rng(43)
    lens, H, Hkv, d, s = [3, 2], 2, 1, 2, 0.9
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = r.standard_normal((T, H, d))
    k = r.standard_normal((T, Hkv, d))
    v = r.standard_normal((T, Hkv, d))
    do = r.standard_normal((T, H, d))
    for causal in (False, True):
        G = dict(zip("qkv", A.backward_varlen(q, k, v, do, cu, s, causal)))
        eps = 1e-6
        for name, X in (("q", q), ("k", k), ("v", v)):
            num = np.zeros_like(X)
            for idx in np.ndindex(*X.shape):
                old = X[idx]
                X[idx] = old + eps
                fp = float((A.forward_varlen(q, k, v, cu, s, causal)[0] * do).sum())
                X[idx] = old - eps
                fm = float((A.forward_varlen(q, k, v, cu, s, causal)[0] * do).sum())
                X[idx] = old
                num[idx] = (fp - fm) / (2 * eps)
            assert np.abs(num - G[name]).max() <= 1e-6 * max(1.0, np.abs(G[name]).max()), (name, causal)


# ------------------------------------------------------- P11 dropout
from oracle import philox as PX  # noqa: E402


def test_philox_known_answers():
    """Philox4x32-10 against the published known-answer vectors of the
    Random123 library (counter, key) -> output."""
    kat = [
        ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
        ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
        ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
         (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
    ]
    for ctr, key, out in kat:
        assert tuple(int(w) for w in PX.philox4x32(ctr, key)) == out


def test_dropout_threshold_and_keep_rate():
    assert PX.drop_threshold(0.0) == 0 and PX.drop_threshold(0.1) == 26 and PX.drop_threshold(0.5) == 128
    for bad in (-0.1, 1.0, 0.999):
        with pytest.raises(ValueError):
            PX.drop_threshold(bad)
    assert PX.keep_matrix(64, 64, 0, 1, 0, 0).all()  # t = 0 keeps everything
    t = PX.drop_threshold(0.3)
    Z = PX.keep_matrix(512, 512, 3, 1234, 7, t)
    rate, expect = Z.mean(), 1 - t / 256
    assert abs(rate - expect) < 5 * math.sqrt(expect * (1 - expect) / Z.size)
    # another head, offset or seed draws a different stream
    for other in (PX.keep_matrix(512, 512, 4, 1234, 7, t), PX.keep_matrix(512, 512, 3, 1234, 8, t),
                  PX.keep_matrix(512, 512, 3, 1235, 7, t)):
        assert 0.4 < (other == Z).mean() < 0.7


def test_dropout_keep_matrix_layout():
    """Element (i, j) reads byte j % 4 of word i % 4 of the draw for counter
    (i // 4, j // 4, head, offset)."""
    seed, head, off, t = (7 << 32) | 99, 5, 3, 100
    Z = PX.keep_matrix(9, 10, head, seed, off, t)
    for i in range(9):
        for j in range(10):
            words = PX.philox4x32((i // 4, j // 4, head, off), (seed & 0xFFFFFFFF, seed >> 32))
            assert Z[i, j] == (((int(words[i % 4]) >> (8 * (j % 4))) & 0xFF) >= t)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_zero_rate_is_plain_attention(causal):
    r = _rng(61)
    n, d = 37, 8
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    keep = np.ones((n, n), dtype=bool)
    O, L = A.forward_head_dropout(q, k, v, 0.4, causal, keep, 0.0)
    O0, L0 = A.forward_head(q, k, v, 0.4, causal)
    np.testing.assert_array_equal(O, O0)
    np.testing.assert_array_equal(L, L0)
    for a, b in zip(A.backward_head_dropout(q, k, v, do, 0.4, causal, keep, 0.0),
                    A.backward_head(q, k, v, do, 0.4, causal)):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_gradients_by_central_differences(causal):
    """With the keep decisions fixed the dropout forward is smooth; its
    gradient against central differences of sum(O o dO)."""
    r = _rng(67 + causal)
    n, d, s, p = 6, 3, 0.8, 0.25
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    keep = r.random((n, n)) >= p
    G = dict(zip("qkv", A.backward_head_dropout(q, k, v, do, s, causal, keep, p)))
    eps = 1e-6
    for name, X in (("q", q), ("k", k), ("v", v)):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            old = X[idx]
            X[idx] = old + eps
            fp = float((A.forward_head_dropout(q, k, v, s, causal, keep, p)[0] * do).sum())
            X[idx] = old - eps
            fm = float((A.forward_head_dropout(q, k, v, s, causal, keep, p)[0] * do).sum())
            X[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        assert np.abs(num - G[name]).max() <= 1e-6 * max(1.0, np.abs(G[name]).max()), name


# Inverted dropout is defined so that the dropped output is an unbiased
# estimate of the plain one: E_Z[(P o Z) V / (1 - p')] = P V because each
# keep decision holds with probability 1 - p'.  O, and through it D and dS,
# are linear in Z, so the same holds for every gradient.  Averaging over
# independent Philox streams (offsets) must reproduce the plain attention;
# a wrong factor (multiplying by 1 - p' instead of dividing, or no factor)
# leaves a bias many standard errors wide.
def _dropout_average(fn, n_draws, n, t, seed):
    outs = []
    for off in range(n_draws):
        keep = PX.keep_matrix(n, n, 0, seed, off, t)
        outs.append(np.concatenate([np.ravel(x) for x in fn(keep)]))
    X = np.stack(outs)
    return X.mean(0), X.std(0, ddof=1) / math.sqrt(n_draws)


def _bias_statistic(mean, sem, ref):
    """(mean squared z-score, max |z|) over elements with spread; elements
    with none must already equal the reference."""
    live = sem > 1e-12
    assert np.allclose(mean[~live], ref[~live], atol=1e-12)
    z = (mean[live] - ref[live]) / sem[live]
    return float(np.mean(z * z)), float(np.abs(z).max())


@pytest.mark.parametrize("p", [0.1, 0.5])
@pytest.mark.parametrize("causal", [False, True])
def test_dropout_is_unbiased_and_wrong_factors_are_caught(p, causal):
    r = _rng(71 + int(10 * p) + causal)
    n, d, s, draws = 20, 3, 0.7, 600
    q, k, v, do = (r.standard_normal((n, d)) for _ in range(4))
    t = PX.drop_threshold(p)
    pd = t / 256.0
    plain = np.concatenate([np.ravel(x) for x in (A.forward_head(q, k, v, s, causal)[0],
                                                  *A.backward_head(q, k, v, do, s, causal))])

    def right(keep):
        return (A.forward_head_dropout(q, k, v, s, causal, keep, pd)[0],
                *A.backward_head_dropout(q, k, v, do, s, causal, keep, pd))

    mean, sem = _dropout_average(right, draws, n, t, seed=99)
    chi2, zmax = _bias_statistic(mean, sem, plain)
    # z-scores of an unbiased estimate: mean square about 1, none beyond ~5
    assert chi2 < 2.0 and zmax < 5.5, (chi2, zmax)

    # planted mistakes, applied to the oracle's outputs on the CPU: every
    # output of the dropout path is linear in the factor, so scaling the
    # results by (1 - p')^2 is the multiply-instead-of-divide mistake and by
    # (1 - p') the dropped factor
    for wrong in ((1.0 - pd) ** 2, 1.0 - pd):
        def planted(keep, f=wrong):
            return tuple(f * x for x in right(keep))
        mean_b, sem_b = _dropout_average(planted, draws, n, t, seed=99)
        chi2_b, _ = _bias_statistic(mean_b, sem_b, plain)
        assert chi2_b > 10.0, (wrong, chi2_b)


# ------------------------------------------------------- P12 fewer queries than keys (KV cache)
def test_kvcache_causal_reading_reduces_to_square_case_and_last_query_sees_all():
    """With n_q = n_k the causal rule is j <= i; with n_q < n_k the last
    query sees every key and query i sees keys 0 .. n_k - n_q + i."""
    for n in (1, 5, 33):
        ok = A.allowed(n, n, True)
        assert (ok == np.tril(np.ones((n, n), dtype=bool))).all()
    for nq, nk in ((1, 40), (3, 17), (7, 7), (5, 2)):
        ok = A.allowed(nq, nk, True)
        for i in range(nq):
            assert ok[i].sum() == max(0, min(nk, nk - nq + i + 1))
        if nk >= nq:
            assert ok[-1].all()


@pytest.mark.parametrize("nq,nk", [(1, 37), (4, 37), (37, 37), (6, 3)])
def test_kvcache_forward_against_bruteforce(nq, nk):
    r = _rng(101 + nq + nk)
    d, s = 5, 0.6
    q = r.standard_normal((nq, d))
    k, v = r.standard_normal((nk, d)), r.standard_normal((nk, d))
    for causal in (False, True):
        O, L = A.forward_head(q, k, v, s, causal)
        Ob, Lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), s,
                                 lambda i, j: (not causal) or j <= i + nk - nq)
        np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(np.isneginf(L), np.isneginf(Lb))
        fin = np.isfinite(Lb)
        np.testing.assert_allclose(L[fin], Lb[fin], rtol=1e-12, atol=1e-12)


def test_kvcache_decoding_continues_the_sequence():
    """The reading that the queries are the last positions of their
    sequence: attending the last n_q queries of a causal self-attention
    problem over the whole key set reproduces that problem's last n_q rows
    (computed with equal lengths, j <= i)."""
    r = _rng(107)
    n, d, s = 29, 6, 0.45
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    Ofull, Lfull = A.forward_head(q, k, v, s, True)
    for nq in (1, 2, 9, n):
        O, L = A.forward_head(q[n - nq:], k, v, s, True)
        np.testing.assert_allclose(O, Ofull[n - nq:], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(L, Lfull[n - nq:], rtol=1e-13, atol=1e-13)


def test_kvcache_grouped_heads_and_cache_lengths():
    """forward_kvcache: query head h reads K/V head h // (H / Hkv) over the
    first L_b cache slots only; slots past L_b never matter; an empty cache
    gives O = 0, LSE = -inf."""
    r = _rng(109)
    B, H, Hkv, nq, nk, d, s = 3, 4, 2, 2, 11, 4, 0.7
    q = r.standard_normal((B, H, nq, d))
    k, v = r.standard_normal((B, Hkv, nk, d)), r.standard_normal((B, Hkv, nk, d))
    lens = [11, 6, 0]
    out = A.forward_kvcache(q, k, v, s, True, lens)
    k2, v2 = k.copy(), v.copy()
    k2[1, :, 6:] = 1e3  # garbage past the valid slots
    v2[1, :, 6:] = -7.0
    out2 = A.forward_kvcache(q, k2, v2, s, True, lens)
    for b in range(B):
        for h in range(H):
            g = h // (H // Hkv)
            if lens[b] == 0:
                assert (out[(b, h)][0] == 0).all() and np.isneginf(out[(b, h)][1]).all()
                continue
            L = lens[b]
            Ob, Lb = brute_attention(q[b, h].tolist(), k[b, g, :L].tolist(), v[b, g, :L].tolist(), s,
                                     lambda i, j: j <= i + L - nq)
            np.testing.assert_allclose(out[(b, h)][0], Ob, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(out[(b, h)][1], Lb, rtol=1e-12, atol=1e-12)
            np.testing.assert_array_equal(out2[(b, h)][0], out[(b, h)][0])
