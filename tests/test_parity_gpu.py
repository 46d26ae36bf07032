"""GPU parity: the C-ABI kernels against the float64 oracle, element by element.

Sizes are small enough for the oracle to finish in seconds yet span several
key tiles (64 keys at d=128, 128 at d=64), several 128-row query blocks and a
ragged tail (N not a multiple of any tile).
"""
import numpy as np
import pytest
import torch

from io_aware_exact_flash_amd import flash, workloads
from oracle import attention as A
from tests._parity import REL_RMS, TOL, compare, compare_lse, fp32_scale, make, to64

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _oracle_fwd(f64, s, causal, mask=None):
    q, k, v = f64[:3]
    B, H = q.shape[:2]
    O = np.zeros(q.shape)
    L = np.zeros(q.shape[:3])
    for b in range(B):
        for h in range(H):
            O[b, h], L[b, h] = A.forward_head(q[b, h], k[b, h], v[b, h], s, causal, mask)
    return O, L


def _oracle_bwd(f64, s, causal, mask=None):
    q, k, v, do = f64
    B, H = q.shape[:2]
    out = [np.zeros(q.shape) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            g = A.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], s, causal, mask)
            for t in range(3):
                out[t][b, h] = g[t]
    return out


SHAPES = [(2, 2, 1), (2, 2, 17), (1, 2, 128), (2, 1, 200), (1, 2, 384), (1, 1, 519)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_backward_small(dtype, d, causal, shape):
    B, H, N = shape
    seed = 100 + N + d + 7 * causal
    (q, k, v, do), f64 = make(B, H, N, d, dtype, seed)
    s = fp32_scale(d)
    o, lse = flash.fwd(q, k, v, scale=s, causal=causal)
    dq, dk, dv = flash.bwd(q, k, v, o, do, lse, scale=s, causal=causal)
    torch.cuda.synchronize()
    O, L = _oracle_fwd(f64, s, causal)
    tol = TOL[dtype]
    compare("O", o, O, tol["o"], REL_RMS[dtype])
    compare_lse("LSE", lse, L, tol["lse"])
    # the backward takes the GPU's own O and LSE (as a training step would);
    # the oracle gradient is the exact gradient at the same inputs
    gQ, gK, gV = _oracle_bwd(f64, s, causal)
    compare("dQ", dq, gQ, tol["grad"], REL_RMS[dtype])
    compare("dK", dk, gK, tol["grad"], REL_RMS[dtype])
    compare("dV", dv, gV, tol["grad"], REL_RMS[dtype])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 256), (2, 3, 100), (1, 2, 33), (1, 1, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_forward_float32(d, causal, shape):
    B, H, N = shape
    (q, k, v, _), f64 = make(B, H, N, d, "f32", seed=1 + N + d)
    s = fp32_scale(d)
    o, lse = flash.fwd(q, k, v, scale=s, causal=causal)
    torch.cuda.synchronize()
    O, L = _oracle_fwd(f64, s, causal)
    compare("O", o, O, TOL["f32"]["o"], REL_RMS["f32"])
    compare_lse("LSE", lse, L, TOL["f32"]["lse"])


def _masks(T, seed):
    g = torch.Generator().manual_seed(seed)
    rnd = (torch.rand((T, T), generator=g) < 0.4).to(torch.uint8)
    rnd.fill_diagonal_(1)
    return {
        "random": rnd,
        "diag": torch.eye(T, dtype=torch.uint8),
        "ones": torch.ones((T, T), dtype=torch.uint8),
        "seeded25": workloads.block_mask(T, 0.25, seed),
    }


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [256, 300, 640])
@pytest.mark.parametrize("kind", ["random", "diag", "ones", "seeded25"])
def test_blocksparse(dtype, d, causal, N, kind):
    B, H = 1, 2
    T = (N + 127) // 128
    mask_cpu = _masks(T, seed=N + d)[kind]
    (q, k, v, do), f64 = make(B, H, N, d, dtype, seed=7 + N + d)
    s = fp32_scale(d)
    m = mask_cpu.cuda()
    o, lse = flash.blocksparse_fwd(q, k, v, m, scale=s, causal=causal)
    dq, dk, dv = flash.blocksparse_bwd(q, k, v, o, do, lse, m, scale=s, causal=causal)
    torch.cuda.synchronize()
    mk = mask_cpu.numpy()
    O, L = _oracle_fwd(f64, s, causal, mk)
    tol = TOL[dtype]
    compare("O", o, O, tol["o"], REL_RMS[dtype])
    compare_lse("LSE", lse, L, tol["lse"])
    gQ, gK, gV = _oracle_bwd(f64, s, causal, mk)
    compare("dQ", dq, gQ, tol["grad"], REL_RMS[dtype])
    compare("dK", dk, gK, tol["grad"], REL_RMS[dtype])
    compare("dV", dv, gV, tol["grad"], REL_RMS[dtype])


def test_blocksparse_float32_forward():
    N, d = 384, 64
    T = 3
    mask_cpu = _masks(T, 5)["random"]
    (q, k, v, _), f64 = make(1, 2, N, d, "f32", seed=9)
    s = fp32_scale(d)
    o, lse = flash.blocksparse_fwd(q, k, v, mask_cpu.cuda(), scale=s)
    torch.cuda.synchronize()
    O, L = _oracle_fwd(f64, s, False, mask_cpu.numpy())
    compare("O", o, O, TOL["f32"]["o"], REL_RMS["f32"])
    compare_lse("LSE", lse, L, TOL["f32"]["lse"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rows_without_keys(dtype):
    """A zero diagonal mask block leaves rows with no allowed key: O = 0,
    LSE = -inf, and (16-bit) zero gradients for them, no NaN anywhere."""
    N, d = 256, 64
    mask_cpu = torch.tensor([[0, 0], [1, 1]], dtype=torch.uint8)
    (q, k, v, do), f64 = make(1, 1, N, d, dtype, seed=3)
    s = fp32_scale(d)
    o, lse = flash.blocksparse_fwd(q, k, v, mask_cpu.cuda(), scale=s)
    torch.cuda.synchronize()
    O, L = _oracle_fwd(f64, s, False, mask_cpu.numpy())
    assert (to64(o)[0, 0, :128] == 0).all()
    assert np.isneginf(to64(lse)[0, 0, :128]).all()
    tol = TOL[dtype]
    compare("O", o, O, tol["o"])
    compare_lse("LSE", lse, L, tol["lse"])
    if dtype != "f32":
        dq, dk, dv = flash.blocksparse_bwd(q, k, v, o, do, lse, mask_cpu.cuda(), scale=s)
        torch.cuda.synchronize()
        gQ, gK, gV = _oracle_bwd(f64, s, False, mask_cpu.numpy())
        assert (to64(dq)[0, 0, :128] == 0).all()
        compare("dQ", dq, gQ, tol["grad"])
        compare("dK", dk, gK, tol["grad"])
        compare("dV", dv, gV, tol["grad"])


def test_empty_inputs():
    for B, H, N in ((0, 2, 64), (1, 0, 64), (1, 2, 0)):
        q = torch.zeros((B, H, N, 64), dtype=torch.bfloat16, device="cuda")
        o, lse = flash.fwd(q, q, q)
        dq, dk, dv = flash.bwd(q, q, q, o, q, lse)
        torch.cuda.synchronize()
        assert o.shape == q.shape and lse.shape == (B, H, N) and dq.shape == q.shape


def test_large_magnitude_scores():
    """Scores of magnitude ~1e3 (Q, K drawn with gain 6, scale 1) exercise the
    max subtraction of the safe softmax; V and dO keep unit scale.

    Bounds: O and dV are the stated 16-bit bounds (their size is set by V and
    dO).  dQ = scale dS K and dK = scale dS^T Q are not: with scale 1 and
    gain-6 operands they reach ~1e2 instead of ~1.  Rounding errors of 16-bit
    arithmetic are relative to the size of the result, so their bound is
    stated relative to the largest gradient element: 2^-6 max|ref| (the
    ratio of the stated 5e-2 to the largest gradients, ~3, of unit-scale
    inputs), with the usual relative-RMS gate.  LSE: each score is a
    float32 dot product of d exactly representable products, so its
    rounding error is at most gamma_d sum_c |q_c| |k_c| (gamma_d = d u /
    (1 - d u), u = 2^-24, the classical dot-product bound); LSE is a smooth
    maximum of the scores (1-Lipschitz in their max norm), and the final
    m ln 2 + ln l adds a few roundings of |LSE|.  The bound per row is that
    sum over its allowed keys plus 8 u |LSE_i|."""
    N, d = 300, 128
    qk = workloads.qkvdo(1, 2, N, d, "bf16", seed=21, gain=6.0)
    vd = workloads.qkvdo(1, 2, N, d, "bf16", seed=22)
    cpu = (qk[0], qk[1], vd[2], vd[3])
    q, k, v, do = (t.cuda() for t in cpu)
    f64 = tuple(t.to(torch.float64).numpy() for t in cpu)
    s = 1.0
    o, lse = flash.fwd(q, k, v, scale=s, causal=True)
    dq, dk, dv = flash.bwd(q, k, v, o, do, lse, scale=s, causal=True)
    torch.cuda.synchronize()
    O, L = _oracle_fwd(f64, s, True)
    gQ, gK, gV = _oracle_bwd(f64, s, True)
    tol = TOL["bf16"]
    compare("O", o, O, tol["o"], REL_RMS["bf16"])
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    ok = A.allowed(N, N, True)
    lg = to64(lse)
    for h in range(2):
        a = np.where(ok, s * (np.abs(f64[0][0, h]) @ np.abs(f64[1][0, h]).T), 0.0).max(1)
        bound = gamma * a + 8 * u * np.abs(L[0, h])
        err = np.abs(lg[0, h] - L[0, h])
        assert (err <= bound).all(), f"LSE head {h}: error {err.max():.3e} vs bound {bound.min():.3e}"
        compare(f"LSE[{h}]", lg[0, h], L[0, h], float(bound.max()))
    compare("dQ", dq, gQ, 2.0 ** -6 * np.abs(gQ).max(), REL_RMS["bf16"])
    compare("dK", dk, gK, 2.0 ** -6 * np.abs(gK).max(), REL_RMS["bf16"])
    compare("dV", dv, gV, tol["grad"], REL_RMS["bf16"])


def test_stream_and_repeatability():
    """Calls run on torch's current stream; two runs give identical bits
    (no atomics anywhere in the path)."""
    (q, k, v, do), _ = make(2, 3, 333, 128, "bf16", seed=5)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        o1, l1 = flash.fwd(q, k, v, causal=True)
        g1 = flash.bwd(q, k, v, o1, do, l1, causal=True)
    st.synchronize()
    o2, l2 = flash.fwd(q, k, v, causal=True)
    g2 = flash.bwd(q, k, v, o2, do, l2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_running_max_refresh_mid_sweep(dtype, d, causal):
    """Key rows scaled up along the sequence make every row's maximum rise
    well past the lazy-refresh margin several times during the sweep, so
    the accumulator rescale runs on tiles after the first, in both halves of
    the unrolled loop and in masked and unmasked iterations."""
    B, H, N = 1, 2, 1100
    q, k, v, do = workloads.qkvdo(B, H, N, d, dtype, seed=31)
    ramp = torch.linspace(0.25, 12.0, N).view(1, 1, N, 1)
    k = (k.float() * ramp).to(k.dtype)
    cpu = (q, k, v, do)
    gq, gk, gv, gdo = (t.cuda() for t in cpu)
    f64 = tuple(t.to(torch.float64).numpy() for t in cpu)
    s = fp32_scale(d)
    o, lse = flash.fwd(gq, gk, gv, scale=s, causal=causal)
    dq, dk, dv = flash.bwd(gq, gk, gv, o, gdo, lse, scale=s, causal=causal)
    torch.cuda.synchronize()
    O, L = _oracle_fwd(f64, s, causal)
    tol = TOL[dtype]
    compare("O", o, O, tol["o"], REL_RMS[dtype])
    compare_lse("LSE", lse, L, tol["lse"])
    gQ, gK, gV = _oracle_bwd(f64, s, causal)
    # dK and dQ scale with the key magnitudes (up to 12x here)
    compare("dQ", dq, gQ, 12 * tol["grad"], REL_RMS[dtype])
    compare("dK", dk, gK, 12 * tol["grad"], REL_RMS[dtype])
    compare("dV", dv, gV, tol["grad"], REL_RMS[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape,splits", [((1, 2, 200), 2), ((2, 1, 519), 3), ((1, 1, 1), 4),
                                          ((1, 3, 1100), 8), ((1, 1, 64), 64), ((1, 2, 700), 1)],
                         ids=lambda x: "x".join(map(str, x)) if isinstance(x, tuple) else str(x))
def test_splitkv_forward(dtype, d, causal, shape, splits):
    """Split-KV forward (key ranges per workgroup + merge) against the plain
    definition; splits beyond the number of key tiles leave empty ranges."""
    B, H, N = shape
    (q, k, v, _), f64 = make(B, H, N, d, dtype, seed=300 + N + d + splits)
    s = fp32_scale(d)
    o, lse = flash.fwd_splitkv(q, k, v, splits, scale=s, causal=causal)
    torch.cuda.synchronize()
    O, L = _oracle_fwd(f64, s, causal)
    tol = TOL[dtype]
    compare("O", o, O, tol["o"], REL_RMS[dtype])
    compare_lse("LSE", lse, L, tol["lse"])


def _oracle_gqa(f64, s, causal):
    q, k, v, do = f64
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    fw = A.forward_gqa(q, k, v, s, causal)
    dQ, dK, dV = A.backward_gqa(q, k, v, do, s, causal)
    O = np.stack([np.stack([fw[(b, h)][0] for h in range(H)]) for b in range(B)])
    L = np.stack([np.stack([fw[(b, h)][1] for h in range(H)]) for b in range(B)])
    gQ = np.stack([np.stack([dQ[(b, h)] for h in range(H)]) for b in range(B)])
    gK = np.stack([np.stack([dK[(b, g)] for g in range(Hkv)]) for b in range(B)])
    gV = np.stack([np.stack([dV[(b, g)] for g in range(Hkv)]) for b in range(B)])
    return O, L, gQ, gK, gV


# The dK/dV pass cuts a group of G = H/Hkv query heads into s = min(G,
# ceil(1024 / units)) ranges, units = B*Hkv*ceil(N/128): the small shapes run
# one head per range (float32 partials + range sum); (8, 256, 32, 128) runs
# ranges of two heads; (8, 128, 64, 200) one range per group (no partials).
GQA_SHAPES = [(1, 4, 1, 200), (2, 6, 2, 333), (1, 4, 4, 130), (1, 3, 1, 1), (2, 4, 2, 519),
              (1, 16, 1, 300)]
GQA_SHAPES_MANY_HEADS = [(8, 256, 32, 128), (8, 128, 64, 200)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", GQA_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gqa_forward_backward(dtype, d, causal, shape):
    _check_gqa(dtype, d, causal, shape)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", GQA_SHAPES_MANY_HEADS, ids=lambda s: "x".join(map(str, s)))
def test_gqa_forward_backward_many_heads(d, causal, shape):
    _check_gqa("bf16", d, causal, shape)


def _check_gqa(dtype, d, causal, shape):
    """Grouped K/V heads: each query head reads its group's K/V head in place;
    dK and dV of a K/V head sum over the group.  A sum of G per-head
    gradients with independent roundings has ~sqrt(G) times the error of one,
    so the absolute gradient bound scales by sqrt(G)."""
    B, H, Hkv, N = shape
    G = H // Hkv
    cpu = workloads.qkvdo_grouped(B, H, Hkv, N, d, dtype, seed=500 + N + d + H + Hkv)
    q, k, v, do = (t.cuda() for t in cpu)
    f64 = tuple(t.to(torch.float64).numpy() for t in cpu)
    s = fp32_scale(d)
    o, lse = flash.fwd_gqa(q, k, v, scale=s, causal=causal)
    dq, dk, dv = flash.bwd_gqa(q, k, v, o, do, lse, scale=s, causal=causal)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape and dq.shape == q.shape
    O, L, gQ, gK, gV = _oracle_gqa(f64, s, causal)
    tol = TOL[dtype]
    compare("O", o, O, tol["o"], REL_RMS[dtype])
    compare_lse("LSE", lse, L, tol["lse"])
    compare("dQ", dq, gQ, tol["grad"], REL_RMS[dtype])
    compare("dK", dk, gK, tol["grad"] * max(1.0, G ** 0.5), REL_RMS[dtype])
    compare("dV", dv, gV, tol["grad"] * max(1.0, G ** 0.5), REL_RMS[dtype])


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_float32_forward(causal):
    B, H, Hkv, N, d = 2, 6, 3, 150, 64
    cpu = workloads.qkvdo_grouped(B, H, Hkv, N, d, "f32", seed=77)
    q, k, v, _ = (t.cuda() for t in cpu)
    f64 = tuple(t.to(torch.float64).numpy() for t in cpu)
    s = fp32_scale(d)
    o, lse = flash.fwd_gqa(q, k, v, scale=s, causal=causal)
    torch.cuda.synchronize()
    O, L, *_ = _oracle_gqa(f64, s, causal)
    compare("O", o, O, TOL["f32"]["o"], REL_RMS["f32"])
    compare_lse("LSE", lse, L, TOL["f32"]["lse"])


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_matches_broadcast_heads_bitwise(causal):
    """Reading the group's K/V head in place gives the same bits as the plain
    calls on K/V copied out to every query head (forward and dQ), and one
    K/V head per query head is the plain call."""
    B, H, Hkv, N, d = 2, 8, 2, 700, 128
    q, k, v, do = (t.cuda() for t in workloads.qkvdo_grouped(B, H, Hkv, N, d, "bf16", seed=91))
    krep = k.repeat_interleave(H // Hkv, dim=1).contiguous()
    vrep = v.repeat_interleave(H // Hkv, dim=1).contiguous()
    o, lse = flash.fwd_gqa(q, k, v, causal=causal)
    dq, dk, dv = flash.bwd_gqa(q, k, v, o, do, lse, causal=causal)
    o2, lse2 = flash.fwd(q, krep, vrep, causal=causal)
    dq2, _, _ = flash.bwd(q, krep, vrep, o2, do, lse2, causal=causal)
    o3, lse3 = flash.fwd_gqa(q, krep, vrep, causal=causal)
    dq3, dk3, dv3 = flash.bwd_gqa(q, krep, vrep, o3, do, lse3, causal=causal)
    dq4, dk4, dv4 = flash.bwd(q, krep, vrep, o3, do, lse3, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and torch.equal(dq, dq2)
    assert torch.equal(o3, o2) and torch.equal(dq3, dq4) and torch.equal(dk3, dk4) and torch.equal(dv3, dv4)


def test_gqa_empty_inputs():
    for B, H, Hkv, N in ((0, 4, 2, 64), (1, 0, 0, 64), (1, 4, 1, 0)):
        q = torch.zeros((B, H, N, 64), dtype=torch.bfloat16, device="cuda")
        k = torch.zeros((B, Hkv, N, 64), dtype=torch.bfloat16, device="cuda")
        o, lse = flash.fwd_gqa(q, k, k)
        dq, dk, dv = flash.bwd_gqa(q, k, k, o, q, lse)
        torch.cuda.synchronize()
        assert o.shape == q.shape and dk.shape == k.shape


VARLEN_CASES = [
    # (lengths, H, Hkv)
    ([200, 1, 333, 0, 64, 519], 4, 2),
    ([300, 300], 2, 2),
    ([17], 3, 1),
    ([1000, 129, 256, 7], 2, 1),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(VARLEN_CASES)))
def test_varlen_forward_backward(dtype, d, causal, case):
    """Packed variable-length batch (token-major [total, heads, d]) against the
    oracle run on each sequence alone; empty and one-token sequences
    included.  dK, dV of a shared head use the grouped-head bound."""
    lens, H, Hkv = VARLEN_CASES[case]
    G = H // Hkv
    q, k, v, do, cu = workloads.packed_qkvdo(lens, H, Hkv, d, dtype, seed=600 + case + d)
    f64 = [t.to(torch.float64).numpy() for t in (q, k, v, do)]
    gq, gk, gv, gdo, gcu = (t.cuda() for t in (q, k, v, do, cu))
    s = fp32_scale(d)
    o, lse = flash.varlen_fwd(gq, gk, gv, gcu, max(lens), scale=s, causal=causal)
    dq, dk, dv = flash.varlen_bwd(gq, gk, gv, o, gdo, lse, gcu, max(lens), scale=s, causal=causal)
    torch.cuda.synchronize()
    O, L = A.forward_varlen(*f64[:3], cu.numpy(), s, causal)
    gQ, gK, gV = A.backward_varlen(*f64, cu.numpy(), s, causal)
    tol = TOL[dtype]
    compare("O", o, O, tol["o"], REL_RMS[dtype])
    compare_lse("LSE", lse, L, tol["lse"])
    compare("dQ", dq, gQ, tol["grad"], REL_RMS[dtype])
    compare("dK", dk, gK, tol["grad"] * max(1.0, G ** 0.5), REL_RMS[dtype])
    compare("dV", dv, gV, tol["grad"] * max(1.0, G ** 0.5), REL_RMS[dtype])


def test_varlen_float32_forward():
    lens, H, Hkv, d = [100, 37, 256], 2, 1, 64
    q, k, v, _, cu = workloads.packed_qkvdo(lens, H, Hkv, d, "f32", seed=71)
    f64 = [t.to(torch.float64).numpy() for t in (q, k, v)]
    s = fp32_scale(d)
    o, lse = flash.varlen_fwd(q.cuda(), k.cuda(), v.cuda(), cu.cuda(), max(lens), scale=s, causal=True)
    torch.cuda.synchronize()
    O, L = A.forward_varlen(*f64, cu.numpy(), s, True)
    compare("O", o, O, TOL["f32"]["o"], REL_RMS["f32"])
    compare_lse("LSE", lse, L, TOL["f32"]["lse"])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hkv", [4, 2])
def test_bnhd_layout_matches_dense_bitwise(causal, Hkv):
    """A [B, N, H, d] batch passed as a packed batch of equal lengths runs the
    same arithmetic as the dense [B, H, N, d] calls: identical bits."""
    B, H, N, d = 3, 4, 700, 128
    q, k, v, do = (t.cuda() for t in workloads.qkvdo_grouped(B, H, Hkv, N, d, "bf16", seed=93))
    o, lse = flash.fwd_gqa(q, k, v, causal=causal)
    dq, dk, dv = flash.bwd_gqa(q, k, v, o, do, lse, causal=causal)
    tok = lambda t: t.transpose(1, 2).contiguous().view(B * N, t.shape[1], d)  # [B,H,N,d] -> [B*N, H, d]
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    o2, lse2 = flash.varlen_fwd(tok(q), tok(k), tok(v), cu, N, causal=causal)
    dq2, dk2, dv2 = flash.varlen_bwd(tok(q), tok(k), tok(v), o2, tok(do), lse2, cu, N, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o2, tok(o))
    assert torch.equal(lse2, lse.permute(1, 0, 2).reshape(H, B * N))
    for a, b in ((dq2, dq), (dk2, dk), (dv2, dv)):
        assert torch.equal(a, tok(b))


def test_varlen_empty_batches():
    for lens in ([], [0, 0]):
        q = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device="cuda")
        cu = torch.zeros(len(lens) + 1, dtype=torch.int32, device="cuda")
        o, lse = flash.varlen_fwd(q, q, q, cu, max(lens, default=0))
        dq, dk, dv = flash.varlen_bwd(q, q, q, o, q, lse, cu, max(lens, default=0))
        torch.cuda.synchronize()
        assert o.shape == q.shape and lse.shape == (2, 0)


# ---------------------------------------------------------------- dropout
from oracle import philox as PX  # noqa: E402


def _oracle_dropout(f64, s, causal, p, seed, offset):
    q, k, v, do = f64
    B, H, N, _ = q.shape
    t = PX.drop_threshold(p)
    pd = t / 256.0
    O = np.zeros(q.shape)
    L = np.zeros(q.shape[:3])
    G = [np.zeros(q.shape) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            keep = PX.keep_matrix(N, N, b * H + h, seed, offset, t)
            O[b, h], L[b, h] = A.forward_head_dropout(q[b, h], k[b, h], v[b, h], s, causal, keep, pd)
            g = A.backward_head_dropout(q[b, h], k[b, h], v[b, h], do[b, h], s, causal, keep, pd)
            for i in range(3):
                G[i][b, h] = g[i]
    return O, L, G


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape,p", [((1, 2, 200), 0.1), ((2, 1, 519), 0.5), ((1, 3, 64), 0.2),
                                     ((1, 1, 1), 0.3), ((1, 2, 300), 0.0)],
                         ids=lambda x: "x".join(map(str, x)) if isinstance(x, tuple) else str(x))
def test_dropout_forward_backward(dtype, d, causal, shape, p):
    """Dropout decisions drawn inside the kernels from Philox4x32-10 equal
    the oracle's draws (any mismatch moves O by O(1)); the gradient is the
    exact gradient through the same decisions.  Kept probabilities carry a
    factor 1/(1-p) <= 2, so O and the gradients get twice the plain bounds."""
    B, H, N = shape
    seed, offset = 0x1234_5678_9ABC + N, 17 + d
    (q, k, v, do), f64 = make(B, H, N, d, dtype, seed=700 + N + d)
    s = fp32_scale(d)
    o, lse = flash.fwd_dropout(q, k, v, p, seed, offset, scale=s, causal=causal)
    dq, dk, dv = flash.bwd_dropout(q, k, v, o, do, lse, p, seed, offset, scale=s, causal=causal)
    torch.cuda.synchronize()
    O, L, (gQ, gK, gV) = _oracle_dropout(f64, s, causal, p, seed, offset)
    tol = TOL[dtype]
    compare("O", o, O, 2 * tol["o"], REL_RMS[dtype])
    compare_lse("LSE", lse, L, tol["lse"])
    # With one key the exact dQ and dK are zero (a one-element softmax has no
    # gradient); the kernels' D = rowsum(dO o O) reads the stored, rounded O,
    # which no longer equals dP exactly once O carries the 1/(1-p) factor, so
    # only the absolute bound is meaningful there.
    rg = REL_RMS[dtype] if N > 1 else None
    compare("dQ", dq, gQ, 2 * tol["grad"], rg)
    compare("dK", dk, gK, 2 * tol["grad"], rg)
    compare("dV", dv, gV, 2 * tol["grad"], REL_RMS[dtype])


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_decisions_read_off_the_output(causal):
    """With V = the identity (N = d = 64), row i of O is row i of
    P o Z / (1 - p): its zero pattern is the dropout decisions, compared
    entry by entry with the oracle's (every allowed P is > 0)."""
    N, d, p, seed, offset = 64, 64, 0.3, 987654321, 5
    q, k, _, _ = workloads.qkvdo(2, 3, N, d, "bf16", seed=42)
    v = torch.eye(N, dtype=torch.bfloat16).expand(2, 3, N, d).contiguous()
    o, _ = flash.fwd_dropout(q.cuda(), k.cuda(), v.cuda(), p, seed, offset, causal=causal)
    torch.cuda.synchronize()
    t = PX.drop_threshold(p)
    allowed = A.allowed(N, N, causal)
    for b in range(2):
        for h in range(3):
            keep = PX.keep_matrix(N, N, b * 3 + h, seed, offset, t)
            nz = to64(o[b, h]) != 0
            assert (nz == (keep & allowed)).all(), (b, h, int((nz != (keep & allowed)).sum()))


def test_dropout_zero_rate_matches_plain_calls():
    """p = 0 keeps every element with factor 1.  The dropout forward (the
    one-wave kernel) and the plain forward (the two-wave kernel, other tile
    sizes and so another summation order) both meet the oracle's bounds.
    Given the same O and LSE, the dK/dV pass with and without the dropout
    code is bit-identical; dQ (a separate, simpler pass) within the gradient
    bound."""
    (q, k, v, do), f64 = make(2, 2, 400, 128, "bf16", seed=3)
    s = 128 ** -0.5
    o, lse = flash.fwd(q, k, v, scale=s, causal=True)
    o2, lse2 = flash.fwd_dropout(q, k, v, 0.0, 11, 0, scale=s, causal=True)
    dq, dk, dv = flash.bwd(q, k, v, o, do, lse, scale=s, causal=True)
    dq2, dk2, dv2 = flash.bwd_dropout(q, k, v, o, do, lse, 0.0, 11, 0, scale=s, causal=True)
    torch.cuda.synchronize()
    O, L = _oracle_fwd(f64, s, True)
    for name, got, ref, tol in (("O plain", o, O, "o"), ("O dropout p=0", o2, O, "o")):
        compare(name, got, ref, TOL["bf16"][tol], REL_RMS["bf16"])
    compare_lse("LSE plain", lse, L, TOL["bf16"]["lse"])
    compare_lse("LSE dropout p=0", lse2, L, TOL["bf16"]["lse"])
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)
    compare("dQ", dq2, to64(dq), TOL["bf16"]["grad"])


def test_dropout_seed_and_offset_select_the_stream():
    (q, k, v, _), _ = make(1, 2, 256, 64, "f16", seed=8)
    a = flash.fwd_dropout(q, k, v, 0.5, 1, 0)[0]
    b = flash.fwd_dropout(q, k, v, 0.5, 1, 0)[0]
    c = flash.fwd_dropout(q, k, v, 0.5, 2, 0)[0]
    e = flash.fwd_dropout(q, k, v, 0.5, 1, 1)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b) and not torch.equal(a, c) and not torch.equal(a, e)


@pytest.mark.parametrize("d", [64, 128])
def test_very_long_sequence_sampled_rows(d):
    """One head of 2^17 + 37 tokens (ragged tail, row offsets past 2^24
    elements): O, LSE and dQ of sampled rows against the oracle row by row
    (each depends only on its own scores), dK/dV against the softmax
    Jacobian's column identities (sum_j dK_j = 0, sum_j dV_j = sum_i dO_i)."""
    N = (1 << 17) + 37
    (q, k, v, do), _ = make(1, 1, N, d, "bf16", seed=123 + d, gain=0.5)
    s = fp32_scale(d)
    o, lse = flash.fwd(q, k, v, scale=s, causal=True)
    dq, dk, dv = flash.bwd(q, k, v, o, do, lse, scale=s, causal=True)
    torch.cuda.synchronize()
    for t in (o, dq, dk, dv):
        assert torch.isfinite(t).all()
    qc, kc, vc, doc = (t[0, 0].to(torch.float64).cpu().numpy() for t in (q, k, v, do))
    rows = np.array([0, 1, 31, 32, 4095, 65536, N - 38, N - 2, N - 1])
    O, L = A.forward_head(qc, kc, vc, s, True, rows=rows)
    tol = TOL["bf16"]
    compare("O rows", to64(o[0, 0])[rows], O, tol["o"])
    compare_lse("LSE rows", to64(lse[0, 0])[rows], L, tol["lse"])
    gq = A.grad_q_rows(qc, kc, vc, doc, s, True, rows=rows)
    compare("dQ rows", to64(dq[0, 0])[rows], gq, tol["grad"])
    sum_dk = dk[0, 0].double().sum(0).cpu().numpy()
    sum_dv = dv[0, 0].double().sum(0).cpu().numpy()
    sum_do = do[0, 0].double().sum(0).cpu().numpy()
    rms_k = float(dk.double().pow(2).mean().sqrt())
    rms_v = float(dv.double().pow(2).mean().sqrt())
    # each column sum adds N values rounded to bf16 (relative 2^-9): the
    # residual grows like sqrt(N) times their size
    assert np.abs(sum_dk).max() <= 4 * np.sqrt(N) * rms_k * 2.0 ** -8
    assert np.abs(sum_dv - sum_do).max() <= 4 * np.sqrt(N) * rms_v * 2.0 ** -8 + 1e-3 * np.abs(sum_do).max()


def _random_case(i):
    g = np.random.default_rng(1000 + i)
    H = int(g.choice([1, 2, 3, 4, 6]))
    Hkv = int(g.choice([h for h in range(1, H + 1) if H % h == 0]))
    return dict(B=int(g.integers(1, 4)), H=H, Hkv=Hkv, N=int(g.integers(1, 700)), d=int(g.choice([64, 128])),
                dtype=str(g.choice(["bf16", "f16"])), causal=bool(g.integers(0, 2)),
                api=str(g.choice(["dense", "gqa", "varlen", "splitkv", "dropout"])), seed=2000 + i)


@pytest.mark.parametrize("i", range(30))
def test_random_shapes_sweep(i):
    """Seeded random shapes through every entry point family, against the
    oracle (grouped-head gradient bound as in the grouped-head test)."""
    c = _random_case(i)
    B, H, Hkv, N, d, dt, causal = c["B"], c["H"], c["Hkv"], c["N"], c["d"], c["dtype"], c["causal"]
    s = fp32_scale(d)
    tol = TOL[dt]
    G = max(1.0, (H // Hkv) ** 0.5)
    if c["api"] == "varlen":
        g = np.random.default_rng(c["seed"])
        lens = [int(x) for x in g.integers(0, N + 1, B)]
        lens[0] = N
        q, k, v, do, cu = workloads.packed_qkvdo(lens, H, Hkv, d, dt, seed=c["seed"])
        f64 = [t.to(torch.float64).numpy() for t in (q, k, v, do)]
        gq, gk, gv, gdo, gcu = (t.cuda() for t in (q, k, v, do, cu))
        o, lse = flash.varlen_fwd(gq, gk, gv, gcu, N, scale=s, causal=causal)
        dq, dk, dv = flash.varlen_bwd(gq, gk, gv, o, gdo, lse, gcu, N, scale=s, causal=causal)
        torch.cuda.synchronize()
        O, L = A.forward_varlen(*f64[:3], cu.numpy(), s, causal)
        gQ, gK, gV = A.backward_varlen(*f64, cu.numpy(), s, causal)
    elif c["api"] == "gqa":
        cpu = workloads.qkvdo_grouped(B, H, Hkv, N, d, dt, seed=c["seed"])
        q, k, v, do = (t.cuda() for t in cpu)
        f64 = tuple(t.to(torch.float64).numpy() for t in cpu)
        o, lse = flash.fwd_gqa(q, k, v, scale=s, causal=causal)
        dq, dk, dv = flash.bwd_gqa(q, k, v, o, do, lse, scale=s, causal=causal)
        torch.cuda.synchronize()
        O, L, gQ, gK, gV = _oracle_gqa(f64, s, causal)
    else:
        (q, k, v, do), f64 = make(B, H, N, d, dt, seed=c["seed"])
        if c["api"] == "splitkv":
            o, lse = flash.fwd_splitkv(q, k, v, 1 + c["seed"] % 7, scale=s, causal=causal)
            torch.cuda.synchronize()
            O, L = _oracle_fwd(f64, s, causal)
            compare("O", o, O, tol["o"], REL_RMS[dt])
            compare_lse("LSE", lse, L, tol["lse"])
            return
        if c["api"] == "dropout":
            p, seed = 0.25, c["seed"]
            o, lse = flash.fwd_dropout(q, k, v, p, seed, 3, scale=s, causal=causal)
            dq, dk, dv = flash.bwd_dropout(q, k, v, o, do, lse, p, seed, 3, scale=s, causal=causal)
            torch.cuda.synchronize()
            O, L, (gQ, gK, gV) = _oracle_dropout(f64, s, causal, p, seed, 3)
            G = 2.0  # the 1/(1-p) factor
            tol = dict(o=2 * tol["o"], lse=tol["lse"], grad=tol["grad"])
        else:
            o, lse = flash.fwd(q, k, v, scale=s, causal=causal)
            dq, dk, dv = flash.bwd(q, k, v, o, do, lse, scale=s, causal=causal)
            torch.cuda.synchronize()
            O, L = _oracle_fwd(f64, s, causal)
            gQ, gK, gV = _oracle_bwd(f64, s, causal)
    rg = REL_RMS[dt] if N > 1 else None
    compare("O", o, O, tol["o"], REL_RMS[dt])
    compare_lse("LSE", lse, L, tol["lse"])
    compare("dQ", dq, gQ, tol["grad"] * (2.0 if c["api"] == "dropout" else 1.0), rg)
    compare("dK", dk, gK, tol["grad"] * G, rg)
    compare("dV", dv, gV, tol["grad"] * G, REL_RMS[dt])


def test_splitkv_default_split_count():
    """num_splits left to the library (its shape heuristic) gives the plain
    forward's result."""
    (q, k, v, _), f64 = make(1, 2, 3000, 128, "bf16", seed=808)
    s = fp32_scale(128)
    o, lse = flash.fwd_splitkv(q, k, v, scale=s, causal=True)
    torch.cuda.synchronize()
    assert flash.fwd_splitkv_num_splits(1, 2, 3000, 128, True) > 1
    O, L = _oracle_fwd(f64, s, True)
    compare("O", o, O, TOL["bf16"]["o"], REL_RMS["bf16"])
    compare_lse("LSE", lse, L, TOL["bf16"]["lse"])


def _oracle_varlen_dropout(f64, cu, s, causal, p, seed, offset):
    q, k, v, do = f64
    T, H, _ = q.shape
    Hkv = k.shape[1]
    t = PX.drop_threshold(p)
    pd = t / 256.0
    O, L = np.zeros(q.shape), np.full((H, T), -np.inf)
    gQ, gK, gV = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(len(cu) - 1):
        a, e = int(cu[b]), int(cu[b + 1])
        if e <= a:
            continue
        for h in range(H):
            g = A.kv_head_of(h, H, Hkv)
            keep = PX.keep_matrix(e - a, e - a, b * H + h, seed, offset, t)
            O[a:e, h], L[h, a:e] = A.forward_head_dropout(q[a:e, h], k[a:e, g], v[a:e, g], s, causal, keep, pd)
            dq_, dk_, dv_ = A.backward_head_dropout(q[a:e, h], k[a:e, g], v[a:e, g], do[a:e, h], s, causal, keep, pd)
            gQ[a:e, h] = dq_
            gK[a:e, g] += dk_
            gV[a:e, g] += dv_
    return O, L, gQ, gK, gV


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", [([300, 0, 129, 1], 4, 2), ([500, 77], 3, 1)])
def test_varlen_dropout(d, causal, case):
    """Dropout on a packed batch with grouped heads: positions in the
    counter count from each sequence's start, the head index is b*H + h."""
    lens, H, Hkv = case
    p, seed, offset = 0.2, 4242 + d, 9
    q, k, v, do, cu = workloads.packed_qkvdo(lens, H, Hkv, d, "bf16", seed=900 + d + H)
    f64 = [t.to(torch.float64).numpy() for t in (q, k, v, do)]
    gq, gk, gv, gdo, gcu = (t.cuda() for t in (q, k, v, do, cu))
    s = fp32_scale(d)
    o, lse = flash.varlen_fwd_dropout(gq, gk, gv, gcu, max(lens), p, seed, offset, scale=s, causal=causal)
    dq, dk, dv = flash.varlen_bwd_dropout(gq, gk, gv, o, gdo, lse, gcu, max(lens), p, seed, offset, scale=s,
                                          causal=causal)
    torch.cuda.synchronize()
    O, L, gQ, gK, gV = _oracle_varlen_dropout(f64, cu.numpy(), s, causal, p, seed, offset)
    tol = TOL["bf16"]
    G = 2.0 * (H // Hkv) ** 0.5
    compare("O", o, O, 2 * tol["o"], REL_RMS["bf16"])
    compare_lse("LSE", lse, L, tol["lse"])
    compare("dQ", dq, gQ, 2 * tol["grad"], REL_RMS["bf16"])
    compare("dK", dk, gK, G * tol["grad"], REL_RMS["bf16"])
    compare("dV", dv, gV, G * tol["grad"], REL_RMS["bf16"])


def _identity_rows(B, H, N, d, dtype):
    """[B, H, N, d] whose row i is the unit vector e_i (N <= d)."""
    x = torch.zeros((B, H, N, d), dtype=DT[dtype])
    x[:, :, torch.arange(N), torch.arange(N)] = 1
    return x


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,N", [(64, 61), (128, 125), (64, 7)])
def test_dropout_decisions_of_the_dkdv_pass(causal, d, N):
    """Keep decisions drawn by the dK/dV pass, element by element.  With
    dO = [I | 0] (row i of dO is e_i), dV = (P o Z)^T dO / (1 - p') has
    dV[j, i] = P_ij Z_ij / (1 - p') for i < N: its zero pattern is
    (Z and allowed)^T exactly (every allowed P_ij > 0).  N is ragged against
    the 4 x 4 decision blocks and the 32-row tiles; several heads check the
    head index of the counter."""
    B, H, p, seed, offset = 2, 3, 0.3, 0x0BAD_5EED_1234 + N, 11 + d
    q, k, v, _ = workloads.qkvdo(B, H, N, d, "bf16", seed=17 + N)
    do = _identity_rows(B, H, N, d, "bf16")
    gq, gk, gv, gdo = (t.cuda() for t in (q, k, v, do))
    o, lse = flash.fwd_dropout(gq, gk, gv, p, seed, offset, causal=causal)
    _, _, dv = flash.bwd_dropout(gq, gk, gv, o, gdo, lse, p, seed, offset, causal=causal)
    torch.cuda.synchronize()
    t = PX.drop_threshold(p)
    allowed = A.allowed(N, N, causal)
    dvc = to64(dv)
    assert (dvc[..., N:] == 0).all()
    for b in range(B):
        for h in range(H):
            keep = PX.keep_matrix(N, N, b * H + h, seed, offset, t)
            got = dvc[b, h, :, :N] != 0            # [key j, query i]
            want = (keep & allowed).T
            assert (got == want).all(), (b, h, int((got != want).sum()))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,N", [(64, 61), (128, 125), (64, 7)])
def test_dropout_decisions_of_the_dq_pass(causal, d, N):
    """Keep decisions drawn by the dQ pass, element by element.  With Q = 0
    every allowed probability is 1/n_i (n_i allowed keys of row i); with
    K = V = [I | 0] and dO = 1, dP'_ij = 1, O_ic = Z_ic / (n_i (1 - p')) and
    D_i = sum_c O_ic, so dQ[i, j] = scale dS_ij = scale (Z_ij / (1 - p') - D_i) / n_i
    for j < N.  Solving for Z_ij (threshold 1/2, far from the rounding
    error) gives the decisions, which must equal the oracle's draws."""
    B, H, p, seed, offset = 2, 3, 0.3, 0x51DE_CAFE + N, 5 + d
    q = torch.zeros((B, H, N, d), dtype=torch.bfloat16)
    k = _identity_rows(B, H, N, d, "bf16")
    v = k.clone()
    do = torch.ones((B, H, N, d), dtype=torch.bfloat16)
    s = 0.5
    gq, gk, gv, gdo = (t.cuda() for t in (q, k, v, do))
    o, lse = flash.fwd_dropout(gq, gk, gv, p, seed, offset, scale=s, causal=causal)
    dq, _, _ = flash.bwd_dropout(gq, gk, gv, o, gdo, lse, p, seed, offset, scale=s, causal=causal)
    torch.cuda.synchronize()
    t = PX.drop_threshold(p)
    pd = t / 256.0
    allowed = A.allowed(N, N, causal)
    n_i = allowed.sum(1).astype(np.float64)
    oc, dqc = to64(o), to64(dq)
    for b in range(B):
        for h in range(H):
            keep = PX.keep_matrix(N, N, b * H + h, seed, offset, t)
            D = oc[b, h].sum(1)                      # rowsum(dO o O) with dO = 1
            z = (dqc[b, h, :, :N] * n_i[:, None] / s + D[:, None]) * (1.0 - pd)
            got = z > 0.5
            assert (got[allowed] == keep[allowed]).all(), (b, h, int((got[allowed] != keep[allowed]).sum()))
            assert (dqc[b, h, :, :N][~allowed] == 0).all()
