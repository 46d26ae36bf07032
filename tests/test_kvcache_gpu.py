"""GPU parity of flash_attn_fwd_kvcache (a few queries per head against a
key/value cache) with the float64 oracle's forward_kvcache.

Shapes cover decoding (Nq = 1) with grouped and multi-query heads, several
new queries per step (the causal rule counting them as the last positions
of the sequence), groups of more than 32 and 64 rows (several row tiles),
per-sequence cache lengths (empty, shorter than Nq, ragged against the
32-key tiles), explicit and library-chosen key splits, and cache slots past
each sequence's length filled with NaN (never read, so never in a result).
"""
import numpy as np
import pytest
import torch

from io_aware_exact_flash_amd import flash, workloads
from oracle import attention as A
from tests._parity import REL_RMS, TOL, compare, compare_lse, fp32_scale

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, Hkv, Nq, Nk, lens or None, splits or None)
    (2, 8, 2, 1, 1000, None, None),
    (2, 8, 2, 1, 1000, None, 1),
    (1, 4, 4, 5, 517, None, 3),
    (3, 6, 1, 3, 300, [300, 2, 0], None),
    (1, 16, 2, 12, 700, None, 5),
    (1, 16, 2, 12, 700, None, 1),
    (2, 4, 2, 129, 129, None, 2),
    (1, 2, 1, 1, 1, None, None),
    (2, 32, 8, 1, 3000, [3000, 1777], 64),
]


def _inputs(B, H, Hkv, Nq, Nk, d, dtype, seed):
    return workloads.kvcache_qkv(B, H, Hkv, Nq, Nk, d, dtype, seed=seed)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_kvcache_forward(dtype, d, causal, case):
    B, H, Hkv, Nq, Nk, lens, splits = CASES[case]
    q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, dtype, seed=1200 + case + d)
    lens_t = None if lens is None else torch.tensor(lens, dtype=torch.int32)
    if lens is not None:
        # slots past each sequence's length hold NaN: they must never be read
        for b, L in enumerate(lens):
            k[b, :, L:] = float("nan")
            v[b, :, L:] = float("nan")
    s = fp32_scale(d)
    o, lse = flash.fwd_kvcache(q.cuda(), k.cuda(), v.cuda(), None if lens_t is None else lens_t.cuda(),
                               num_splits=splits, scale=s, causal=causal)
    torch.cuda.synchronize()
    f64 = [t.to(torch.float64).numpy() for t in (q, k, v)]
    ref = A.forward_kvcache(*f64, s, causal, lens)
    O = np.stack([np.stack([ref[(b, h)][0] for h in range(H)]) for b in range(B)])
    L_ = np.stack([np.stack([ref[(b, h)][1] for h in range(H)]) for b in range(B)])
    tol = TOL[dtype]
    compare("O", o, O, tol["o"], REL_RMS[dtype])
    compare_lse("LSE", lse, L_, tol["lse"])


def test_kvcache_equal_lengths_match_the_grouped_forward():
    """With Nq = Nk the call is causal self-attention: it agrees with
    flash_attn_fwd_gqa (a different kernel) within the stated bound."""
    B, H, Hkv, N, d = 2, 8, 4, 333, 128
    q, k, v, _ = (t.cuda() for t in workloads.qkvdo_grouped(B, H, Hkv, N, d, "bf16", seed=1300))
    o1, l1 = flash.fwd_kvcache(q, k, v, causal=True)
    o2, l2 = flash.fwd_gqa(q, k, v, causal=True)
    torch.cuda.synchronize()
    compare("O", o1, o2.double().cpu().numpy(), TOL["bf16"]["o"])
    compare_lse("LSE", l1, l2.double().cpu().numpy(), TOL["bf16"]["lse"])


def test_kvcache_split_count_changes_only_rounding():
    """Every split count gives the oracle's result; the library's choice
    splits a long cache."""
    B, H, Hkv, Nq, Nk, d = 1, 8, 1, 1, 8192, 128
    assert flash.fwd_kvcache_num_splits(B, H, Hkv, Nq, Nk, d) > 1
    q, k, v = _inputs(B, H, Hkv, Nq, Nk, d, "bf16", seed=1400)
    f64 = [t.to(torch.float64).numpy() for t in (q, k, v)]
    ref = A.forward_kvcache(*f64, fp32_scale(d), True)
    O = np.stack([np.stack([ref[(0, h)][0] for h in range(H)])])
    for sp in (1, 2, 7, 64, None):
        o, _ = flash.fwd_kvcache(q.cuda(), k.cuda(), v.cuda(), num_splits=sp, causal=True)
        torch.cuda.synchronize()
        compare(f"O splits={sp}", o, O, TOL["bf16"]["o"], REL_RMS["bf16"])


def test_kvcache_empty_problems():
    q = torch.zeros((2, 4, 0, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((2, 2, 10, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = flash.fwd_kvcache(q, k, k)
    q1 = torch.ones((2, 4, 1, 64), dtype=torch.bfloat16, device="cuda")
    k0 = torch.zeros((2, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    o1, lse1 = flash.fwd_kvcache(q1, k0, k0)
    torch.cuda.synchronize()
    assert o.shape == q.shape and (o1 == 0).all() and torch.isneginf(lse1).all()
