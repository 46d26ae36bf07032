"""flash_attn_bwd_noalloc (the backward with its workspace held by the
library) against flash_attn_bwd, which takes a caller workspace: two calls
in a row, the second smaller, each identical to the allocating call's
result (same kernels, so the same bits), plus the oracle's gradient on the
second call."""
import pytest
import torch

from io_aware_exact_flash_amd import flash
from tests._parity import REL_RMS, TOL, compare, fp32_scale, make

pytestmark = pytest.mark.gpu


def _oracle_grads(f64, s, causal):
    from oracle import attention as A
    import numpy as np
    q, k, v, do = f64
    out = [np.zeros(q.shape) for _ in range(3)]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            g = A.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], s, causal)
            for i in range(3):
                out[i][b, h] = g[i]
    return out


def test_noalloc_backward_matches_workspace_backward_twice():
    cases = [((2, 4, 700, 128), "bf16", True), ((1, 2, 130, 64), "f16", False)]
    for (B, H, N, d), dtype, causal in cases:
        print(f"noalloc case B={B} H={H} N={N} d={d} {dtype} causal={causal}", flush=True)
        (q, k, v, do), f64 = make(B, H, N, d, dtype, seed=40 + N)
        s = fp32_scale(d)
        o, lse = flash.fwd(q, k, v, scale=s, causal=causal)
        ref = flash.bwd(q, k, v, o, do, lse, scale=s, causal=causal)
        got = flash.bwd_noalloc(q, k, v, o, do, lse, scale=s, causal=causal)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
    gQ, gK, gV = _oracle_grads(f64, s, causal)
    tol = TOL[dtype]
    for name, g, r in zip(("dQ", "dK", "dV"), got, (gQ, gK, gV)):
        compare(name, g, r, tol["grad"], REL_RMS[dtype])


def test_noalloc_rejects_problems_beyond_its_scratch():
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, 8), dtype=torch.float32, device="cuda")
    lib = flash.lib()
    # 2^23 query rows need 64 MiB of workspace, beyond the 32 MiB held
    st = lib.flash_attn_bwd_noalloc(1, 1, 1 << 23, 64, flash.FA_BF16, q.data_ptr(), q.data_ptr(), q.data_ptr(),
                                    q.data_ptr(), q.data_ptr(), lse.data_ptr(), 0.125, 0, q.data_ptr(),
                                    q.data_ptr(), q.data_ptr(), None)
    assert st == flash.FA_ERR_UNSUPPORTED
    assert b"workspace" in lib.flash_attn_last_error()
