"""Thin ctypes binding of libflashattn.so (argument marshalling only).

Every function here checks tensor metadata, allocates outputs with torch on
the inputs' device, and calls the C entry point of the same name on torch's
current HIP stream.  All arithmetic happens in the gfx950 kernels; there is
no fallback: if the library is missing or the tensors are not on a HIP
device the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FLASHATTN_LIB", os.path.join(_HERE, "libflashattn.so"))

FA_OK, FA_ERR_INVALID_ARGUMENT, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE_TOO_SMALL, FA_ERR_HIP = range(5)
FA_F32, FA_F16, FA_BF16 = 0, 1, 2
MASK_BLOCK = 128

_DT = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}

# exported symbol -> (restype, argtypes)
_I, _P, _F, _Z, _U8P = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = {
    "flash_attn_abi_version": (_I, []),
    "flash_attn_fwd": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _F, _I, _P, _P, _P]),
    "flash_attn_bwd_workspace_size": (_Z, [_I, _I, _I, _I, _I]),
    "flash_attn_bwd": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _F, _I, _P, _P, _P, _P, _Z, _P]),
    "flash_attn_blocksparse_fwd": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _F, _I, _U8P, _I, _P, _P, _P]),
    "flash_attn_blocksparse_bwd": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _F, _I, _U8P, _I,
                                        _P, _P, _P, _P, _Z, _P]),
    "flash_attn_fwd_splitkv_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I]),
    "flash_attn_fwd_splitkv_num_splits": (_I, [_I, _I, _I, _I, _I]),
    "flash_attn_fwd_splitkv": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _F, _I, _I, _P, _P, _P, _Z, _P]),
    "flash_attn_fwd_gqa": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _F, _I, _P, _P, _P]),
    "flash_attn_bwd_gqa_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I]),
    "flash_attn_bwd_gqa": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _F, _I, _P, _P, _P, _P, _Z,
                                _P]),
    "flash_attn_varlen_fwd": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _F, _I, _P, _P, _P]),
    "flash_attn_varlen_bwd_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "flash_attn_varlen_bwd": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _F, _I, _P, _P, _P,
                                   _P, _Z, _P]),
    "flash_attn_fwd_dropout": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _F, _I, _F, ctypes.c_uint64, ctypes.c_uint32,
                                    _P, _P, _P]),
    "flash_attn_bwd_dropout": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _F, _I, _F, ctypes.c_uint64,
                                    ctypes.c_uint32, _P, _P, _P, _P, _Z, _P]),
    "flash_attn_varlen_fwd_dropout": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _F, _I, _F, ctypes.c_uint64,
                                           ctypes.c_uint32, _P, _P, _P]),
    "flash_attn_varlen_bwd_dropout": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _F, _I, _F,
                                           ctypes.c_uint64, ctypes.c_uint32, _P, _P, _P, _P, _Z, _P]),
    "flash_attn_bwd_noalloc": (_I, [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _F, _I, _P, _P, _P, _P]),
    "flash_attn_fwd_kvcache_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "flash_attn_fwd_kvcache_num_splits": (_I, [_I, _I, _I, _I, _I, _I]),
    "flash_attn_fwd_kvcache": (_I, [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _F, _I, _I, _P, _P, _P, _Z, _P]),
    "flash_attn_status_string": (ctypes.c_char_p, [_I]),
    "flash_attn_last_error": (ctypes.c_char_p, []),
    "flash_attn_timing_enable": (_I, [_I]),
    "flash_attn_timing_collect": (_I, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int), _I]),
    "flash_attn_kernel_name": (ctypes.c_char_p, [_I]),
}
KERNELS = 13  # timing classes (names from flash_attn_kernel_name)

_lib = None
_lock = threading.Lock()


class FlashAttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library with argtypes set; raises if it was not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                                   "(python -c 'import __graft_entry__ as g; g.build()')")
            h = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                f = getattr(h, name)
                f.restype = res
                f.argtypes = args
            _lib = h
    return _lib


def status_string(status: int) -> str:
    return lib().flash_attn_status_string(status).decode()


def _check(status: int):
    if status != FA_OK:
        raise FlashAttnError(status, lib().flash_attn_last_error().decode())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _shape(q: torch.Tensor, *others: torch.Tensor):
    if q.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    if q.dtype not in _DT:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if not q.is_cuda:
        raise ValueError("tensors must live on a HIP device (no CPU path exists)")
    for t in (q,) + others:
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v (and o, dout) must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous [B, H, N, d]")
    B, H, N, d = q.shape
    return B, H, N, d, _DT[q.dtype]


def _shape_gqa(q, k, v, *per_query):
    """q (and o, dout) [B, H, N, d]; k, v [B, Hkv, N, d] with Hkv dividing H."""
    B, H, N, d, dt = _shape(q, *per_query)
    B2, Hkv, N2, d2, _ = _shape(k, v)
    if (B2, N2, d2) != (B, N, d) or k.dtype != q.dtype or k.device != q.device:
        raise ValueError("k, v must be [B, Hkv, N, d] with the batch, length, head size, dtype and device of q")
    return B, H, Hkv, N, d, dt


def _scale(scale, d):
    return float(1.0 / math.sqrt(d)) if scale is None else float(scale)


def _lse_ok(lse, q):
    B, H, N, _ = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on the inputs' device")


def _mask_ok(mask, q):
    N = q.shape[2]
    T = (N + MASK_BLOCK - 1) // MASK_BLOCK
    if mask.shape != (T, T) or mask.dtype != torch.uint8 or mask.device != q.device or not mask.is_contiguous():
        raise ValueError(f"block_mask must be a contiguous uint8 [{T}, {T}] tensor on the inputs' device")


def timing_enable(on: bool = True):
    _check(lib().flash_attn_timing_enable(int(bool(on))))


def timing_collect():
    """{kernel name: (total ms, launches)} since the last collect."""
    ms = (ctypes.c_double * KERNELS)()
    cnt = (ctypes.c_int * KERNELS)()
    _check(lib().flash_attn_timing_collect(ms, cnt, KERNELS))
    return {lib().flash_attn_kernel_name(i).decode(): (ms[i], cnt[i]) for i in range(KERNELS)}


def fwd(q, k, v, scale=None, causal=False):
    """(O, LSE) = flash_attn_fwd(q, k, v, scale, causal)."""
    B, H, N, d, dt = _shape(q, k, v)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(lib().flash_attn_fwd(B, H, N, d, dt, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                _scale(scale, d), int(bool(causal)), o.data_ptr(), lse.data_ptr(),
                                _stream(q)))
    return o, lse


def fwd_splitkv_workspace_size(B, H, N, d, num_splits, dtype=torch.bfloat16) -> int:
    return int(lib().flash_attn_fwd_splitkv_workspace_size(B, H, N, d, _DT[dtype], int(num_splits)))


def fwd_splitkv_num_splits(B, H, N, d, causal=False) -> int:
    return int(lib().flash_attn_fwd_splitkv_num_splits(B, H, N, d, int(bool(causal))))


def fwd_splitkv(q, k, v, num_splits=None, scale=None, causal=False, workspace=None):
    """(O, LSE) = flash_attn_fwd_splitkv(q, k, v, scale, causal, num_splits);
    num_splits None: flash_attn_fwd_splitkv_num_splits()."""
    B, H, N, d, dt = _shape(q, k, v)
    if num_splits is None:
        num_splits = fwd_splitkv_num_splits(B, H, N, d, causal)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = fwd_splitkv_workspace_size(B, H, N, d, num_splits, q.dtype)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib().flash_attn_fwd_splitkv(B, H, N, d, dt, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        _scale(scale, d), int(bool(causal)), int(num_splits), o.data_ptr(),
                                        lse.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(q)))
    return o, lse


def fwd_kvcache_workspace_size(B, H, Hkv, Nq, Nk, d, num_splits, dtype=torch.bfloat16) -> int:
    return int(lib().flash_attn_fwd_kvcache_workspace_size(B, H, Hkv, Nq, Nk, d, _DT[dtype], int(num_splits)))


def fwd_kvcache_num_splits(B, H, Hkv, Nq, Nk, d) -> int:
    return int(lib().flash_attn_fwd_kvcache_num_splits(B, H, Hkv, Nq, Nk, d))


def fwd_kvcache(q, k, v, cache_seqlens=None, num_splits=None, scale=None, causal=False, workspace=None):
    """(O [B, H, Nq, d], LSE [B, H, Nq]) = flash_attn_fwd_kvcache(...): q [B, H, Nq, d] against the
    key/value cache k, v [B, Hkv, Nk, d] (first cache_seqlens[b] slots valid, int32 [B] on the device,
    or all Nk); num_splits None: flash_attn_fwd_kvcache_num_splits()."""
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, Hkv, Nk, d]")
    if q.dtype not in _DT or not q.is_cuda:
        raise ValueError("tensors must be float16/bfloat16 on a HIP device (no CPU path exists)")
    B, H, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    for t in (k, v):
        if t.shape[0] != B or t.shape[3] != d or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError("k, v must be contiguous [B, Hkv, Nk, d] with q's batch, head size, dtype and device")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    lens = 0
    if cache_seqlens is not None:
        if cache_seqlens.dtype != torch.int32 or cache_seqlens.shape != (B,) or cache_seqlens.device != q.device \
                or not cache_seqlens.is_contiguous():
            raise ValueError("cache_seqlens must be a contiguous int32 [B] tensor on the inputs' device")
        lens = cache_seqlens.data_ptr()
    if num_splits is None:
        num_splits = fwd_kvcache_num_splits(B, H, Hkv, Nq, Nk, d)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    nbytes = fwd_kvcache_workspace_size(B, H, Hkv, Nq, Nk, d, num_splits, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib().flash_attn_fwd_kvcache(B, H, Hkv, Nq, Nk, d, _DT[q.dtype], q.data_ptr(), k.data_ptr(),
                                        v.data_ptr(), lens, _scale(scale, d), int(bool(causal)), int(num_splits),
                                        o.data_ptr(), lse.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                        _stream(q)))
    return o, lse


def bwd_workspace_size(B, H, N, d, dtype=torch.bfloat16) -> int:
    return int(lib().flash_attn_bwd_workspace_size(B, H, N, d, _DT[dtype]))


def _workspace(q):
    B, H, N, d = q.shape
    nbytes = bwd_workspace_size(B, H, N, d, q.dtype)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device), nbytes


def bwd(q, k, v, o, dout, lse, scale=None, causal=False, workspace=None):
    """(dQ, dK, dV) = flash_attn_bwd(q, k, v, o, dout, lse, scale, causal)."""
    B, H, N, d, dt = _shape(q, k, v, o, dout)
    _lse_ok(lse, q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws, nbytes = _workspace(q) if workspace is None else (workspace, workspace.numel())
    _check(lib().flash_attn_bwd(B, H, N, d, dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                dout.data_ptr(), lse.data_ptr(), _scale(scale, d), int(bool(causal)),
                                dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), nbytes,
                                _stream(q)))
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, dout, lse, scale=None, causal=False, dq=None, dk=None, dv=None):
    """(dQ, dK, dV) = flash_attn_bwd_noalloc(...): the backward with its
    workspace held by the library (no device allocation in the call; pass
    dq, dk, dv to avoid torch allocating the outputs too)."""
    B, H, N, d, dt = _shape(q, k, v, o, dout)
    _lse_ok(lse, q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t in (dq, dk, dv):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError("dq, dk, dv must be contiguous tensors shaped like q")
    _check(lib().flash_attn_bwd_noalloc(B, H, N, d, dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        dout.data_ptr(), lse.data_ptr(), _scale(scale, d), int(bool(causal)),
                                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _stream(q)))
    return dq, dk, dv


def blocksparse_fwd(q, k, v, block_mask, scale=None, causal=False):
    """(O, LSE) = flash_attn_blocksparse_fwd(..., block_mask [T, T] uint8, 128)."""
    B, H, N, d, dt = _shape(q, k, v)
    _mask_ok(block_mask, q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(lib().flash_attn_blocksparse_fwd(B, H, N, d, dt, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                            _scale(scale, d), int(bool(causal)), block_mask.data_ptr(),
                                            MASK_BLOCK, o.data_ptr(), lse.data_ptr(), _stream(q)))
    return o, lse


def blocksparse_bwd(q, k, v, o, dout, lse, block_mask, scale=None, causal=False, workspace=None):
    """(dQ, dK, dV) = flash_attn_blocksparse_bwd(...)."""
    B, H, N, d, dt = _shape(q, k, v, o, dout)
    _lse_ok(lse, q)
    _mask_ok(block_mask, q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws, nbytes = _workspace(q) if workspace is None else (workspace, workspace.numel())
    _check(lib().flash_attn_blocksparse_bwd(B, H, N, d, dt, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                            o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                                            _scale(scale, d), int(bool(causal)), block_mask.data_ptr(),
                                            MASK_BLOCK, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                            ws.data_ptr(), nbytes, _stream(q)))
    return dq, dk, dv


def fwd_gqa(q, k, v, scale=None, causal=False):
    """(O, LSE) = flash_attn_fwd_gqa(q [B,H,N,d], k, v [B,Hkv,N,d], scale, causal)."""
    B, H, Hkv, N, d, dt = _shape_gqa(q, k, v)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(lib().flash_attn_fwd_gqa(B, H, Hkv, N, d, dt, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    _scale(scale, d), int(bool(causal)), o.data_ptr(), lse.data_ptr(),
                                    _stream(q)))
    return o, lse


def bwd_gqa_workspace_size(B, H, Hkv, N, d, dtype=torch.bfloat16) -> int:
    return int(lib().flash_attn_bwd_gqa_workspace_size(B, H, Hkv, N, d, _DT[dtype]))


def bwd_gqa(q, k, v, o, dout, lse, scale=None, causal=False, workspace=None):
    """(dQ, dK, dV) = flash_attn_bwd_gqa(...); dK, dV have the shape of k, v."""
    B, H, Hkv, N, d, dt = _shape_gqa(q, k, v, o, dout)
    _lse_ok(lse, q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        nbytes = bwd_gqa_workspace_size(B, H, Hkv, N, d, q.dtype)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    else:
        ws, nbytes = workspace, workspace.numel()
    _check(lib().flash_attn_bwd_gqa(B, H, Hkv, N, d, dt, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    o.data_ptr(), dout.data_ptr(), lse.data_ptr(), _scale(scale, d),
                                    int(bool(causal)), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                    ws.data_ptr(), nbytes, _stream(q)))
    return dq, dk, dv


def _varlen(q, k, v, cu_seqlens, *per_query):
    """Packed batch: q (and o, dout) [total, H, d], k, v [total, Hkv, d], cu_seqlens int32 [B + 1]."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed tensors must be [total, heads, d]")
    if q.dtype not in _DT or not q.is_cuda:
        raise ValueError("packed tensors must be float32/float16/bfloat16 on a HIP device (no CPU path exists)")
    total, H, d = q.shape
    for t in per_query:
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError("o and dout must match q")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    Hkv = k.shape[1]
    for t in (k, v):
        if t.shape != (total, Hkv, d) or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError("k, v must be contiguous [total, Hkv, d] with q's length, head size, dtype, device")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != q.device \
            or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 [B + 1] tensor on the inputs' device")
    return cu_seqlens.numel() - 1, H, Hkv, total, d, _DT[q.dtype]


def varlen_fwd(q, k, v, cu_seqlens, max_seqlen, scale=None, causal=False):
    """(O [total, H, d], LSE [H, total]) = flash_attn_varlen_fwd(...)."""
    B, H, Hkv, total, d, dt = _varlen(q, k, v, cu_seqlens)
    o = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    _check(lib().flash_attn_varlen_fwd(B, H, Hkv, total, int(max_seqlen), d, dt, cu_seqlens.data_ptr(),
                                       q.data_ptr(), k.data_ptr(), v.data_ptr(), _scale(scale, d),
                                       int(bool(causal)), o.data_ptr(), lse.data_ptr(), _stream(q)))
    return o, lse


def varlen_bwd_workspace_size(B, H, Hkv, total, max_seqlen, d, dtype=torch.bfloat16) -> int:
    return int(lib().flash_attn_varlen_bwd_workspace_size(B, H, Hkv, total, max_seqlen, d, _DT[dtype]))


def varlen_bwd(q, k, v, o, dout, lse, cu_seqlens, max_seqlen, scale=None, causal=False, workspace=None):
    """(dQ, dK, dV) = flash_attn_varlen_bwd(...); lse is the forward's [H, total]."""
    B, H, Hkv, total, d, dt = _varlen(q, k, v, cu_seqlens, o, dout)
    if lse.shape != (H, total) or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [H, total] tensor on the inputs' device")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        nbytes = varlen_bwd_workspace_size(B, H, Hkv, total, int(max_seqlen), d, q.dtype)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    else:
        ws, nbytes = workspace, workspace.numel()
    _check(lib().flash_attn_varlen_bwd(B, H, Hkv, total, int(max_seqlen), d, dt, cu_seqlens.data_ptr(),
                                       q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                       lse.data_ptr(), _scale(scale, d), int(bool(causal)), dq.data_ptr(),
                                       dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), nbytes, _stream(q)))
    return dq, dk, dv


def fwd_dropout(q, k, v, dropout_p, seed, offset=0, scale=None, causal=False):
    """(O, LSE) = flash_attn_fwd_dropout(...): dropout on P, decisions from Philox4x32-10(seed, offset)."""
    B, H, N, d, dt = _shape(q, k, v)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(lib().flash_attn_fwd_dropout(B, H, N, d, dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), _scale(scale, d),
                                        int(bool(causal)), float(dropout_p), int(seed), int(offset), o.data_ptr(),
                                        lse.data_ptr(), _stream(q)))
    return o, lse


def bwd_dropout(q, k, v, o, dout, lse, dropout_p, seed, offset=0, scale=None, causal=False, workspace=None):
    """(dQ, dK, dV) = flash_attn_bwd_dropout(...) with the forward's dropout_p, seed and offset."""
    B, H, N, d, dt = _shape(q, k, v, o, dout)
    _lse_ok(lse, q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws, nbytes = _workspace(q) if workspace is None else (workspace, workspace.numel())
    _check(lib().flash_attn_bwd_dropout(B, H, N, d, dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        dout.data_ptr(), lse.data_ptr(), _scale(scale, d), int(bool(causal)),
                                        float(dropout_p), int(seed), int(offset), dq.data_ptr(), dk.data_ptr(),
                                        dv.data_ptr(), ws.data_ptr(), nbytes, _stream(q)))
    return dq, dk, dv


def varlen_fwd_dropout(q, k, v, cu_seqlens, max_seqlen, dropout_p, seed, offset=0, scale=None, causal=False):
    """(O [total, H, d], LSE [H, total]) = flash_attn_varlen_fwd_dropout(...)."""
    B, H, Hkv, total, d, dt = _varlen(q, k, v, cu_seqlens)
    o = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    _check(lib().flash_attn_varlen_fwd_dropout(B, H, Hkv, total, int(max_seqlen), d, dt, cu_seqlens.data_ptr(),
                                               q.data_ptr(), k.data_ptr(), v.data_ptr(), _scale(scale, d),
                                               int(bool(causal)), float(dropout_p), int(seed), int(offset),
                                               o.data_ptr(), lse.data_ptr(), _stream(q)))
    return o, lse


def varlen_bwd_dropout(q, k, v, o, dout, lse, cu_seqlens, max_seqlen, dropout_p, seed, offset=0, scale=None,
                       causal=False, workspace=None):
    """(dQ, dK, dV) = flash_attn_varlen_bwd_dropout(...)."""
    B, H, Hkv, total, d, dt = _varlen(q, k, v, cu_seqlens, o, dout)
    if lse.shape != (H, total) or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [H, total] tensor on the inputs' device")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        nbytes = varlen_bwd_workspace_size(B, H, Hkv, total, int(max_seqlen), d, q.dtype)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    else:
        ws, nbytes = workspace, workspace.numel()
    _check(lib().flash_attn_varlen_bwd_dropout(B, H, Hkv, total, int(max_seqlen), d, dt, cu_seqlens.data_ptr(),
                                               q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                               dout.data_ptr(), lse.data_ptr(), _scale(scale, d),
                                               int(bool(causal)), float(dropout_p), int(seed), int(offset),
                                               dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), nbytes,
                                               _stream(q)))
    return dq, dk, dv
