"""Exact IO-aware attention for MI355X (gfx950).

The compute lives in ``libflashattn.so`` (HIP kernels behind a C ABI declared
in ``include/flash_attn.h``); ``flash`` is its ctypes binding and
``workloads`` the seeded synthetic inputs.  Importing the package loads
nothing; the library is loaded on the first call and its absence is an
error, never a fallback.
"""
from .flash import (  # noqa: F401
    FlashAttnError,
    blocksparse_bwd,
    blocksparse_fwd,
    bwd,
    bwd_dropout,
    bwd_gqa,
    bwd_gqa_workspace_size,
    bwd_noalloc,
    bwd_workspace_size,
    fwd,
    fwd_kvcache,
    fwd_kvcache_num_splits,
    fwd_kvcache_workspace_size,
    fwd_dropout,
    fwd_gqa,
    fwd_splitkv,
    fwd_splitkv_num_splits,
    fwd_splitkv_workspace_size,
    lib,
    varlen_bwd,
    varlen_bwd_workspace_size,
    varlen_fwd,
    varlen_fwd_dropout,
    varlen_bwd_dropout,
)

__all__ = ["fwd", "bwd", "blocksparse_fwd", "blocksparse_bwd", "bwd_workspace_size", "fwd_splitkv", "fwd_splitkv_num_splits",
           "fwd_splitkv_workspace_size", "fwd_gqa", "bwd_gqa", "bwd_gqa_workspace_size", "varlen_fwd",
           "varlen_bwd", "varlen_bwd_workspace_size", "fwd_dropout", "bwd_dropout", "varlen_fwd_dropout", "varlen_bwd_dropout", "bwd_noalloc", "fwd_kvcache",
           "fwd_kvcache_num_splits", "fwd_kvcache_workspace_size", "lib", "FlashAttnError"]
