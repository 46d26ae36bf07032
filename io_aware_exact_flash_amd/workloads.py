"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module draws random numbers and nothing else: it holds none of the
attention arithmetic, imports neither the GPU library nor the oracle, and
both sides receive exactly the tensors it returns.

Recipe (one generator per purpose, CPU ``torch.Generator``):

* ``qkvdo(B, H, N, d, dtype, seed, gain)`` draws Q, K, V, dO in that order as
  iid N(0, 1) float32 ``[B, H, N, d]``, multiplies by ``gain`` and rounds to
  ``dtype``.  The bench workloads use seed = workload number and gain 0.5
  only for the 8192-token causal workload.
* ``qkvdo_grouped(B, H, Hkv, N, d, dtype, seed, gain)`` draws the same way
  Q ``[B, H, N, d]``, K and V ``[B, Hkv, N, d]``, dO ``[B, H, N, d]``, in
  that order (grouped K/V heads).
* ``seq_lengths(B, max_len, seed)`` draws B sequence lengths uniformly in
  [1, max_len] and sets the first to max_len (the longest sequence of a
  packed batch); ``packed_qkvdo(lengths, H, Hkv, d, dtype, seed, gain)``
  draws Q ``[T, H, d]``, K, V ``[T, Hkv, d]``, dO ``[T, H, d]`` (T = the
  sum of the lengths) in that order and returns them with the int32
  offsets ``cu`` = 0, l0, l0 + l1, ... .
* ``kvcache_qkv(B, H, Hkv, Nq, Nk, d, dtype, seed, gain)`` draws, for a
  decoding step, Q ``[B, H, Nq, d]`` then the cache K, V ``[B, Hkv, Nk, d]``
  in that order.
* ``block_mask(T, density, seed)`` keeps every diagonal block and each
  off-diagonal block with probability p = (density T^2 - T) / (T^2 - T), so
  the expected kept fraction is ``density``; drawn as ``rand(T, T) < p``.
* ``head_subset(B, H, count, seed)`` picks (b, h) pairs for oracle checks of
  large workloads, always including (0, 0) and (B-1, H-1).
"""
from __future__ import annotations

import torch

_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# The five workloads of the benchmark suite: (B, H, N, d, dtype, causal,
# sparse density or None, gain, passes).
WORKLOADS = {
    1: dict(name="single-head fp32 forward", B=1, H=1, N=256, d=64, dtype="f32",
            causal=False, density=None, gain=1.0, backward=False),
    2: dict(name="batched training shape", B=8, H=16, N=1024, d=64, dtype="bf16",
            causal=False, density=None, gain=1.0, backward=True),
    3: dict(name="gpt-style causal", B=4, H=32, N=2048, d=128, dtype="bf16",
            causal=True, density=None, gain=1.0, backward=True),
    4: dict(name="long-context causal", B=4, H=40, N=8192, d=128, dtype="bf16",
            causal=True, density=None, gain=0.5, backward=True),
    5: dict(name="block-sparse", B=2, H=16, N=16384, d=64, dtype="f16",
            causal=False, density=0.25, gain=1.0, backward=True),
}


def torch_dtype(name: str) -> torch.dtype:
    return _DTYPES[name]


def qkvdo(B, H, N, d, dtype="bf16", seed=0, gain=1.0):
    """Q, K, V, dO as CPU tensors of ``dtype``, drawn in that order."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    out = []
    for _ in range(4):
        x = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
        if gain != 1.0:
            x = x * gain
        out.append(x.to(_DTYPES[dtype]))
    return tuple(out)


def qkvdo_grouped(B, H, Hkv, N, d, dtype="bf16", seed=0, gain=1.0):
    """Q, K, V, dO as CPU tensors of ``dtype``; K and V have Hkv heads."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    out = []
    for heads in (H, Hkv, Hkv, H):
        x = torch.randn((B, heads, N, d), generator=g, dtype=torch.float32)
        if gain != 1.0:
            x = x * gain
        out.append(x.to(_DTYPES[dtype]))
    return tuple(out)


def kvcache_qkv(B, H, Hkv, Nq, Nk, d, dtype="bf16", seed=0, gain=1.0):
    """Q [B, H, Nq, d] and the key/value cache K, V [B, Hkv, Nk, d] as CPU
    tensors of ``dtype``, drawn in that order."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    out = []
    for heads, n in ((H, Nq), (Hkv, Nk), (Hkv, Nk)):
        x = torch.randn((B, heads, n, d), generator=g, dtype=torch.float32)
        if gain != 1.0:
            x = x * gain
        out.append(x.to(_DTYPES[dtype]))
    return tuple(out)


def seq_lengths(B: int, max_len: int, seed: int):
    """B lengths uniform in [1, max_len], the first one max_len."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    lens = torch.randint(1, max_len + 1, (B,), generator=g).tolist()
    if B:
        lens[0] = max_len
    return lens


def packed_qkvdo(lengths, H, Hkv, d, dtype="bf16", seed=0, gain=1.0):
    """Packed batch: Q, K, V, dO as CPU tensors and int32 offsets cu [B + 1]."""
    T = int(sum(lengths))
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    out = []
    for heads in (H, Hkv, Hkv, H):
        x = torch.randn((T, heads, d), generator=g, dtype=torch.float32)
        if gain != 1.0:
            x = x * gain
        out.append(x.to(_DTYPES[dtype]))
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if lengths:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return (*out, cu)


def block_mask(T: int, density: float, seed: int) -> torch.Tensor:
    """uint8 [T, T] block mask, diagonal kept, expected density ``density``."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    if T <= 1:
        return torch.ones((T, T), dtype=torch.uint8)
    p = (density * T * T - T) / (T * T - T)
    p = min(max(p, 0.0), 1.0)
    m = (torch.rand((T, T), generator=g) < p).to(torch.uint8)
    m.fill_diagonal_(1)
    return m


def head_subset(B: int, H: int, count: int, seed: int):
    """``count`` distinct (b, h) pairs including (0, 0) and (B-1, H-1)."""
    pairs = [(0, 0)]
    if (B - 1, H - 1) not in pairs:
        pairs.append((B - 1, H - 1))
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    order = torch.randperm(B * H, generator=g).tolist()
    for idx in order:
        if len(pairs) >= min(count, B * H):
            break
        p = (idx // H, idx % H)
        if p not in pairs:
            pairs.append(p)
    return pairs


def workload_inputs(num: int):
    """Inputs of benchmark workload ``num`` (seed = workload number)."""
    w = WORKLOADS[num]
    q, k, v, do = qkvdo(w["B"], w["H"], w["N"], w["d"], w["dtype"], seed=num, gain=w["gain"])
    mask = None
    if w["density"] is not None:
        T = (w["N"] + 127) // 128
        mask = block_mask(T, w["density"], seed=num + 1000)
    return q, k, v, do, mask
