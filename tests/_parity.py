"""Helpers for GPU-vs-oracle parity tests (comparison and input plumbing)."""
from __future__ import annotations

import math

import numpy as np
import torch

from io_aware_exact_flash_amd import workloads

# Tolerances (max abs error over every compared element).  O and gradient
# bounds for 16-bit inputs and the float32 bound are the stated targets; the
# LSE bound for 16-bit inputs is derived: LSE depends on Q and K only through
# float32 arithmetic on exactly representable inputs, so its error is a few
# float32 roundings of values of magnitude |S| < 100, far below 1e-3.
TOL = {
    "f32": dict(o=1e-5, lse=1e-5),
    "bf16": dict(o=2e-2, lse=1e-3, grad=5e-2),
    "f16": dict(o=2e-2, lse=1e-3, grad=5e-2),
}
# Relative RMS error ceiling for 16-bit paths, a much tighter second gate: a
# 16-bit rounding of P or dS contributes ~2^-9 relative error per element and
# output rounding another 2^-9, so 1e-2 leaves a wide margin while a dropped
# term or mis-indexed tile gives O(1).
REL_RMS = {"bf16": 1e-2, "f16": 1e-2, "f32": 1e-6}


def fp32_scale(d):
    return float(np.float32(1.0 / math.sqrt(d)))


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


# Achieved errors of every comparison in this process, {test: [(name, max
# abs error, relative RMS error, bound)]}; tests/conftest.py writes them to
# the JSON file named by FA_PARITY_LOG at the end of the session.
RECORD = {}
CURRENT_TEST = ["(none)"]


def compare(name, got, ref, atol, rel_rms=None, mask=None):
    """Assert max|got - ref| <= atol (and the relative RMS gate); returns stats."""
    g = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, f"{name}: shape {g.shape} vs {r.shape}"
    if mask is not None:
        g, r = g[mask], r[mask]
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    if g.size == 0:
        return 0.0, 0.0
    err = float(np.abs(g - r).max())
    nr = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(g - r) / nr) if nr > 0 else float(np.linalg.norm(g - r))
    RECORD.setdefault(CURRENT_TEST[0], []).append((name, err, rel, float(atol)))
    assert err <= atol, f"{name}: max abs error {err:.3e} > {atol:.1e} (rel rms {rel:.2e})"
    if rel_rms is not None:
        assert rel <= rel_rms, f"{name}: relative RMS error {rel:.2e} > {rel_rms:.1e} (max abs {err:.2e})"
    return err, rel


def compare_lse(name, got, ref, atol):
    g = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got)
    r = np.asarray(ref)
    ninf_r = np.isneginf(r)
    assert (np.isneginf(g) == ninf_r).all(), f"{name}: -inf pattern differs"
    return compare(name, g[~ninf_r], r[~ninf_r], atol)


def make(B, H, N, d, dtype, seed, gain=1.0, device="cuda"):
    """CPU tensors from the shared generator, their GPU copies, float64 views."""
    cpu = workloads.qkvdo(B, H, N, d, dtype, seed=seed, gain=gain)
    gpu = tuple(t.to(device) for t in cpu)
    f64 = tuple(t.to(torch.float64).numpy() for t in cpu)
    return gpu, f64
