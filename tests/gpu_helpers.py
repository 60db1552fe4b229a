"""Shared helpers for the GPU parity tests: moving stored values between numpy
and torch, and the parity metrics."""
from __future__ import annotations

import numpy as np
import torch

from workloads import as_f32

# Tolerances: bf16 storage with fp32 accumulation, and the fp32 mode.
BF16_MAX_ABS, BF16_REL_L2 = 2e-2, 5e-3
F32_MAX_ABS, F32_REL_L2 = 1e-5, 1e-5


def to_dev(a: np.ndarray) -> torch.Tensor:
    """Stored values (float32, or bf16 bits as uint16) onto the GPU."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_stored(t: torch.Tensor) -> np.ndarray:
    """Device tensor back to its stored representation on the host."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def metrics(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300))
    return max_abs, rel


def assert_parity(got, ref, bf16: bool, what: str = ""):
    max_abs, rel = metrics(got, ref)
    lim_abs, lim_rel = (BF16_MAX_ABS, BF16_REL_L2) if bf16 else (F32_MAX_ABS, F32_REL_L2)
    assert max_abs <= lim_abs and rel <= lim_rel, \
        f"{what}: max-abs {max_abs:.3e} (limit {lim_abs}), rel-L2 {rel:.3e} (limit {lim_rel})"
    return max_abs, rel


def bf16_ulp(v):
    """Spacing of bf16 numbers at |v| (8 significant bits)."""
    mag = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 1e-38)
    return np.ldexp(1.0, np.floor(np.log2(mag)).astype(np.int64) - 7)


def assert_projection_bf16(stored_bits: np.ndarray, ref: np.ndarray, abs_terms: np.ndarray, d: int,
                           what: str = "", rel_slack: float = 0.0):
    """A bf16 projection output against the fp64 projection.

    The kernel accumulates the d products in fp32 and rounds once to bf16, so
    each stored value may differ from the fp64 value by one bf16 ulp plus the
    fp32 dot-product error bound gamma_d * sum_c |y_c W_cj| (gamma_d = d*u/(1-d*u),
    u = 2^-24), and a few fp32 roundings of the row scale.  That bound only
    matters where the sum cancels; at least 99.9% of the values must also be
    within one ulp outright.  ``rel_slack`` widens the accumulation term for
    outputs that pass through further single-precision steps (the RoPE
    rotation's sine and cosine)."""
    got = as_f32(stored_bits).astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    err = np.abs(got - ref)
    ulp = bf16_ulp(np.maximum(np.abs(ref), np.abs(got)))
    terms = np.asarray(abs_terms, dtype=np.float64)
    bound = ulp + (gamma + rel_slack) * terms + 8 * u * np.abs(ref)
    bad = err > bound
    assert not np.any(bad), f"{what}: {int(bad.sum())} values outside one ulp + fp32 accumulation bound"
    frac = float(np.mean(err <= ulp))
    assert frac >= 0.999, f"{what}: only {frac:.5f} of values within one bf16 ulp"
