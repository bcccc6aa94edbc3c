"""Shared helpers of the GPU parity tests (marshalling and error measures only)."""
from __future__ import annotations

import numpy as np

# Tolerances of the attention output against the fp64 oracle (bf16 inputs,
# fp32 accumulation): max-abs 1e-2 and mean-abs 1e-3.
ATT_MAX_ABS = 1e-2
ATT_MEAN_ABS = 1e-3
# Sigmoid scores: |gpu - ref| <= 1e-6 |ref| + 2^-126 (the fp32 underflow floor).
SCORE_REL = 1e-6
SCORE_ABS = 2.0 ** -126


def to_dev_bf16(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)


def to_dev(a: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def check_scores(gpu: np.ndarray, ref: np.ndarray):
    g = gpu.astype(np.float64)
    bad = np.abs(g - ref) > SCORE_REL * np.abs(ref) + SCORE_ABS
    assert not bad.any(), f"{bad.sum()} scores off; worst rel {np.max(np.abs(g - ref) / np.abs(ref)):.3e}"


# The absolute bars above are loose where outputs are small (a softmax over
# thousands of N(0,1) tokens has output RMS about 0.01), so every check also
# bounds the largest error relative to the reference's RMS: 1e-3 by default,
# 1e-4 for the full-size workloads.  The kernel keeps about 16 significant
# bits of each softmax weight, so errors run near 1e-5 of the RMS.
ATT_MAX_REL_RMS = 1e-3
ATT_MAX_REL_RMS_FULL = 1e-4


def check_attention(gpu: np.ndarray, ref: np.ndarray, what: str = "", max_rel_rms: float = ATT_MAX_REL_RMS) -> dict:
    g = gpu.astype(np.float64)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) or 1.0
    stats = dict(max_abs=float(err.max()), mean_abs=float(err.mean()), max_rel_rms=float(err.max() / rms),
                 mean_rel_rms=float(err.mean() / rms), ref_rms=rms)
    assert stats["max_abs"] <= ATT_MAX_ABS and stats["mean_abs"] <= ATT_MEAN_ABS, f"{what}: {stats}"
    assert stats["max_rel_rms"] <= max_rel_rms, f"{what}: error relative to the output RMS too large: {stats}"
    return stats
