"""Helpers shared by the GPU tests: host <-> device copies of bf16 bit
patterns and the acceptance rules for scores and masks."""
from __future__ import annotations

import numpy as np
import torch


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda() if dtype is None else torch.from_numpy(a.astype(dtype)).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def padded(a: np.ndarray, ld: int, fill: int = 0) -> torch.Tensor:
    """Device copy of a uint16 matrix with row stride ld (extra columns = fill);
    returns the [rows][ld] tensor (callers slice [:, :width])."""
    rows, w = a.shape
    buf = np.full((rows, ld), fill, dtype=np.uint16)
    buf[:, :w] = a
    return dev(buf)


def scores_close(got, ref, rel=1e-2):
    """|got - ref| <= rel * max(|ref|, 1e-6 * max|ref|), elementwise."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    floor = 1e-6 * max(float(np.abs(ref).max()), 1e-30)
    bound = rel * np.maximum(np.abs(ref), floor)
    err = np.abs(got - ref)
    ok = err <= bound
    return bool(ok.all()), float((err / np.maximum(np.abs(ref), floor)).max())


def mask_acceptable(mask_gpu, mask_ref, scores_ref, theta_ref, rel=1e-2):
    """Masks may differ only on blocks whose oracle score lies within rel of
    the oracle threshold."""
    diff = np.nonzero(np.asarray(mask_gpu) != np.asarray(mask_ref))[0]
    near = np.abs(np.asarray(scores_ref, np.float64)[diff] - float(theta_ref)) <= rel * abs(float(theta_ref))
    return bool(near.all()), diff
