"""Helpers shared by the GPU parity tests (host-side marshalling only)."""
from __future__ import annotations

import sys

import numpy as np
import torch

TORCH16 = {"bf16": torch.bfloat16, "f16": torch.float16}
OUT = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def dev16(bits: np.ndarray, dtype: str) -> torch.Tensor:
    """uint16 patterns -> a GPU tensor of the 16-bit type (bit copy)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH16[dtype])
    return t.cuda()


def host_stored(y: torch.Tensor, dtype: str) -> np.ndarray:
    """GPU output -> the stored representation the oracle returns
    (uint16 patterns for 16-bit outputs, float32 values for f32)."""
    y = y.cpu()
    if dtype == "f32":
        return y.numpy()
    return y.view(torch.int16).numpy().view(np.uint16)


def rel_fro(a: np.ndarray, ref: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(a - ref) / den) if den > 0 else float(np.linalg.norm(a))


def row_rel_fro(a: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Relative Frobenius error of each row (massive-activation rows would
    otherwise dominate a single global norm)."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref, axis=1)
    num = np.linalg.norm(a - ref, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def announce(*parts) -> None:
    """Name the case on stdout before a GPU step, flushed."""
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()
