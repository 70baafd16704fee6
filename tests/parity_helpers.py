"""Helpers for the GPU parity tests: host<->device transfer and the
comparison metrics.

Metrics (the contract for float outputs):
  * row-normalised error: max over (i, j) of |y - R| / ||R[i, :]||_2 <= 1e-3,
    and |y - R| <= 1e-6 on rows whose reference norm is 0 -- applied as is
    to every output of rows of n >= 256 values (rows_ok);
  * short rows (n < 256): the output is one bf16 rounding of a value that
    meets the bound, so the allowance is 1e-3 * ||R[i, :]||_2 + 2^-8 * |R|
    (half a bf16 step; at n = 1 the row norm is |R| itself and bf16 rounding
    alone can reach 2^-9 |R| > 1e-3 |R|);
  * BF16-dequant fallback: ||Y - R||_F / ||R||_F <= 2e-2;
  * elementwise bf16 results computed in binary32 (silu_mul): at most one
    bf16 step from the oracle's fp64 value rounded to bf16.
"""
from __future__ import annotations

import numpy as np
import torch

import inputs

ROW_TOL = 1e-3
FROB_TOL = 2e-2


def dev_u8(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device)


def dev_bf16(a: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bfloat16 tensor (bit copy)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).to(device)
    return t.view(torch.bfloat16)


def empty_bf16(shape, device) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.bfloat16, device=device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """device bf16 tensor -> uint16 bit patterns."""
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return inputs.bf16_bits_to_f32(host_bits(t)).astype(np.float64)


def row_error(y: np.ndarray, R: np.ndarray) -> float:
    """max |y - R| / ||R_row||_2; rows with zero norm are checked absolutely."""
    y = np.atleast_2d(y)
    R = np.atleast_2d(R)
    norms = np.linalg.norm(R, axis=1)
    err = np.abs(y - R)
    out = 0.0
    for i in range(R.shape[0]):
        if norms[i] == 0:
            if err[i].max() > 1e-6:
                return float("inf")
        else:
            out = max(out, float(err[i].max() / norms[i]))
    return out


def rounded_row_ok(y: np.ndarray, R: np.ndarray) -> bool:
    """Edge-shape check: |y - R| <= 1e-3 ||R_row|| + 2^-8 |R| elementwise."""
    y = np.atleast_2d(y)
    R = np.atleast_2d(R)
    bound = ROW_TOL * np.linalg.norm(R, axis=1, keepdims=True) + 2.0 ** -8 * np.abs(R) + 1e-6
    return bool(np.all(np.abs(y - R) <= bound))


def rows_ok(y: np.ndarray, R: np.ndarray) -> bool:
    """The row-normalised bound for rows of n >= 256 outputs; the short-row
    allowance (one bf16 rounding on top of it) below that."""
    R = np.atleast_2d(R)
    if R.shape[1] >= 256:
        return row_error(y, R) <= ROW_TOL
    return rounded_row_ok(y, R)


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps between two bf16 bit arrays (sign-magnitude order)."""
    def ordered(b):
        b = np.asarray(b, dtype=np.uint16).astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def frob_error(y: np.ndarray, R: np.ndarray) -> float:
    return float(np.linalg.norm(y - R) / np.linalg.norm(R))


def q8_planes(q8: np.ndarray, m: int, k: int):
    kp = (k + 255) // 256 * 256
    return q8[: m * kp].reshape(m, kp), q8[m * kp:].reshape(m, kp // 32, 4)
