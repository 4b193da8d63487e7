"""Helpers for the GPU parity tests: moving synthetic layers to the device,
sampling rows, and the tolerances.

Tolerances (stated for the method's three outputs):
  block masses     elementwise relative error <= 1e-3 against the fp64 oracle;
  index lists      bit-exact when both selectors read the same fp32 masses;
  attention output max absolute error <= 1e-2 against the fp64 oracle
                   (bf16 inputs, fp32 accumulation, bf16 probabilities).
"""
from __future__ import annotations

import sys
import time
from typing import List, Sequence, Tuple

import numpy as np
import torch

import oracle as O
import synthetic as S

MASS_RTOL = 1e-3
ATTN_ATOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def layer_to_device(layer: S.Layer):
    return tuple(to_device(getattr(layer, n), layer.dtype) for n in ("q", "k", "v"))


def csr_to_device(row_ptr: np.ndarray, col_idx: np.ndarray, capacity: int = 0):
    rp = torch.from_numpy(np.asarray(row_ptr, np.int32)).cuda()
    ci_np = np.zeros(max(capacity, len(col_idx), 1), np.int32)
    ci_np[:len(col_idx)] = col_idx
    return rp, torch.from_numpy(ci_np).cuda()


def sample_rows(heads: int, n_q: int, seed: int, n_uniform: int = 48,
                extra: Sequence[Tuple[int, int, int]] = ()) -> List[Tuple[int, int, int]]:
    """Seeded row sample: the last (partial) query block of every head, the first
    block of head 0, and n_uniform uniform (h, i) rows."""
    rng = np.random.default_rng(seed)
    rows = {(0, h, n_q - 1) for h in range(heads)}
    rows.add((0, 0, 0))
    for _ in range(n_uniform):
        rows.add((0, int(rng.integers(heads)), int(rng.integers(n_q))))
    rows.update(extra)
    return sorted(rows)


def mass_rel_err(M_gpu: np.ndarray, M_ref: np.ndarray) -> float:
    assert np.all(M_ref > 0), "reference mass underflowed to 0"
    return float(np.max(np.abs(M_gpu.astype(np.float64) - M_ref) / M_ref))


def check_masses_with_floor(M_gpu, M_ref, label):
    """Relative error <= MASS_RTOL for masses in fp32's normal range; below
    2^-126 (unrepresentable in the fp32 output) absolute error <= 2^-126."""
    tiny = 2.0 ** -126
    small = M_ref < tiny
    if small.any():
        assert np.abs(M_gpu[small] - M_ref[small]).max() <= tiny
    rel = float((np.abs(M_gpu[~small] - M_ref[~small]) / M_ref[~small]).max())
    say(f"{label}: mass rel err {rel:.2e} on {(~small).sum()} normal masses ({small.sum()} below 2^-126)")
    assert rel <= MASS_RTOL
    return small


def row_csr(row_ptr: np.ndarray, col_idx: np.ndarray, r: int) -> np.ndarray:
    return np.asarray(col_idx[int(row_ptr[r]):int(row_ptr[r + 1])])


class Timer:
    def __init__(self, label):
        self.label = label

    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *a):
        say(f"  [{self.label}] {time.time() - self.t:.2f}s")
