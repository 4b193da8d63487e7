"""Seeded synthetic attention-layer inputs shaped like video-DiT self-attention.

This module only draws numbers.  It holds none of the method's arithmetic
(no softmax, no masses, no selection) and is the one piece of code that both
the fp64 oracle (``oracle/``) and the GPU path's tests and benchmark use, so
that both sides see bit-identical inputs.

Workloads (layer shapes of the video diffusion transformers that the LoSA
paper evaluates, "LoSA: Near-Lossless Sparse Attention ...", Experiments
Summary / Experimental setup; the trained checkpoints and prompts are not
available, so seeded synthetic activations of the same shape stand in for
them):

  id  name            heads  d    grid T x H x W   tokens   block  dtype
  0   tiny            2      64   4 x 16 x 16      1024     64     f32
  1   wan13b_480p     12     128  21 x 30 x 52     32760    64     bf16
  2   wan14b_720p     40     128  21 x 45 x 80     75600    64     bf16
  3   hunyuan_720p    24     128  33 x 45 x 80     118800   128    bf16
  4   reuse           = id 1, 50 denoising steps with Q/K drift, per-head p
  1s  wan13b_sparse   = id 1 with feature amplitude 11 (coverage ~0.6 at
                        p = 0.99, the "~40% of blocks removed" regime)

Recipe, per workload id c, with ``rng = Generator(PCG64(seed))`` (seed = c,
11 for "1s") and draws in exactly this order:

1. Token n = (t*H + y)*W + x in raster order at position (t/T, y/H, x/W).
2. Sinks: floor(N/100) distinct tokens ``rng.choice(N, n_sink, replace=False)``,
   shared by all heads.
3. For each head, in order: sigma ~ U[2, sigma_max]; Omega ~ N(0, sigma^2)
   of shape 3 x d; b ~ U[0, 2 pi) of shape d; phi = cos(x Omega + b) scaled
   to unit L2 norm per token; q = a*phi + N(0,1)^(N x d);
   k = a*phi + N(0,1)^(N x d); k[sinks] *= 2; v = N(0,1)^(N x d).
   a = 3 (11 for "1s"); sigma_max = 16 (24 for id 2).
4. Rounding: to fp32 (round to nearest even); bf16 workloads then round the
   fp32 value to bf16 (round to nearest even).  Padding rows N..N_alloc-1
   (N_alloc = ceil(N/block)*block) are zero.
5. Workload 4 only: after the heads, p_h is drawn per head uniformly from
   {0.90, 0.95, 0.99, 0.995}; step s (0..49) uses q_s = q_0 + 0.02*s*z_q and
   k_s = k_0 + 0.02*s*z_k, where q_0/k_0 are the unrounded fp64 values of
   step 3 (sinks applied) and z_q, z_k ~ N(0,1) are drawn (z_q first, head
   by head) from ``Generator(PCG64([4, s]))``; V does not drift.

bf16 tensors are held as uint16 bit patterns (numpy has no bf16 type).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "get_workload",
    "Layer",
    "make_layer",
    "drift_qk",
    "bf16_bits_from_f32",
    "f64_from_bf16_bits",
    "to_f64",
    "f32_round",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: str
    name: str
    heads: int
    head_dim: int
    grid: Tuple[int, int, int]
    block: int
    dtype: str  # "f32" | "bf16"
    p: float
    sigma_max: float = 16.0
    amplitude: float = 3.0
    seed: int = 0
    batch: int = 1
    steps: int = 1
    construct_step: int = 0
    per_head_p: Tuple[float, ...] = ()
    k_block: int = 0  # key-block size C when it differs from the query-block size R (= block)

    @property
    def key_block(self) -> int:
        return self.k_block or self.block

    @property
    def tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def n_blocks(self) -> int:
        return -(-self.tokens // self.block)

    @property
    def n_key_blocks(self) -> int:
        return -(-self.tokens // self.key_block)

    @property
    def tokens_alloc(self) -> int:
        return max(self.n_blocks * self.block, self.n_key_blocks * self.key_block)


WORKLOADS: Dict[str, Workload] = {
    "0": Workload("0", "tiny", 2, 64, (4, 16, 16), 64, "f32", 0.99, seed=0),
    "1": Workload("1", "wan13b_480p", 12, 128, (21, 30, 52), 64, "bf16", 0.99, seed=1),
    "2": Workload("2", "wan14b_720p", 40, 128, (21, 45, 80), 64, "bf16", 0.99,
                  sigma_max=24.0, seed=2),
    "3": Workload("3", "hunyuan_720p", 24, 128, (33, 45, 80), 128, "bf16", 0.99, seed=3),
    "4": Workload("4", "reuse", 12, 128, (21, 30, 52), 64, "bf16", 0.99, seed=4,
                  steps=50, construct_step=2, per_head_p=(0.90, 0.95, 0.99, 0.995)),
    "1s": Workload("1s", "wan13b_sparse", 12, 128, (21, 30, 52), 64, "bf16", 0.99,
                   amplitude=11.0, seed=11),
    # workload 3's layer (same seed) with the page's own block shape: 128-token
    # query blocks, 32-token key blocks
    "3n": Workload("3n", "hunyuan_720p_r128_c32", 24, 128, (33, 45, 80), 128, "bf16", 0.99, seed=3,
                   k_block=32),
}


def get_workload(wid) -> Workload:
    return WORKLOADS[str(wid)]


def f32_round(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32, round to nearest even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def bf16_bits_from_f32(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest even.  Inputs here are finite."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def f64_from_bf16_bits(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array (f32 values or bf16 bit patterns) -> exact fp64 values."""
    if dtype == "bf16":
        return f64_from_bf16_bits(arr)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = f32_round(x64)
    if dtype == "bf16":
        return bf16_bits_from_f32(x32)
    return x32


@dataclasses.dataclass
class Layer:
    """One synthetic self-attention layer: storage arrays [B, H, N_alloc, d]."""
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    heads: Tuple[int, ...]
    p_heads: Optional[np.ndarray] = None  # workload 4: per-head p (over all heads)
    q0_f64: Optional[np.ndarray] = None   # workload 4: unrounded step-0 values
    k0_f64: Optional[np.ndarray] = None

    @property
    def dtype(self) -> str:
        return self.wl.dtype

    def f64(self, name: str) -> np.ndarray:
        return to_f64(getattr(self, name), self.wl.dtype)


def _positions(grid: Tuple[int, int, int]) -> np.ndarray:
    T, Hg, Wg = grid
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(Wg), indexing="ij")
    return np.stack([t.ravel() / T, y.ravel() / Hg, x.ravel() / Wg], axis=1).astype(np.float64)


def make_layer(wl, heads: Optional[Sequence[int]] = None, keep_f64: bool = False,
               tokens: Optional[int] = None, n_heads: Optional[int] = None) -> Layer:
    """Draw one layer of workload ``wl`` (a Workload or its id).

    ``heads`` restricts which heads are materialised (all draws still happen,
    in order, so head h is identical whether or not others are kept).
    ``tokens``/``n_heads`` override the grid size for small test cases
    (the grid becomes 1 x 1 x tokens); draws follow the same recipe.
    """
    if not isinstance(wl, Workload):
        wl = get_workload(wl)
    if tokens is not None or n_heads is not None:
        n_tok = tokens if tokens is not None else wl.tokens
        wl = dataclasses.replace(wl, grid=(1, 1, n_tok) if tokens is not None else wl.grid,
                                 heads=n_heads if n_heads is not None else wl.heads)
    H, d, N, Na = wl.heads, wl.head_dim, wl.tokens, wl.tokens_alloc
    keep = tuple(range(H)) if heads is None else tuple(int(h) for h in heads)
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    pos = _positions(wl.grid)
    n_sink = N // 100
    sinks = rng.choice(N, size=n_sink, replace=False) if n_sink > 0 else np.zeros(0, np.int64)
    sdt = np.uint16 if wl.dtype == "bf16" else np.float32
    shape = (wl.batch, len(keep), Na, d)
    q = np.zeros(shape, sdt)
    k = np.zeros(shape, sdt)
    v = np.zeros(shape, sdt)
    q0 = np.zeros(shape, np.float64) if keep_f64 else None
    k0 = np.zeros(shape, np.float64) if keep_f64 else None
    slot = {h: i for i, h in enumerate(keep)}
    for b in range(wl.batch):
        for h in range(H):
            sigma = rng.uniform(2.0, wl.sigma_max)
            omega = rng.normal(0.0, sigma, size=(3, d))
            bias = rng.uniform(0.0, 2.0 * np.pi, size=d)
            phi = np.cos(pos @ omega + bias)
            phi /= np.linalg.norm(phi, axis=1, keepdims=True)
            qh = wl.amplitude * phi + rng.standard_normal((N, d))
            kh = wl.amplitude * phi + rng.standard_normal((N, d))
            kh[sinks] *= 2.0
            vh = rng.standard_normal((N, d))
            if h in slot:
                s = slot[h]
                q[b, s, :N] = _store(qh, wl.dtype)
                k[b, s, :N] = _store(kh, wl.dtype)
                v[b, s, :N] = _store(vh, wl.dtype)
                if keep_f64:
                    q0[b, s, :N] = qh
                    k0[b, s, :N] = kh
    p_heads = None
    if wl.per_head_p:
        p_heads = rng.choice(np.asarray(wl.per_head_p, dtype=np.float64), size=H)
    return Layer(wl, q, k, v, keep, p_heads, q0, k0)


def drift_qk(layer: Layer, step: int) -> Tuple[np.ndarray, np.ndarray]:
    """Workload-4 step ``step``: (q_s, k_s) storage arrays from the kept fp64 base.

    z_q and z_k are drawn for every head (all heads of the workload, z_q for all
    heads first), so a head subset sees the same drift as the full layer.
    """
    wl = layer.wl
    if layer.q0_f64 is None:
        raise ValueError("drift_qk needs make_layer(..., keep_f64=True)")
    H, d, N = wl.heads, wl.head_dim, wl.tokens
    rng = np.random.Generator(np.random.PCG64([4, int(step)]))
    slot = {h: i for i, h in enumerate(layer.heads)}
    q = np.zeros_like(layer.q)
    k = np.zeros_like(layer.k)
    amp = 0.02 * step
    for name, base, out in (("q", layer.q0_f64, q), ("k", layer.k0_f64, k)):
        for b in range(wl.batch):
            for h in range(H):
                z = rng.standard_normal((N, d))
                if h in slot:
                    s = slot[h]
                    out[b, s, :N] = _store(base[b, s, :N] + amp * z, wl.dtype)
    return q, k
