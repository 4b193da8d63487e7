"""GPU parity of the block masses across fp32's range (LoSA page, Methodology
Summary: the construction step's masses are exact, not estimated).

Inputs whose scores form a ladder: each wave's first key block (blocks 0..3)
scores highest and every later block sits a fixed 50..120 log2 units lower,
so the masses run from about 2^-52 down to 2^-122 -- small, but normal fp32
numbers, which must come out with relative error <= 1e-3.  A second ladder
puts the four waves' first blocks far apart (0, -150, -100, 0) with later
blocks of the far-down waves much higher than their first ones.  Checked for
the mass call, the construction call (masses and dense O) and the sparse
attention with masses within full lists, against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from tests.gpu_util import ATTN_ATOL, check_masses_with_floor, csr_to_device, say, to_device

pytestmark = pytest.mark.gpu

import free_block_sparse_exact_amd as F  # noqa: E402

LOG2E = 1.4426950408889634


def ladder_levels(n_blocks, kind):
    if kind == "first_high":
        return [0.0] * 4 + list(-np.linspace(50.0, 120.0, n_blocks - 4))
    cyc = [-80.0, -60.0, -55.0, -90.0, -110.0, -120.0, -70.0, -65.0]
    return [0.0, -150.0, -100.0, 0.0] + [cyc[t % len(cyc)] for t in range(n_blocks - 4)]


def ladder_inputs(H, Na, N, d, C, levels, seed):
    """Scores of every query against key block j near levels[j] (log2 units):
    queries a*e0, keys of block j x_j*e0, plus small noise elsewhere."""
    rng = np.random.default_rng(seed)
    a = 16.0
    q = rng.standard_normal((1, H, Na, d)) * 0.05
    k = rng.standard_normal((1, H, Na, d)) * 0.05
    q[..., 0] = a
    for j, lv in enumerate(levels):
        x = lv * np.sqrt(d) / (a * LOG2E)
        k[:, :, j * C:(j + 1) * C, 0] = x + 0.1 * rng.standard_normal((1, H, min(C, Na - j * C)))
    v = rng.standard_normal((1, H, Na, d))
    for t in (q, k, v):
        t[:, :, N:] = 0.0
    return [S.bf16_bits_from_f32(x.astype(np.float32)) for x in (q, k, v)]


@pytest.mark.parametrize("kind", ["first_high", "first_apart"])
@pytest.mark.parametrize("R,C", [(64, 64), (128, 128), (64, 32), (128, 32)])
def test_masses_far_below_the_first_chunks(kind, R, C):
    H, d = 2, 128
    nb = 16
    N = nb * C - 24
    Na = max(-(-N // R) * R, nb * C)
    levels = ladder_levels(nb, kind)
    bits = ladder_inputs(H, Na, N, d, C, levels, seed=R + C + len(kind))
    q64, k64, v64 = (S.f64_from_bf16_bits(b) for b in bits)
    qd, kd, vd = (to_device(b, "bf16") for b in bits)
    say(f"ladder {kind} R={R} C={C} N={N}")
    M_ref = O.block_mass(q64, k64, N, R, C)
    assert M_ref.min() > 0.0
    normal = M_ref >= 2.0 ** -126
    say(f"  reference masses from {M_ref[normal].min():.3e} to {M_ref.max():.3e}")
    if kind == "first_high":
        assert normal.all() and M_ref.min() < 2.0 ** -100
    Mg = F.losa_block_mass(qd, kd, N, R, C).cpu().numpy().astype(np.float64)
    check_masses_with_floor(Mg, M_ref, f"  losa_block_mass {kind} R={R} C={C}")

    Od, Md = F.losa_dense_attn_mass(qd, kd, vd, N, R, C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_masses_with_floor(Md.cpu().numpy().astype(np.float64), M_ref, f"  losa_dense_attn_mass {kind} R={R} C={C}")
    O_ref = O.dense_attention(q64, k64, v64, N)
    err = float(np.abs(Od.cpu().numpy()[:, :, :N] - O_ref[:, :, :N]).max())
    say(f"  dense O max abs err {err:.3e}")
    assert err <= ATTN_ATOL

    nq, nk = -(-N // R), -(-N // C)
    rows = H * nq
    rp = np.arange(rows + 1, dtype=np.int64) * nk
    ci = np.tile(np.arange(nk, dtype=np.int32), rows)
    rp_d, ci_d = csr_to_device(rp, ci)
    Os, Ml = F.losa_sparse_attn_mass(qd, kd, vd, rp_d, ci_d, None, N, R, C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_masses_with_floor(Ml.cpu().numpy().astype(np.float64), M_ref, f"  losa_sparse_attn_mass {kind} R={R} C={C}")
    err = float(np.abs(Os.cpu().numpy()[:, :, :N] - O_ref[:, :, :N]).max())
    assert err <= ATTN_ATOL


@pytest.mark.parametrize("d,R,C", [(64, 64, 64), (128, 32, 64)])
def test_masses_far_below_simt_path(d, R, C):
    """The fp32 (and R = 32) path: per-row maximum and sum first, then the
    block sums against that maximum."""
    H = 1
    nb = 12
    N = nb * C - 10
    Na = max(-(-N // R) * R, nb * C)
    levels = ladder_levels(nb, "first_high")
    bits = ladder_inputs(H, Na, N, d, C, levels, seed=d + R)
    q64, k64 = (S.f64_from_bf16_bits(b) for b in bits[:2])
    M_ref = O.block_mass(q64, k64, N, R, C)
    for dtype in ("f32", "bf16"):
        if dtype == "bf16" and R != 32:
            continue
        qd = to_device(q64.astype(np.float32) if dtype == "f32" else bits[0], dtype)
        kd = to_device(k64.astype(np.float32) if dtype == "f32" else bits[1], dtype)
        Mg = F.losa_block_mass(qd, kd, N, R, C).cpu().numpy().astype(np.float64)
        check_masses_with_floor(Mg, M_ref, f"SIMT {dtype} d={d} R={R} C={C}")
