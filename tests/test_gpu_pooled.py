"""GPU parity of losa_pooled_mass (pooled proxy masses, the coarse estimate
the LoSA page contrasts with exact masses -- Motivation Summary) against the
fp64 oracle, and of the lists the same selector builds from them.

Reading (the pages give no formula): P[i, j] = |B_j| exp(qbar_i . kbar_j *
scale) / sum_j' |B_j'| exp(qbar_i . kbar_j' * scale) over block means.
Tolerance as for the exact masses: relative 1e-3 (below fp32's normal range,
2^-126 absolute).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from tests.gpu_util import Timer, layer_to_device, row_csr, say, to_device
from tests.test_gpu_parity import IDS, _case, check_masses_with_floor

pytestmark = pytest.mark.gpu

import free_block_sparse_exact_amd as F  # noqa: E402


@pytest.mark.parametrize("name", IDS)
def test_pooled_small_cases(name):
    c = _case(name)
    L = c["layer"]
    q, k, _ = layer_to_device(L)
    Pg = F.losa_pooled_mass(q, k, c["N"], c["R"], c["C"]).cpu().numpy().astype(np.float64)
    Pref = O.pooled_mass(L.f64("q"), L.f64("k"), c["N"], c["R"], c["C"])
    check_masses_with_floor(Pg, Pref, f"pooled {name}")
    # the selector on the GPU's P, against the oracle's selection on the oracle's P
    rp, ci, _ = F.losa_select(torch.from_numpy(Pg.astype(np.float32)).cuda(), c["p"], c["N"], c["R"], c["C"],
                              tokens_alloc=c["Na"])
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci[:int(rp_h[-1])].cpu().numpy()
    rp_ref, ci_ref = O.select_contract(Pref.astype(np.float32), c["p"])
    rows = len(rp_ref) - 1
    n_diff = sum(not np.array_equal(row_csr(rp_h, ci_h, r), row_csr(rp_ref, ci_ref, r)) for r in range(rows))
    say(f"pooled {name}: {n_diff} of {rows} lists differ from the oracle's")
    assert n_diff <= max(1, rows // 20)


def test_pooled_equals_exact_masses_on_gpu_for_blockwise_constant_inputs():
    """Q constant within query blocks, K within key blocks (ragged tail, R != C):
    the GPU's proxy and the GPU's exact masses agree."""
    rng = np.random.default_rng(9)
    H, d, N, R, C = 2, 128, 1000, 64, 32
    Na = 1024
    q = rng.standard_normal((1, H, Na, d))
    k = rng.standard_normal((1, H, Na, d))
    for i in range(-(-N // R)):
        q[:, :, i * R:min((i + 1) * R, N)] = rng.standard_normal((1, H, 1, d)) * 0.3
    for j in range(-(-N // C)):
        k[:, :, j * C:min((j + 1) * C, N)] = rng.standard_normal((1, H, 1, d)) * 0.3
    qd = to_device(S.bf16_bits_from_f32(q.astype(np.float32)), "bf16")
    kd = to_device(S.bf16_bits_from_f32(k.astype(np.float32)), "bf16")
    P = F.losa_pooled_mass(qd, kd, N, R, C)
    M = F.losa_block_mass(qd, kd, N, R, C)
    torch.cuda.synchronize()
    rel = float(((P - M).abs() / M).max())
    say(f"pooled vs exact on block-constant inputs: max rel diff {rel:.2e}")
    assert rel <= 1e-4


def test_pooled_full_layer():
    """Wan2.1-1.3B 480p layer: every row of P against the oracle."""
    wl = S.get_workload("1")
    R, C = wl.block, wl.key_block
    with Timer("generate"):
        layer = S.make_layer(wl)
    q, k, _ = layer_to_device(layer)
    with Timer("gpu pooled"):
        Pg = F.losa_pooled_mass(q, k, wl.tokens, R, C).cpu().numpy().astype(np.float64)
    with Timer("oracle pooled"):
        Pref = O.pooled_mass(layer.f64("q"), layer.f64("k"), wl.tokens, R, C)
    check_masses_with_floor(Pg, Pref, "pooled full layer")
