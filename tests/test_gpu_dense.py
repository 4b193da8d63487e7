"""GPU parity of losa_dense_attn_mass -- dense attention and the exact block
masses in one pass (the construction step) -- against the fp64 oracle.

LoSA page: Methodology Summary (the pattern is constructed once, at a dense
step, from exact block masses); Experiments Summary (the construction step's
kernel is a full attention pass that also sums the exact block masses).  O is checked
against the oracle's dense attention (absolute 1e-2), M against the oracle's
block masses (relative 1e-3), on the small seeded cases of the sparse
parity tests, on rows whose logits all lie far below zero, on rows that drive
the kernel into its exact fallback, and on sampled rows of the full
Wan2.1-1.3B 480p layer.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from tests.gpu_util import ATTN_ATOL, MASS_RTOL, Timer, layer_to_device, mass_rel_err, sample_rows, say, to_device
from tests.test_gpu_parity import IDS, _case, check_masses_with_floor, negative_logit_inputs, score_gap_inputs

pytestmark = pytest.mark.gpu

import free_block_sparse_exact_amd as F  # noqa: E402


def _dense_ref(q64, k64, v64, N, R):
    ref = O.dense_attention(q64, k64, v64, N)
    nqR = -(-N // R) * R
    return ref[:, :, :nqR], nqR


@pytest.mark.parametrize("name", IDS)
def test_dense_attn_mass_small(name):
    c = _case(name)
    L = c["layer"]
    q, k, v = layer_to_device(L)
    Og, Mg = F.losa_dense_attn_mass(q, k, v, c["N"], c["R"], c["C"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    m_err = mass_rel_err(Mg.cpu().numpy(), c["M"])
    ref, nqR = _dense_ref(L.f64("q"), L.f64("k"), L.f64("v"), c["N"], c["R"])
    o_err = float(np.abs(Og.cpu().numpy()[:, :, :nqR] - ref).max())
    say(f"{name}: dense O max abs err {o_err:.2e}; M max rel err {m_err:.2e}")
    assert o_err <= ATTN_ATOL
    assert m_err <= MASS_RTOL


def test_dense_matches_two_calls():
    """Same masses as losa_block_mass (to fp32 rounding-order level), same O as
    sparse attention with every block listed (both are the dense softmax)."""
    c = _case("bf16_d128_r64_ragged")
    q, k, v = layer_to_device(c["layer"])
    N, R, C = c["N"], c["R"], c["C"]
    Od, Md = F.losa_dense_attn_mass(q, k, v, N, R, C, out_dtype=torch.float32)
    M2 = F.losa_block_mass(q, k, N, R, C)
    rp, ci, order = F.losa_select(M2, 1.0, N, R, C, tokens_alloc=c["Na"])
    Os = F.losa_sparse_attn(q, k, v, rp, ci, order, N, R, C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert float(((Md - M2).abs() / M2).max()) <= 1e-5
    nqR = -(-N // R) * R
    assert float((Od[:, :, :nqR] - Os[:, :, :nqR]).abs().max()) <= 1e-2


@pytest.mark.parametrize("N", [1000, 970, 1024])
def test_dense_negative_logits(N):
    """All logits far below zero with padded key tails (N = 970: a wholly padded
    32-key chunk; 1024: no padding)."""
    H, d, R = 2, 128, 64
    Na = -(-N // R) * R
    bits = negative_logit_inputs(np.random.default_rng(N), 225.0, H, Na, d)
    q64, k64, v64 = (S.f64_from_bf16_bits(b) for b in bits)
    qd, kd, vd = (to_device(b, "bf16") for b in bits)
    Og, Mg = F.losa_dense_attn_mass(qd, kd, vd, N, R, R, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, nqR = _dense_ref(q64, k64, v64, N, R)
    o_err = float(np.abs(Og.cpu().numpy()[:, :, :nqR] - ref).max())
    m_err = mass_rel_err(Mg.cpu().numpy(), O.block_mass(q64, k64, N, R, R))
    say(f"dense negative logits N={N}: O err {o_err:.2e}, M rel err {m_err:.2e}")
    assert o_err <= ATTN_ATOL
    assert m_err <= MASS_RTOL


@pytest.mark.parametrize("R", [64, 128])
def test_dense_overflow_fallback(R):
    """Every wave's first chunk lies far below later keys: the exact fallback."""
    H, d, N = 2, 128, 1000
    Na = -(-N // R) * R
    bits = score_gap_inputs(np.random.default_rng(4048 + R), H, Na, d)
    q64, k64, v64 = (S.f64_from_bf16_bits(b) for b in bits)
    qd, kd, vd = (to_device(b, "bf16") for b in bits)
    Og, Mg = F.losa_dense_attn_mass(qd, kd, vd, N, R, R, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_masses_with_floor(Mg.cpu().numpy().astype(np.float64), O.block_mass(q64, k64, N, R, R),
                            f"dense fallback R={R}")
    ref, nqR = _dense_ref(q64, k64, v64, N, R)
    o_err = float(np.abs(Og.cpu().numpy()[:, :, :nqR] - ref).max())
    say(f"dense fallback R={R}: O err {o_err:.2e}")
    assert o_err <= ATTN_ATOL


def test_dense_fullsize_sampled_rows():
    """Wan2.1-1.3B 480p layer: O and M of sampled query blocks against the oracle."""
    wl = S.get_workload("1")
    R, C = wl.block, wl.key_block
    N, H = wl.tokens, wl.heads
    with Timer("generate"):
        layer = S.make_layer(wl)
    q, k, v = layer_to_device(layer)
    with Timer("gpu dense + masses"):
        Og, Mg = F.losa_dense_attn_mass(q, k, v, N, R, C)
        torch.cuda.synchronize()
    nq = wl.n_blocks
    rows = sample_rows(H, nq, seed=301, n_uniform=12)
    worst_m = worst_o = 0.0
    with Timer("oracle rows"):
        by_head = {}
        for (b, h, i) in rows:
            by_head.setdefault(h, []).append(i)
        for h, iis in by_head.items():
            qh, kh, vh = (S.to_f64(getattr(layer, n)[:, h:h + 1], wl.dtype) for n in ("q", "k", "v"))
            Mref = O.block_mass_rows(qh, kh, N, R, C, [(0, 0, i) for i in iis])
            for s_, i in enumerate(iis):
                worst_m = max(worst_m, mass_rel_err(Mg[0, h, i].cpu().numpy(), Mref[s_]))
                r0, r1 = i * R, min((i + 1) * R, N)
                a = O.attention_probs(qh[0, 0, r0:r1], kh[0, 0, :N], O.softmax_scale(wl.head_dim))
                oref = a @ vh[0, 0, :N]
                worst_o = max(worst_o, float(np.abs(Og[0, h, r0:r1].float().cpu().numpy() - oref).max()))
    say(f"dense full size: M max rel err {worst_m:.2e}, O max abs err {worst_o:.2e} on {len(rows)} blocks")
    assert worst_m <= MASS_RTOL
    assert worst_o <= ATTN_ATOL
