"""GPU parity of losa_select_threshold -- online block thresholding (Sol-Attn
page: critical blocks picked against a threshold during the online-softmax
pass), read as: in index order, keep block j when its mass is at least
theta times the running maximum.

Max and an fp64 comparison are exact, so the lists must equal the oracle's
bit for bit, with the same per-head work order.  Inputs: random masses with
zeros, NaN, inf and negatives; widths around the 64-block step and the
4096-block maximum; per-head theta; the oracle's exact masses and pooled
proxies of the parity layers; the full Wan2.1-1.3B 480p shape; and sparse
attention on the thresholded lists against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from tests.gpu_util import ATTN_ATOL, layer_to_device, say
from tests.test_gpu_parity import CASES, _case

pytestmark = pytest.mark.gpu

import free_block_sparse_exact_amd as F  # noqa: E402


def _check(M32, theta, N, R, C, what):
    rp_ref, ci_ref = O.select_threshold(M32, theta)
    Na = max(M32.shape[2] * R, M32.shape[3] * C)
    rp, ci, order = F.losa_select_threshold(torch.from_numpy(M32).cuda(), theta, N, R, C, tokens_alloc=Na)
    torch.cuda.synchronize()
    rp = rp.cpu().numpy().astype(np.int64)
    assert np.array_equal(rp, rp_ref), what
    assert np.array_equal(ci[:int(rp[-1])].cpu().numpy(), ci_ref), what
    assert np.array_equal(order.cpu().numpy(), O.budget_order(rp_ref, M32.shape[2])), what
    n = M32.shape[0] * M32.shape[1] * M32.shape[2] * M32.shape[3]
    say(f"{what}: {int(rp[-1])} of {n} blocks kept, bit-exact")
    return rp_ref, ci_ref


def _random_masses(rng, shape):
    kind = rng.integers(0, 4, size=shape[:3] + (1,))
    base = rng.random(shape)
    M = np.where(kind == 0, base ** 8, np.where(kind == 1, np.exp(rng.standard_normal(shape) * 3.0),
                                                 np.where(kind == 2, np.round(base * 4) / 4, base)))
    M = M / M.sum(axis=-1, keepdims=True)
    M = M.astype(np.float32)
    flat = M.reshape(-1)
    idx = rng.choice(flat.size, size=min(flat.size, 40), replace=False)
    flat[idx[:10]] = np.nan
    flat[idx[10:20]] = -flat[idx[10:20]]
    flat[idx[20:25]] = np.inf
    flat[idx[25:]] = 0.0
    return M


@pytest.mark.parametrize("nk,C,R,H", [(1, 64, 64, 3), (2, 64, 64, 3), (63, 64, 64, 3), (64, 64, 64, 3),
                                      (65, 64, 64, 3), (130, 32, 128, 2), (512, 64, 64, 1), (4096, 32, 128, 1)])
def test_threshold_random_masses(nk, C, R, H):
    rng = np.random.default_rng(nk)
    N = nk * C - 5 if nk > 1 else 40
    nq = -(-N // R)
    M = _random_masses(rng, (1, H, nq, nk))
    thetas = (1.0, 0.3, 1e-3, [0.05, 0.5, 0.9][:H] if H > 1 else 0.05)
    for theta in (thetas if nk < 4096 else thetas[1:3]):
        _check(M, theta, N, R, C, f"n_k={nk} theta={theta}")


@pytest.mark.parametrize("name", [c[0] for c in CASES if c[0] != "wl0_f32_d64"])
def test_threshold_on_oracle_masses_and_proxies(name):
    c = _case(name)
    q64, k64 = c["layer"].f64("q"), c["layer"].f64("k")
    _check(c["M32"], 0.02, c["N"], c["R"], c["C"], f"{name} exact masses")
    P32 = O.pooled_mass(q64, k64, c["N"], c["R"], c["C"]).astype(np.float32)
    _check(P32, 0.02, c["N"], c["R"], c["C"], f"{name} pooled proxies")


def test_threshold_fullsize_shape():
    wl = S.get_workload("1")
    nq, nk = wl.n_blocks, wl.n_key_blocks
    rng = np.random.default_rng(77)
    s = rng.standard_normal((1, wl.heads, nq, nk)) * rng.uniform(1.0, 4.0, size=(1, wl.heads, 1, 1))
    M = np.exp(s - s.max(axis=-1, keepdims=True))
    M = (M / M.sum(axis=-1, keepdims=True)).astype(np.float32)
    _check(M, [0.01, 0.05] * (wl.heads // 2), wl.tokens, wl.block, wl.key_block, "Wan2.1-1.3B 480p shape")


def test_threshold_then_sparse_attention():
    c = _case("bf16_d128_r64_ragged")
    rp_ref, ci_ref = _check(c["M32"], 0.05, c["N"], c["R"], c["C"], "lists for attention")
    q, k, v = layer_to_device(c["layer"])
    rp, ci, order = F.losa_select_threshold(torch.from_numpy(c["M32"]).cuda(), 0.05, c["N"], c["R"], c["C"],
                                            tokens_alloc=c["Na"])
    Og = F.losa_sparse_attn(q, k, v, rp, ci, order, c["N"], c["R"], c["C"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    L = c["layer"]
    ref = O.sparse_attention(L.f64("q"), L.f64("k"), L.f64("v"), c["N"], c["R"], c["C"], rp_ref, ci_ref)
    N = c["N"]
    err = float(np.abs(Og.cpu().numpy()[:, :, :N] - ref[:, :, :N]).max())
    say(f"sparse attention on thresholded lists: O max abs err {err:.2e}")
    assert err <= ATTN_ATOL


def test_work_order_many_short_groups():
    """1024 heads of 33 query blocks (a 32-row and a 1-row group each) and
    nine key blocks: 2048 work groups, few distinct counts; the selector's
    lists and its work order against the oracle, bit for bit."""
    rng = np.random.default_rng(99)
    H, R, C, N = 1024, 32, 128, 1049
    nq, nk = -(-N // R), -(-N // C)
    assert (nq, nk) == (33, 9)
    M = rng.random((1, H, nq, nk)).astype(np.float32) ** 3
    rp_ref, ci_ref = O.select_contract(M, 0.7)
    rp, ci, order = F.losa_select(torch.from_numpy(M).cuda(), 0.7, N, R, C, tokens_alloc=max(nq * R, nk * C))
    torch.cuda.synchronize()
    rp = rp.cpu().numpy().astype(np.int64)
    assert np.array_equal(rp, rp_ref)
    assert np.array_equal(ci[:int(rp[-1])].cpu().numpy(), ci_ref)
    assert np.array_equal(order.cpu().numpy(), O.budget_order(rp_ref, nq))
    say(f"{H} heads x {nq} rows: lists and work order bit-exact")
