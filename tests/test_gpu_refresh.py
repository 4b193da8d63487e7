"""GPU parity of the drift-triggered refresh: losa_qk_drift (per-head relative
drift of Q and K since a reference step, and the heads to refresh) and
losa_merge_lists (refreshed heads' lists replace the frozen ones).

HASTE page, temporal mask reuse (mask prediction skipped while queries and
keys drift little), read as: drift = ||X - X_ref||_F / ||X_ref||_F per head
over the valid tokens, refresh when the Q or the K drift exceeds tau.

Bars: drift within a relative 1e-12 of the fp64 oracle (both sides sum
exact fp64 squares, in different orders; 0, inf and NaN exactly), refresh
flags and merged lists bit-exact, the merged work order equal to the
oracle's.  Cases: bf16 and f32, d = 64 and 128, one token, ragged token
counts, strided and head-interleaved layouts, padding rows holding NaN
(never read), a NaN in a valid token, a zero reference, the full
Wan2.1-1.3B 480p layer along the drift trajectory, and one refresh step
end to end (drift -> masses -> selection -> merge -> sparse attention).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from tests.gpu_util import ATTN_ATOL, Timer, csr_to_device, say, to_device
from tests.test_gpu_sparse_mass import _random_lists

pytestmark = pytest.mark.gpu

import free_block_sparse_exact_amd as F  # noqa: E402

DRIFT_RTOL = 1e-12


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return S.bf16_bits_from_f32(x32) if dtype == "bf16" else x32.astype(np.float32)


def _f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return S.f64_from_bf16_bits(a) if dtype == "bf16" else a.astype(np.float64)


def _check_drift(dg: np.ndarray, dref: np.ndarray, what: str):
    assert dg.shape == dref.shape
    same_special = (np.isnan(dg) == np.isnan(dref)) & (np.isinf(dg) == np.isinf(dref))
    assert np.all(same_special), f"{what}: 0/inf/NaN pattern differs"
    fin = np.isfinite(dref)
    assert np.all(dg[dref == 0] == 0), f"{what}: zero drift"
    err = float(np.max(np.abs(dg[fin] - dref[fin]) / np.maximum(np.abs(dref[fin]), 1e-300))) if fin.any() else 0.0
    say(f"{what}: drift max rel err {err:.1e} over {int(fin.sum())} values")
    assert err <= DRIFT_RTOL


def _tau_between(dref: np.ndarray) -> float:
    """A threshold halfway between two distinct drifts (no drift lies near it)."""
    v = np.unique(dref[np.isfinite(dref)])
    if v.size < 2:
        return float(v[0]) + 1.0 if v.size else 1.0
    i = v.size // 2
    return float(0.5 * (v[i - 1] + v[i]))


def _pair(rng, shape, N, amps, dtype, pad_nan=True):
    """(cur, ref) storage arrays: ref random, cur = ref + amp_h * noise; padding rows NaN."""
    ref32 = (rng.standard_normal(shape) * 1.5).astype(np.float32)
    noise = rng.standard_normal(shape).astype(np.float32)
    cur32 = ref32 + np.asarray(amps, np.float32)[None, :, None, None] * noise
    cur, ref = _store(cur32, dtype), _store(ref32, dtype)
    if pad_nan:
        nan = _store(np.full((1,), np.nan, np.float32), dtype)[0]
        cur[:, :, N:] = nan
        ref[:, :, N:] = nan
    return cur, ref


def _gpu_drift(cur_q, cur_k, ref_q, ref_k, N, tau, dtype, R=64, C=64):
    q, k, qr, kr = (to_device(a, dtype) for a in (cur_q, cur_k, ref_q, ref_k))
    d, f = F.losa_qk_drift(q, k, qr, kr, N, tau, R, C)
    torch.cuda.synchronize()
    return d.cpu().numpy(), f.cpu().numpy()


@pytest.mark.parametrize("B,H,N,Na,d,dtype", [
    (2, 3, 1000, 1024, 128, "bf16"),
    (1, 2, 130, 192, 64, "bf16"),
    (1, 1, 1, 64, 128, "bf16"),
    (2, 2, 777, 832, 128, "f32"),
    (1, 3, 64, 64, 64, "f32"),
    (1, 4, 4159, 4160, 128, "bf16"),
])
def test_drift_matches_oracle(B, H, N, Na, d, dtype):
    rng = np.random.default_rng(N + d + H)
    shape = (B, H, Na, d)
    amps = [0.0, 0.05, 0.4, 1.5][:H]
    cq, rq = _pair(rng, shape, N, amps, dtype)
    ck, rk = _pair(rng, shape, N, amps[::-1], dtype)
    dref = O.qk_drift(*(_f64(a, dtype) for a in (cq, ck, rq, rk)), N)
    tau = _tau_between(dref)
    dg, fg = _gpu_drift(cq, ck, rq, rk, N, tau, dtype)
    _check_drift(dg, dref, f"B={B} H={H} N={N} d={d} {dtype}")
    assert np.array_equal(fg.astype(bool), O.refresh_heads(dref, tau))
    # the same inputs give the same bits
    dg2, _ = _gpu_drift(cq, ck, rq, rk, N, tau, dtype)
    assert np.array_equal(dg.view(np.uint64), dg2.view(np.uint64))


@pytest.mark.parametrize("layout", ["token_stride", "head_interleaved"])
def test_drift_strided(layout):
    rng = np.random.default_rng(7)
    B, H, N, Na, d = 2, 3, 500, 512, 128
    cq, rq = _pair(rng, (B, H, Na, d), N, [0.1, 0.2, 0.3], "bf16")
    ck, rk = _pair(rng, (B, H, Na, d), N, [0.3, 0.0, 0.6], "bf16")
    dref = O.qk_drift(*(_f64(a, "bf16") for a in (cq, ck, rq, rk)), N)

    def view(a):
        t = to_device(a, "bf16")
        if layout == "token_stride":       # token stride 2d: the first half of a wider row
            big = torch.full((B, H, Na, 2 * d), float("nan"), dtype=torch.bfloat16, device="cuda")
            big[..., :d] = t
            return big[..., :d]
        big = torch.empty((B, Na, H, d), dtype=torch.bfloat16, device="cuda")   # [B, N, H, d] storage
        big.copy_(t.permute(0, 2, 1, 3))
        return big.permute(0, 2, 1, 3)

    q, k, qr, kr = (view(a) for a in (cq, ck, rq, rk))
    assert not q.is_contiguous()
    tau = _tau_between(dref)
    dg, fg = F.losa_qk_drift(q, k, qr, kr, N, tau)
    torch.cuda.synchronize()
    _check_drift(dg.cpu().numpy(), dref, layout)
    assert np.array_equal(fg.cpu().numpy().astype(bool), O.refresh_heads(dref, tau))


def test_drift_special_values():
    rng = np.random.default_rng(8)
    B, H, N, Na, d = 1, 4, 100, 128, 64
    ref = S.bf16_bits_from_f32(rng.standard_normal((B, H, Na, d)).astype(np.float32))
    cur = ref.copy()
    zero = np.zeros_like(ref)
    nan = S.bf16_bits_from_f32(np.array([np.nan], np.float32))[0]
    cur_q = cur.copy()
    cur_q[0, 1, 5, 3] = nan                                  # head 1: NaN in a valid token of Q
    ref_k = ref.copy()
    ref_k[0, 2] = zero[0, 2]                                 # head 2: zero K reference, K unchanged -> inf
    cur_k = cur.copy()
    cur_k[0, 3, :N] = S.bf16_bits_from_f32(                  # head 3: K moved, Q unchanged
        S.f64_from_bf16_bits(cur_k[0, 3, :N]).astype(np.float32) * 2.0)
    dref = O.qk_drift(*(S.f64_from_bf16_bits(a) for a in (cur_q, cur_k, ref, ref_k)), N)
    assert dref[0, 0].tolist() == [0.0, 0.0] and np.isnan(dref[0, 1, 0]) and np.isinf(dref[0, 2, 1])
    for tau in (0.5, 2.0):
        dg, fg = _gpu_drift(cur_q, cur_k, ref, ref_k, N, tau, "bf16")
        _check_drift(dg, dref, f"special values, tau {tau}")
        assert np.array_equal(fg.astype(bool), O.refresh_heads(dref, tau))
    # zero everywhere: no drift, no refresh
    dg, fg = _gpu_drift(zero, zero, zero, zero, N, 0.0, "bf16")
    assert np.all(dg == 0) and not fg.any()


def test_drift_fullsize_trajectory():
    """Wan2.1-1.3B 480p layer (12 heads x 32760 tokens x 128): drift of steps
    10, 30 and 49 against the construction step, every head."""
    wl = S.get_workload("4")
    N = wl.tokens
    with Timer("generate base"):
        layer = S.make_layer(wl, keep_f64=True)
    q_r, k_r = S.drift_qk(layer, wl.construct_step)
    qr_d, kr_d = to_device(q_r, wl.dtype), to_device(k_r, wl.dtype)
    qr64, kr64 = S.to_f64(q_r, wl.dtype), S.to_f64(k_r, wl.dtype)
    last = None
    for step in (10, 30, 49):
        q_s, k_s = S.drift_qk(layer, step)
        dg, fg = F.losa_qk_drift(to_device(q_s, wl.dtype), to_device(k_s, wl.dtype), qr_d, kr_d, N, 0.5,
                                 wl.block, wl.key_block)
        torch.cuda.synchronize()
        with Timer("oracle drift"):
            dref = O.qk_drift(S.to_f64(q_s, wl.dtype), S.to_f64(k_s, wl.dtype), qr64, kr64, N)
        _check_drift(dg.cpu().numpy(), dref, f"step {step}")
        assert np.array_equal(fg.cpu().numpy().astype(bool), O.refresh_heads(dref, 0.5))
        if last is not None:
            assert np.all(dref > last)  # the trajectory moves away from the construction step
        last = dref


@pytest.mark.parametrize("B,H,N,R,C,pattern", [
    (1, 2, 1000, 64, 64, [0, 1]),
    (2, 3, 19200, 64, 64, [1, 0, 1, 0, 0, 1]),     # 300 query blocks per head: ragged order chunks
    (1, 4, 1000, 128, 32, [1, 1, 1, 1]),
    (1, 4, 1000, 64, 128, [0, 0, 0, 0]),
    (1, 1, 1, 64, 64, [1]),
])
def test_merge_matches_oracle(B, H, N, R, C, pattern):
    rng = np.random.default_rng(N + H + R)
    n_q, n_k = -(-N // R), -(-N // C)
    rows = B * H * n_q
    rp_a, ci_a = _random_lists(rng, rows, n_k, 0.3)
    rp_b, ci_b = _random_lists(rng, rows, n_k, 0.6)
    take = np.asarray(pattern, np.int32).reshape(B, H)
    rp_ref, ci_ref = O.merge_lists(rp_a, ci_a, rp_b, ci_b, take.astype(bool), n_q)
    a = csr_to_device(rp_a, ci_a)
    b = csr_to_device(rp_b, ci_b)
    rp, ci, order = F.losa_merge_lists(torch.from_numpy(take).cuda(), a[0], a[1], b[0], b[1], N, R, C)
    torch.cuda.synchronize()
    rp = rp.cpu().numpy().astype(np.int64)
    assert np.array_equal(rp, rp_ref)
    assert np.array_equal(ci[:int(rp[-1])].cpu().numpy(), ci_ref)
    assert np.array_equal(order.cpu().numpy(), O.budget_order(rp_ref, n_q))
    say(f"merge B={B} H={H} n_q={n_q} n_k={n_k} take={pattern}: {int(rp[-1])} indices bit-exact")


def test_refresh_step_end_to_end():
    """One drift-triggered refresh: lists built at a reference step; at the
    current step the drifted heads get lists from the current masses, the
    others keep theirs; sparse attention runs on the merged lists."""
    rng = np.random.default_rng(31)
    B, H, N, Na, d, R, C, p = 1, 4, 1000, 1024, 128, 64, 64, 0.95
    amps = [0.0, 0.02, 0.6, 1.2]
    k_ref32 = (rng.standard_normal((B, H, Na, d)) * 1.5).astype(np.float32)
    q_ref32 = (rng.standard_normal((B, H, Na, d)) * 1.5).astype(np.float32)
    v32 = rng.standard_normal((B, H, Na, d)).astype(np.float32)
    a4 = np.asarray(amps, np.float32)[None, :, None, None]
    q_cur32 = q_ref32 + a4 * rng.standard_normal((B, H, Na, d)).astype(np.float32)
    k_cur32 = k_ref32 + a4 * rng.standard_normal((B, H, Na, d)).astype(np.float32)
    bits = {n: S.bf16_bits_from_f32(x) for n, x in
            (("qr", q_ref32), ("kr", k_ref32), ("q", q_cur32), ("k", k_cur32), ("v", v32))}
    for x in bits.values():
        x[:, :, N:] = 0
    f64 = {n: S.f64_from_bf16_bits(x) for n, x in bits.items()}
    dev = {n: to_device(x, "bf16") for n, x in bits.items()}
    tau = 0.1
    # oracle: lists at the reference step, drift, lists at the current step, merge
    M_r = O.block_mass(f64["qr"], f64["kr"], N, R, C).astype(np.float32)
    M_c = O.block_mass(f64["q"], f64["k"], N, R, C).astype(np.float32)
    rp_r, ci_r = O.select_contract(M_r, p)
    rp_c, ci_c = O.select_contract(M_c, p)
    dref = O.qk_drift(f64["q"], f64["k"], f64["qr"], f64["kr"], N)
    flags = O.refresh_heads(dref, tau)
    assert flags.tolist() == [[False, False, True, True]]
    rp_m, ci_m = O.merge_lists(rp_r, ci_r, rp_c, ci_c, flags, -(-N // R))
    # GPU: the same steps through the library (both selectors read the oracle's fp32 masses)
    rpa, cia, _ = F.losa_select(torch.from_numpy(M_r).cuda(), p, N, R, C, tokens_alloc=Na, want_order=False)
    dg, fg = F.losa_qk_drift(dev["q"], dev["k"], dev["qr"], dev["kr"], N, tau, R, C)
    rpb, cib, _ = F.losa_select(torch.from_numpy(M_c).cuda(), p, N, R, C, tokens_alloc=Na, want_order=False)
    rp, ci, order = F.losa_merge_lists(fg, rpa, cia, rpb, cib, N, R, C, tokens_alloc=Na)
    Og = F.losa_sparse_attn(dev["q"], dev["k"], dev["v"], rp, ci, order, N, R, C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    _check_drift(dg.cpu().numpy(), dref, "end to end")
    assert np.array_equal(fg.cpu().numpy().astype(bool), flags)
    rp_h = rp.cpu().numpy().astype(np.int64)
    assert np.array_equal(rp_h, rp_m) and np.array_equal(ci[:int(rp_h[-1])].cpu().numpy(), ci_m)
    ref = O.sparse_attention(f64["q"], f64["k"], f64["v"], N, R, C, rp_m, ci_m)
    err = float(np.abs(Og.cpu().numpy()[:, :, :N] - ref[:, :, :N]).max())
    say(f"refresh step: heads {np.flatnonzero(flags[0]).tolist()} rebuilt, O max abs err {err:.2e}")
    assert err <= ATTN_ATOL
