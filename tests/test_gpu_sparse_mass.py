"""GPU parity of losa_sparse_attn_mass -- frozen-pattern sparse attention that
also returns the exact block masses within each row's lists -- against the
fp64 oracle.

GSRS card (reduced search: later top-p searches restricted to an early
candidate set, with exact attention weights computed inside the attention
pass).  O is checked against the oracle's sparse attention (absolute 1e-2),
M against the oracle's masses within the lists (relative 1e-3 on listed
blocks; exactly 0 elsewhere), on the small seeded cases with the oracle's
lists, on random lists (empty rows, rows with and without the padded last
block, every block listed), with and without a work order, on the exact
fallback, and on sampled rows of the full Wan2.1-1.3B 480p layer.  The
reduced search itself (losa_select on these masses) must keep a subset of
each row's candidates.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from tests.gpu_util import (ATTN_ATOL, MASS_RTOL, Timer, csr_to_device, layer_to_device, row_csr, sample_rows,
                            say, to_device)
from tests.test_gpu_parity import IDS, _case, score_gap_inputs

pytestmark = pytest.mark.gpu

import free_block_sparse_exact_amd as F  # noqa: E402

MATRIX_CORE = [n for n in IDS if not (n.startswith("wl0") or n.startswith("f32") or "simt" in n)]


def check_masses(Mg: np.ndarray, Mref: np.ndarray, rp: np.ndarray, ci: np.ndarray, what: str):
    """Listed entries within MASS_RTOL of the oracle, the rest exactly 0."""
    rows, n_k = Mref.reshape(-1, Mref.shape[-1]).shape
    Mg = Mg.reshape(rows, n_k).astype(np.float64)
    Mref = Mref.reshape(rows, n_k)
    listed = np.zeros((rows, n_k), bool)
    for r in range(rows):
        listed[r, row_csr(rp, ci, r)] = True
    assert np.all(Mg[~listed] == 0.0), f"{what}: mass outside the lists"
    ref = Mref[listed]
    assert np.all(ref > 0), "reference mass underflowed to 0"
    err = float(np.max(np.abs(Mg[listed] - ref) / ref)) if ref.size else 0.0
    say(f"{what}: M max rel err {err:.2e} over {ref.size} listed blocks")
    assert err <= MASS_RTOL


def run(layer_or_bits, N, R, C, rp, ci, order=None, Na=None):
    if isinstance(layer_or_bits, (tuple, list)):
        q, k, v = (to_device(b, "bf16") for b in layer_or_bits)
    else:
        q, k, v = layer_to_device(layer_or_bits)
    rpd, cid = csr_to_device(rp, ci)
    od = None if order is None else torch.from_numpy(np.asarray(order, np.int32)).cuda()
    Og, Mg = F.losa_sparse_attn_mass(q, k, v, rpd, cid, od, N, R, C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    return Og.cpu().numpy(), Mg.cpu().numpy()


@pytest.mark.parametrize("name", MATRIX_CORE)
def test_sparse_mass_on_oracle_lists(name):
    c = _case(name)
    L = c["layer"]
    q64, k64, v64 = L.f64("q"), L.f64("k"), L.f64("v")
    Og, Mg = run(L, c["N"], c["R"], c["C"], c["rp"], c["ci"], c["order"])
    nqR = -(-c["N"] // c["R"]) * c["R"]
    o_err = float(np.abs(Og[:, :, :nqR] - c["O"][:, :, :nqR]).max())
    say(f"{name}: O max abs err {o_err:.2e}")
    assert o_err <= ATTN_ATOL
    check_masses(Mg, O.restricted_mass(q64, k64, c["N"], c["R"], c["C"], c["rp"], c["ci"]), c["rp"], c["ci"], name)


def _random_lists(rng, rows, n_k, keep):
    rp, cols = [0], []
    for r in range(rows):
        kind = r % 5
        if kind == 0:
            sel = np.zeros(0, np.int64)                       # empty row
        elif kind == 1:
            sel = np.arange(n_k)                              # every block
        elif kind == 2:
            sel = np.flatnonzero(rng.random(n_k) < keep)
            sel = sel[sel != n_k - 1]                         # without the padded last block
        else:
            sel = np.flatnonzero(rng.random(n_k) < keep)
            sel = np.union1d(sel, [n_k - 1])                  # with it
        if kind == 4:
            sel = rng.permutation(sel)                        # any order is accepted
        cols.append(sel)
        rp.append(rp[-1] + sel.size)
    return np.asarray(rp, np.int64), np.concatenate(cols).astype(np.int32)


@pytest.mark.parametrize("N,R,C,use_order", [(1000, 64, 64, True), (1000, 128, 32, False), (970, 64, 32, True),
                                             (1024, 128, 128, True), (777, 64, 128, False)])
def test_sparse_mass_random_lists(N, R, C, use_order):
    wl = S.get_workload("1")
    layer = S.make_layer(wl, tokens=N, n_heads=2)
    Na = max(-(-N // R) * R, -(-N // C) * C)

    def pad(a):
        out = np.zeros(a.shape[:2] + (Na, a.shape[3]), a.dtype)
        out[:, :, :N] = a[:, :, :N]
        return out
    layer.q, layer.k, layer.v = pad(layer.q), pad(layer.k), pad(layer.v)
    n_q, n_k = -(-N // R), -(-N // C)
    rp, ci = _random_lists(np.random.default_rng(N + R + C), 2 * n_q, n_k, 0.5)
    order = O.budget_order(rp, n_q) if use_order else None
    q64, k64, v64 = layer.f64("q"), layer.f64("k"), layer.f64("v")
    Og, Mg = run(layer, N, R, C, rp, ci, order)
    ref = O.sparse_attention(q64, k64, v64, N, R, C, rp, ci)
    nqR = n_q * R
    o_err = float(np.abs(Og[:, :, :nqR] - ref[:, :, :nqR]).max())
    say(f"random lists N={N} R={R} C={C}: O max abs err {o_err:.2e}")
    assert o_err <= ATTN_ATOL
    check_masses(Mg, O.restricted_mass(q64, k64, N, R, C, rp, ci), rp, ci, f"random lists N={N} R={R} C={C}")


def test_every_block_listed_equals_the_construction_call():
    """Every block listed: the masses are losa_dense_attn_mass's (fp32 rounding-order level)."""
    c = _case("bf16_d128_r64_ragged")
    N, R, C = c["N"], c["R"], c["C"]
    q, k, v = layer_to_device(c["layer"])
    n_q, n_k = -(-N // R), -(-N // C)
    rows = 2 * n_q
    rp = np.arange(rows + 1) * n_k
    ci = np.tile(np.arange(n_k, dtype=np.int32), rows)
    rpd, cid = csr_to_device(rp, ci)
    Os, Ms = F.losa_sparse_attn_mass(q, k, v, rpd, cid, None, N, R, C, out_dtype=torch.float32)
    Od, Md = F.losa_dense_attn_mass(q, k, v, N, R, C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert float(((Ms - Md).abs() / Md).max()) <= 1e-5
    assert float((Os[:, :, :n_q * R] - Od[:, :, :n_q * R]).abs().max()) <= 1e-3


def test_sparse_mass_fallback():
    """Every wave's first chunk lies far below later keys: the exact two-pass path."""
    H, d, N, R = 2, 128, 1000, 64
    Na = -(-N // R) * R
    bits = score_gap_inputs(np.random.default_rng(4101), H, Na, d)
    q64, k64, v64 = (S.f64_from_bf16_bits(b) for b in bits)
    n_q = n_k = -(-N // R)
    rp, ci = _random_lists(np.random.default_rng(5), H * n_q, n_k, 0.6)
    Og, Mg = run(bits, N, R, R, rp, ci)
    ref = O.sparse_attention(q64, k64, v64, N, R, R, rp, ci)
    o_err = float(np.abs(Og[:, :, :n_q * R] - ref[:, :, :n_q * R]).max())
    say(f"fallback: O max abs err {o_err:.2e}")
    assert o_err <= ATTN_ATOL
    Mref = O.restricted_mass(q64, k64, N, R, R, rp, ci)
    # masses of blocks far below the row maximum fall under fp32 resolution; compare those with an absolute floor
    Mg2 = Mg.reshape(-1, n_k).astype(np.float64)
    Mr2 = Mref.reshape(-1, n_k)
    assert np.all(np.abs(Mg2 - Mr2) <= MASS_RTOL * Mr2 + 1e-7)


def test_reduced_search_keeps_a_subset():
    """Config-1 shapes on two heads: lists at p = 0.995 from the GPU masses, then
    the masses within them and a reduced search at p' = 0.9 -- every new list
    lies inside its candidate list, and matches the oracle's reduced search
    wherever both read the same fp32 masses."""
    wl = S.get_workload("1")
    N, R, C = 4096, 64, 64
    layer = S.make_layer(wl, tokens=N, n_heads=2)
    q, k, v = layer_to_device(layer)
    M = F.losa_block_mass(q, k, N, R, C)
    rp, ci, order = F.losa_select(M, 0.995, N, R, C, tokens_alloc=layer.q.shape[2])
    _, ML = F.losa_sparse_attn_mass(q, k, v, rp, ci, order, N, R, C)
    rp2, ci2, _ = F.losa_select(ML, 0.9, N, R, C, tokens_alloc=layer.q.shape[2])
    torch.cuda.synchronize()
    rp_h, ci_h = rp.cpu().numpy().astype(np.int64), ci.cpu().numpy()
    rp2_h, ci2_h = rp2.cpu().numpy().astype(np.int64), ci2.cpu().numpy()
    rows = len(rp_h) - 1
    for r in range(rows):
        assert set(row_csr(rp2_h, ci2_h, r)) <= set(row_csr(rp_h, ci_h, r))
    ref_rp, ref_ci = O.select_contract(ML.cpu().numpy(), 0.9)
    assert np.array_equal(rp2_h, ref_rp) and np.array_equal(ci2_h[:int(rp2_h[-1])], ref_ci)
    kept = (rp2_h[-1]) / max(1, rp_h[-1])
    say(f"reduced search: {rp2_h[-1]} of {rp_h[-1]} candidate blocks kept ({kept:.3f})")


def test_sparse_mass_fullsize_sampled_rows():
    """Wan2.1-1.3B 480p layer with its p = 0.99 lists: O and the masses within
    the lists of sampled query blocks against the oracle."""
    wl = S.get_workload("1")
    R, C, N, H = wl.block, wl.key_block, wl.tokens, wl.heads
    with Timer("generate"):
        layer = S.make_layer(wl)
    q, k, v = layer_to_device(layer)
    with Timer("gpu masses, lists, sparse attention with masses"):
        M = F.losa_block_mass(q, k, N, R, C)
        rp, ci, order = F.losa_select(M, wl.p, N, R, C, tokens_alloc=wl.tokens_alloc)
        Og, Mg = F.losa_sparse_attn_mass(q, k, v, rp, ci, order, N, R, C)
        torch.cuda.synchronize()
    rp_h, ci_h = rp.cpu().numpy().astype(np.int64), ci.cpu().numpy()
    nq = wl.n_blocks
    rows = sample_rows(H, nq, seed=401, n_uniform=10)
    worst_m = worst_o = 0.0
    with Timer("oracle rows"):
        for (b, h, i) in rows:
            qh, kh, vh = (S.to_f64(getattr(layer, n)[:, h:h + 1], wl.dtype) for n in ("q", "k", "v"))
            # this head's CSR on its own (one head: row = i)
            rp_head = rp_h[h * nq:(h + 1) * nq + 1] - rp_h[h * nq]
            ci_head = ci_h[rp_h[h * nq]:rp_h[(h + 1) * nq]]
            lst = row_csr(rp_head, ci_head, i)
            Mref = O.restricted_mass_rows(qh, kh, N, R, C, rp_head, ci_head, [(0, 0, i)])
            mg = Mg[0, h, i].cpu().numpy().astype(np.float64)
            assert np.all(mg[np.setdiff1d(np.arange(wl.n_key_blocks), lst)] == 0.0)
            ref = Mref[0][lst]
            worst_m = max(worst_m, float(np.max(np.abs(mg[lst] - ref) / ref)))
            oref = O.sparse_attention_rows(qh, kh, vh, N, R, C, rp_head, ci_head, [(0, 0, i)])[0]
            r0 = i * R
            worst_o = max(worst_o, float(np.abs(Og[0, h, r0:r0 + oref.shape[0]].float().cpu().numpy() - oref).max()))
    say(f"full size: M max rel err {worst_m:.2e}, O max abs err {worst_o:.2e} on {len(rows)} blocks")
    assert worst_m <= MASS_RTOL
    assert worst_o <= ATTN_ATOL
