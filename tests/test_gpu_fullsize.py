"""GPU parity at the full layer sizes (Wan2.1-1.3B 480p, Wan2.1-14B 720p,
HunyuanVideo 720p shapes), in the launch configuration the benchmark times:
GPU masses -> GPU selection -> GPU sparse attention on the GPU's own lists.

The fp64 oracle cannot compute every row at these sizes, so a seeded sample
of rows is checked one by one (the last, partial query block of every head,
the first block, and uniform rows):
  * masses of the sampled rows against the oracle (relative 1e-3);
  * the oracle's lists for those rows (from the oracle's masses) against the
    GPU's lists; a row may differ only where the oracle's cut lies within the
    masses' fp32 resolution;
  * O of the sampled rows against the oracle's sparse attention on the
    oracle's lists, wherever the GPU's list equals the oracle's (absolute 1e-2).
The selector's bit-exactness at full shape is checked separately on seeded
synthetic masses of the full [B, H, n_q, n_k] shape.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from tests.gpu_util import ATTN_ATOL, MASS_RTOL, Timer, layer_to_device, mass_rel_err, row_csr, sample_rows, say

pytestmark = pytest.mark.gpu

import free_block_sparse_exact_amd as F  # noqa: E402


def _head_f64(arr, dtype, b, h):
    return S.to_f64(arr[b:b + 1, h:h + 1], dtype)


@pytest.mark.parametrize("wid", ["1", "2", "3", "3n"])
def test_fullsize_pipeline_sampled_rows(wid):
    wl = S.get_workload(wid)
    R, C = wl.block, wl.key_block
    N, Na, H = wl.tokens, wl.tokens_alloc, wl.heads
    say(f"workload {wid} ({wl.name}): H={H} N={N} R={R} C={C}")
    with Timer("generate"):
        layer = S.make_layer(wl)
    q, k, v = layer_to_device(layer)
    with Timer("gpu pipeline"):
        M = F.losa_block_mass(q, k, N, R, C)
        rp, ci, order = F.losa_select(M, wl.p, N, R, C, tokens_alloc=Na)
        Og = F.losa_sparse_attn(q, k, v, rp, ci, order, N, R, C)
        torch.cuda.synchronize()
    nq = wl.n_blocks
    nk = wl.n_key_blocks
    rows = sample_rows(H, nq, seed=100 + wl.seed, n_uniform=24)
    ridx = [O.row_id(b, h, i, H, nq) for (b, h, i) in rows]
    M_rows = M.view(-1, M.shape[-1])[torch.tensor(ridx, device="cuda")].cpu().numpy()
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci[:int(rp_h[-1])].cpu().numpy()
    order_h = order.cpu().numpy()
    # the work order is a permutation: each head's rows in its own range, by
    # count descending, equal counts by row index
    cnt = np.diff(rp_h)
    assert np.array_equal(np.sort(order_h), np.arange(len(cnt)))
    assert np.array_equal(order_h, O.budget_order(rp_h, nq))
    say(f"  nnz={int(rp_h[-1])} coverage={rp_h[-1] / (len(cnt) * nk):.4f} budgets {cnt.min()}..{cnt.max()}")

    by_head = {}
    for t, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append((t, i))
    worst_m, worst_o, n_diff, n_cmp = 0.0, 0.0, 0, 0
    with Timer("oracle rows"):
        for (b, h), items in by_head.items():
            qh, kh, vh = (_head_f64(getattr(layer, n), wl.dtype, b, h) for n in ("q", "k", "v"))
            sub = [(0, 0, i) for (_, i) in items]
            Mref = O.block_mass_rows(qh, kh, N, R, C, sub)
            # lists of these rows from the oracle's masses (fp32, as the ABI carries them)
            lists = [O.select_contract_row(Mref[s].astype(np.float32), wl.p)[0] for s in range(len(sub))]
            for s, (t, i) in enumerate(items):
                worst_m = max(worst_m, mass_rel_err(M_rows[t], Mref[s]))
                r = ridx[t]
                g_list = row_csr(rp_h, ci_h, r)
                if not np.array_equal(g_list, lists[s]):
                    n_diff += 1
                    continue
                n_cmp += 1
                r0, r1 = i * R, min((i + 1) * R, N)
                keys = np.concatenate([np.arange(j * C, min((j + 1) * C, N)) for j in lists[s]])
                a = O.attention_probs(qh[0, 0, r0:r1], kh[0, 0, keys], O.softmax_scale(wl.head_dim))
                oref = a @ vh[0, 0, keys]
                og = Og[b, h, r0:r1].float().cpu().numpy()
                worst_o = max(worst_o, float(np.abs(og - oref).max()))
    say(f"  mass max rel err {worst_m:.3e}; O max abs err {worst_o:.3e} on {n_cmp} rows; "
        f"{n_diff} of {len(rows)} sampled rows have different lists")
    assert worst_m <= MASS_RTOL
    assert worst_o <= ATTN_ATOL
    assert n_cmp >= len(rows) - max(1, len(rows) // 20)


def _synthetic_masses(rng, shape):
    """Seeded mass rows of a given shape: softmax-like rows with a spread of concentration,
    plus adversarial rows (ties, zeros, one-hot, denormals, non-finite)."""
    B, H, nq, nk = shape
    rows = B * H * nq
    conc = rng.uniform(0.05, 3.0, size=(rows, 1))
    M = rng.gamma(conc, size=(rows, nk))
    M /= M.sum(axis=1, keepdims=True)
    M = M.astype(np.float32)
    adv = rng.choice(rows, size=min(rows, 64), replace=False)
    for t, r in enumerate(adv):
        kind = t % 8
        if kind == 0:
            M[r] = np.float32(1.0 / nk)
        elif kind == 1:
            M[r] = 0
        elif kind == 2:
            M[r] = 0
            M[r, rng.integers(nk)] = 1
        elif kind == 3:
            M[r] = np.float32(1e-40) * rng.integers(1, 4, nk).astype(np.float32)
        elif kind == 4:
            M[r, rng.integers(nk, size=3)] = [np.nan, np.inf, -1.0]
        elif kind == 5:
            M[r] = np.round(M[r] * 8, 0) / 8  # many exact ties
        elif kind == 6:
            M[r] = -0.0
            M[r, :2] = 0.5
        else:
            M[r] = np.float32(2.0) ** -rng.integers(1, 40, nk).astype(np.float32)
    return M.reshape(shape)


@pytest.mark.parametrize("wid", ["1", "2", "3", "4", "3n"])
def test_select_bit_exact_full_shape(wid):
    wl = S.get_workload(wid)
    R, C = wl.block, wl.key_block
    nq, nk = wl.n_blocks, wl.n_key_blocks
    shape = (1, wl.heads, nq, nk)
    rng = np.random.default_rng(200 + wl.seed + (50 if wl.k_block else 0))
    M = _synthetic_masses(rng, shape)
    p = wl.p
    if wl.per_head_p:
        p = list(rng.choice(np.asarray(wl.per_head_p), size=wl.heads))
    say(f"workload {wid}: select on synthetic masses {shape}, p={p if np.isscalar(p) else 'per head'}")
    with Timer("oracle select"):
        rp_ref, ci_ref = O.select_contract(M, p)
    Md = torch.from_numpy(M).cuda()
    rp, ci, order = F.losa_select(Md, p, wl.tokens, R, C, tokens_alloc=wl.tokens_alloc)
    torch.cuda.synchronize()
    rp = rp.cpu().numpy().astype(np.int64)
    assert np.array_equal(rp, rp_ref)
    assert np.array_equal(ci[:int(rp[-1])].cpu().numpy(), ci_ref)
    assert np.array_equal(order.cpu().numpy(), O.budget_order(rp_ref, M.shape[2]))


@pytest.mark.parametrize("nk", [1, 2, 63, 64, 65, 127, 129, 200, 400, 500, 600, 800, 900, 1000, 1200, 1217, 1400, 1550,
                                1700, 1800, 1984, 2047, 2048, 2500, 3200, 3500])
def test_select_widths_and_ties(nk):
    """Row widths around multiples of the 64-lane step, at least one width in
    every instance of the one-wave cut (odd runs of 1 .. 31 blocks per lane:
    up to 1984 blocks) and of the workgroup-per-row cut (runs of 9 .. 17 per
    thread: 1985 .. 4096 blocks; 4096 itself in test_maximum_key_block_count,
    3713 in the full-shape tests); most rows adversarial (equal masses, exact
    ties, zeros, one-hot, denormals, non-finite): lists and order bit-exact
    for several p, ties cut in index order."""
    rng = np.random.default_rng(300 + nk)
    C, R = 32, 128
    N = nk * C - 3 if nk > 1 else 20
    nq = -(-N // R)
    M = _synthetic_masses(rng, (1, 2, nq, nk))
    for p in (0.5, 0.9, 0.99, 0.999):
        rp_ref, ci_ref = O.select_contract(M, p)
        rp, ci, order = F.losa_select(torch.from_numpy(M).cuda(), p, N, R, C, tokens_alloc=max(nq * R, nk * C))
        torch.cuda.synchronize()
        rp = rp.cpu().numpy().astype(np.int64)
        assert np.array_equal(rp, rp_ref), (nk, p)
        assert np.array_equal(ci[:int(rp[-1])].cpu().numpy(), ci_ref), (nk, p)
        assert np.array_equal(order.cpu().numpy(), O.budget_order(rp_ref, nq)), (nk, p)
    say(f"n_k={nk}: lists bit-exact for p in 0.5 .. 0.999")


def test_maximum_key_block_count():
    """n_k = 4096 (the largest the ABI accepts): one head of 131072 tokens with
    128-token query and 32-token key blocks through masses, selection and
    sparse attention; sampled rows against the oracle, and the selector
    bit-exact on synthetic masses of the full [1, 1, 1024, 4096] shape."""
    wl = S.Workload("max", "max_key_blocks", 1, 128, (32, 64, 64), 128, "bf16", 0.99, seed=12, k_block=32)
    R, C = wl.block, wl.key_block
    N, Na = wl.tokens, wl.tokens_alloc
    assert wl.n_key_blocks == 4096
    with Timer("generate"):
        layer = S.make_layer(wl)
    q, k, v = layer_to_device(layer)
    M = F.losa_block_mass(q, k, N, R, C)
    rp, ci, order = F.losa_select(M, wl.p, N, R, C, tokens_alloc=Na)
    Og = F.losa_sparse_attn(q, k, v, rp, ci, order, N, R, C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci[:int(rp_h[-1])].cpu().numpy()
    qh, kh, vh = (_head_f64(getattr(layer, n), wl.dtype, 0, 0) for n in ("q", "k", "v"))
    iis = [0, 511, 1023] + list(np.random.default_rng(12).choice(1023, 5, replace=False))
    Mref = O.block_mass_rows(qh, kh, N, R, C, [(0, 0, i) for i in iis])
    Mg = M[0, 0].cpu().numpy()
    worst_m = max(mass_rel_err(Mg[i], Mref[s_]) for s_, i in enumerate(iis))
    worst_o, n_cmp = 0.0, 0
    for s_, i in enumerate(iis):
        lst = O.select_contract_row(Mref[s_].astype(np.float32), wl.p)[0]
        if not np.array_equal(lst, row_csr(rp_h, ci_h, i)):
            continue
        n_cmp += 1
        keys = np.concatenate([np.arange(j * C, min((j + 1) * C, N)) for j in lst])
        r0, r1 = i * R, min((i + 1) * R, N)
        a = O.attention_probs(qh[0, 0, r0:r1], kh[0, 0, keys], O.softmax_scale(wl.head_dim))
        worst_o = max(worst_o, float(np.abs(Og[0, 0, r0:r1].cpu().numpy() - a @ vh[0, 0, keys]).max()))
    say(f"n_k = 4096: mass rel err {worst_m:.2e}; O err {worst_o:.2e} on {n_cmp} of {len(iis)} rows")
    assert worst_m <= MASS_RTOL
    assert worst_o <= ATTN_ATOL
    assert n_cmp >= len(iis) - 1
    # the selector at the full width, bit-exact
    Msyn = _synthetic_masses(np.random.default_rng(13), (1, 1, 1024, 4096))
    rp2, ci2, order2 = F.losa_select(torch.from_numpy(Msyn).cuda(), wl.p, N, R, C, tokens_alloc=Na)
    torch.cuda.synchronize()
    rp_ref, ci_ref = O.select_contract(Msyn, wl.p)
    rp2 = rp2.cpu().numpy().astype(np.int64)
    assert np.array_equal(rp2, rp_ref)
    assert np.array_equal(ci2[:int(rp2[-1])].cpu().numpy(), ci_ref)
    assert np.array_equal(order2.cpu().numpy(), O.budget_order(rp_ref, Msyn.shape[2]))
