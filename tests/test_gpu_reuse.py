"""Frozen-pattern reuse across denoising steps with per-head p (Wan2.1-1.3B 480p
layer shape, 50 steps, Q/K drift).

LoSA page: Methodology Summary -- the pattern is constructed once, from exact
masses at one dense step, and only the block indices are frozen; Q/K/V are
recomputed every later step.  Motivation Summary -- Recall of a pattern under
the dense masses of a later step.  Per-head thresholds follow the head-wise
top-p page (HASTE).  Construction here happens at step 2 of 50; the other
steps run sparse attention on the frozen lists.

Checked on sampled rows against the fp64 oracle: the construction-step lists
(oracle masses -> oracle selection), O at several steps (oracle sparse
attention on the oracle's lists), and the per-step recall of the frozen lists
under GPU masses against the same recall under oracle masses.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from tests.gpu_util import ATTN_ATOL, MASS_RTOL, Timer, mass_rel_err, row_csr, sample_rows, say, to_device

pytestmark = pytest.mark.gpu

import free_block_sparse_exact_amd as F  # noqa: E402


def test_frozen_reuse_per_head_p():
    wl = S.get_workload("4")
    R = C = wl.block
    N, Na, H, d = wl.tokens, wl.tokens_alloc, wl.heads, wl.head_dim
    nq = wl.n_blocks
    with Timer("generate base"):
        layer = S.make_layer(wl, keep_f64=True)
    p_heads = [float(x) for x in layer.p_heads]
    say(f"workload 4: per-head p {p_heads}")
    v = to_device(layer.v, wl.dtype)
    vh64 = {}
    rows = sample_rows(H, nq, seed=104, n_uniform=20)
    ridx = [O.row_id(b, h, i, H, nq) for (b, h, i) in rows]

    def head_rows(q_store, k_store):
        """oracle masses of the sampled rows, grouped by head"""
        out = {}
        for (b, h, i) in rows:
            out.setdefault(h, []).append(i)
        res = {}
        for h, iis in out.items():
            qh = S.to_f64(q_store[:, h:h + 1], wl.dtype)
            kh = S.to_f64(k_store[:, h:h + 1], wl.dtype)
            res[h] = (qh, kh, iis, O.block_mass_rows(qh, kh, N, R, C, [(0, 0, i) for i in iis]))
        return res

    # ---- construction at step 2
    q2, k2 = S.drift_qk(layer, wl.construct_step)
    q2d, k2d = to_device(q2, wl.dtype), to_device(k2, wl.dtype)
    M2 = F.losa_block_mass(q2d, k2d, N, R, C)
    rp, ci, order = F.losa_select(M2, p_heads, N, R, C, tokens_alloc=Na)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci[:int(rp_h[-1])].cpu().numpy()
    counts = np.diff(rp_h)
    per_head = counts.reshape(H, nq).sum(axis=1)
    say(f"  construction: nnz {rp_h[-1]}, per-head kept blocks {per_head.tolist()}")
    with Timer("oracle construction rows"):
        ref2 = head_rows(q2, k2)
    M2_rows = M2.view(-1, nq).cpu().numpy()
    oracle_lists = {}
    n_diff = 0
    worst_m = 0.0
    for h, (_, _, iis, Mref) in ref2.items():
        for s_, i in enumerate(iis):
            r = O.row_id(0, h, i, H, nq)
            worst_m = max(worst_m, mass_rel_err(M2_rows[r], Mref[s_]))
            lst = O.select_contract_row(Mref[s_].astype(np.float32), p_heads[h])[0]
            oracle_lists[r] = lst
            n_diff += not np.array_equal(lst, row_csr(rp_h, ci_h, r))
    say(f"  construction masses max rel err {worst_m:.2e}; {n_diff} of {len(oracle_lists)} sampled lists differ")
    assert worst_m <= MASS_RTOL
    assert n_diff <= max(1, len(oracle_lists) // 20)

    # ---- frozen lists at other steps
    for step in (0, 3, 25, 49):
        with Timer(f"step {step}"):
            qs_, ks_ = S.drift_qk(layer, step)
            qd, kd = to_device(qs_, wl.dtype), to_device(ks_, wl.dtype)
            Og = F.losa_sparse_attn(qd, kd, v, rp, ci, order, N, R, C, out_dtype=torch.float32)
            Ms = F.losa_block_mass(qd, kd, N, R, C)
            kept = F.losa_retained_mass(Ms, rp, ci, N, R, C)
            torch.cuda.synchronize()
            kept = kept.cpu().numpy().astype(np.float64)
            w = np.array([min(R, N - i * R) for i in range(nq)], np.float64)
            wr = np.tile(w, H)
            recall_gpu = float((kept[:, 0] * wr).sum() / (kept[:, 1] * wr).sum())
            ref = head_rows(qs_, ks_)
            worst_o, rec_num_o, rec_den_o, rec_num_g, rec_den_g = 0.0, 0.0, 0.0, 0.0, 0.0
            for h, (qh, kh, iis, Mref) in ref.items():
                if h not in vh64:
                    vh64[h] = S.to_f64(layer.v[:, h:h + 1], wl.dtype)
                for s_, i in enumerate(iis):
                    r = O.row_id(0, h, i, H, nq)
                    lst = oracle_lists[r]
                    if not np.array_equal(lst, row_csr(rp_h, ci_h, r)):
                        continue  # compare recall and O only where the frozen lists agree
                    wi = min(R, N - i * R)
                    rec_num_o += wi * Mref[s_][lst].sum()
                    rec_den_o += wi * Mref[s_].sum()
                    rec_num_g += wi * kept[r, 0]
                    rec_den_g += wi * kept[r, 1]
                    r0, r1 = i * R, min((i + 1) * R, N)
                    keys = np.concatenate([np.arange(j * C, min((j + 1) * C, N)) for j in lst])
                    a = O.attention_probs(qh[0, 0, r0:r1], kh[0, 0, keys], O.softmax_scale(d))
                    oref = a @ vh64[h][0, 0, keys]
                    worst_o = max(worst_o, float(np.abs(Og[0, h, r0:r1].cpu().numpy() - oref).max()))
            rec_o, rec_g = rec_num_o / rec_den_o, rec_num_g / rec_den_g
            say(f"  step {step}: recall (all rows, GPU masses) {recall_gpu:.6f}; sampled rows oracle {rec_o:.6f} "
                f"vs GPU {rec_g:.6f}; O max abs err {worst_o:.2e}")
            assert worst_o <= ATTN_ATOL
            assert abs(rec_o - rec_g) < 1e-5
            assert 0.5 < recall_gpu <= 1.0 + 1e-6


def test_recall_every_step_sampled_rows():
    """Recall of the frozen lists at every one of the 50 steps (BASELINE
    reuse workload; LoSA page, Motivation Summary: recall of a pattern under
    a later step's dense masses): on sampled rows of two heads, the GPU's
    kept/total masses against the oracle's, step by step."""
    from concurrent.futures import ThreadPoolExecutor
    wl = S.get_workload("4")
    R = C = wl.block
    N, Na, nq = wl.tokens, wl.tokens_alloc, wl.n_blocks
    heads = [1, 7]
    layer = S.make_layer(wl, heads=heads, keep_f64=True)
    p_heads = [float(layer.p_heads[h]) for h in heads]
    rows = [(0, s, i) for s in range(2) for i in (0, 257, nq - 1)]   # slot s of the subset
    with ThreadPoolExecutor(8) as pool:  # the generator's bulk draws release the GIL
        steps = list(pool.map(lambda s: S.drift_qk(layer, s), range(wl.steps)))
    q2d, k2d = to_device(steps[wl.construct_step][0], wl.dtype), to_device(steps[wl.construct_step][1], wl.dtype)
    M2 = F.losa_block_mass(q2d, k2d, N, R, C)
    rp, ci, _ = F.losa_select(M2, p_heads, N, R, C, tokens_alloc=Na, want_order=False)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci[:int(rp_h[-1])].cpu().numpy()
    worst = 0.0
    for s, (qs_, ks_) in enumerate(steps):
        qd, kd = to_device(qs_, wl.dtype), to_device(ks_, wl.dtype)
        Ms = F.losa_block_mass(qd, kd, N, R, C)
        kept = F.losa_retained_mass(Ms, rp, ci, N, R, C).cpu().numpy().astype(np.float64)
        num_o = den_o = num_g = den_g = 0.0
        for slot in range(2):
            qh, kh = S.to_f64(qs_[:, slot:slot + 1], wl.dtype), S.to_f64(ks_[:, slot:slot + 1], wl.dtype)
            iis = [i for (_, sl, i) in rows if sl == slot]
            Mref = O.block_mass_rows(qh, kh, N, R, C, [(0, 0, i) for i in iis])
            for t, i in enumerate(iis):
                r = slot * nq + i
                wi = min(R, N - i * R)
                lst = row_csr(rp_h, ci_h, r)
                num_o += wi * Mref[t][lst].sum()
                den_o += wi * Mref[t].sum()
                num_g += wi * kept[r, 0]
                den_g += wi * kept[r, 1]
        rec_o, rec_g = num_o / den_o, num_g / den_g
        worst = max(worst, abs(rec_o - rec_g))
        if s % 7 == 0 or s == wl.steps - 1:
            say(f"  step {s}: sampled-row recall oracle {rec_o:.6f}, GPU {rec_g:.6f}")
        assert abs(rec_o - rec_g) < 1e-5, s
    say(f"recall at all {wl.steps} steps: largest oracle/GPU difference {worst:.2e}")
