"""Pins for the fp64 oracle: checks against what the LoSA page and the
mathematics fix, independent of the oracle's own code paths.

Page cited throughout: "LoSA: Near-Lossless Sparse Attention for
Training-Free Video Diffusion Acceleration".
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_qkv(rng, B, H, Na, d, n_valid, scale_q=1.0):
    q = rng.standard_normal((B, H, Na, d)) * scale_q
    k = rng.standard_normal((B, H, Na, d))
    v = rng.standard_normal((B, H, Na, d))
    for t in (q, k, v):
        t[:, :, n_valid:] = 0.0
    return q, k, v


# ---------------------------------------------------------------- dense attention

@pytest.mark.parametrize("n_valid,Na", [(200, 256), (256, 256), (97, 128)])
def test_dense_matches_library_sdpa(n_valid, Na):
    """Motivation Summary: A = softmax(Q K^T / sqrt(d)); pinned to torch's SDPA (fp64, CPU)."""
    rng = np.random.default_rng(1)
    q, k, v = _rand_qkv(rng, 1, 2, Na, 32, n_valid, scale_q=2.0)
    ours = O.dense_attention(q, k, v, n_valid)
    mask = torch.zeros(Na, dtype=torch.bool)
    mask[:n_valid] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=mask[None, None, None, :].expand(1, 2, Na, Na))
    ref = ref.numpy()
    assert np.abs(ours[:, :, :n_valid] - ref[:, :, :n_valid]).max() < 1e-12
    assert np.all(ours[:, :, n_valid:] == 0.0)


def test_attention_two_key_closed_form():
    """Scores 0 and ln 3 give weights 1/4 and 3/4."""
    q = np.array([[1.0]])
    k = np.array([[0.0], [math.log(3.0)]])
    a = O.attention_probs(q, k, 1.0)
    assert np.allclose(a, [[0.25, 0.75]], atol=1e-15, rtol=0)


# ---------------------------------------------------------------- block masses

@pytest.mark.parametrize("n_valid,R,C", [(300, 64, 64), (256, 32, 64), (333, 128, 32), (64, 64, 64)])
def test_mass_rows_sum_to_one_and_nonnegative(n_valid, R, C):
    """Methodology Summary: every query row's probabilities add up to 1, so a block of R query
    rows carries mass R (row-mean form: each row of blocks sums to 1)."""
    rng = np.random.default_rng(2)
    Na = max(-(-n_valid // R) * R, -(-n_valid // C) * C)
    q, k, _ = _rand_qkv(rng, 2, 2, Na, 16, n_valid, scale_q=3.0)
    M = O.block_mass(q, k, n_valid, R, C)
    assert M.min() >= 0.0
    assert np.abs(M.sum(axis=-1) - 1.0).max() < 1e-12


def test_mass_zero_query_closed_form():
    """Q = 0 => A uniform over the N valid keys => M(i, j) = |valid keys of block j| / N."""
    n_valid, R, C = 150, 32, 64
    rng = np.random.default_rng(3)
    Na = 192
    _, k, _ = _rand_qkv(rng, 1, 1, Na, 8, n_valid)
    q = np.zeros_like(k)
    M = O.block_mass(q, k, n_valid, R, C)
    expect = np.array([64, 64, 22], np.float64) / n_valid
    assert np.abs(M[0, 0] - expect[None, :]).max() < 1e-15


def test_mass_single_key_block():
    """n_k = 1 => every mass is 1."""
    rng = np.random.default_rng(4)
    q, k, _ = _rand_qkv(rng, 1, 1, 64, 8, 50, 4.0)
    M = O.block_mass(q, k, 50, 16, 64)
    assert M.shape[-1] == 1 and np.abs(M - 1.0).max() < 1e-14


def test_mass_brute_force_double_sum():
    """Row-mean mass equals the page's double sum over (q, k) divided by the valid rows, by direct loops."""
    rng = np.random.default_rng(5)
    n_valid, R, C, d = 45, 16, 8, 4
    Na = 48
    q, k, _ = _rand_qkv(rng, 1, 1, Na, d, n_valid, 2.0)
    M = O.block_mass(q, k, n_valid, R, C)
    sc = 1.0 / math.sqrt(d)
    for i in range(3):
        for j in range(6):
            tot, rows = 0.0, 0
            for qq in range(i * R, min((i + 1) * R, n_valid)):
                rows += 1
                logits = [sum(q[0, 0, qq, t] * k[0, 0, kk, t] for t in range(d)) * sc for kk in range(n_valid)]
                mx = max(logits)
                z = sum(math.exp(x - mx) for x in logits)
                tot += sum(math.exp(logits[kk] - mx) / z for kk in range(j * C, min((j + 1) * C, n_valid)))
            assert abs(M[0, 0, i, j] - tot / rows) < 1e-13


# ---------------------------------------------------------------- selection

def test_golden_selection_cases():
    with open(os.path.join(GOLDEN, "selection_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        m = np.array(c["masses"], np.float32)
        kept, s = O.select_contract_row(m, c["p"])
        assert kept.tolist() == c["kept"], c
        assert s == len(c["kept"])
        kept_f, s_f, _ = O.select_float_row(m, c["p"])
        assert kept_f.tolist() == c["kept"], c


def _exact_units(m32):
    """Independent exact restatement of q_j = ceil(m_j * 2^(51-e)) with Fractions."""
    vals = [Fraction(float(x)) for x in m32]
    mx = max(vals)
    if mx == 0:
        return [0] * len(vals)
    _, e = math.frexp(float(mx))
    scale = Fraction(2) ** (51 - e)
    return [math.ceil(v * scale) for v in vals]


def test_fixed_point_units_exact():
    rng = np.random.default_rng(6)
    rows = [rng.random(40).astype(np.float32),
            (rng.random(40) ** 8).astype(np.float32),
            np.array([1e-40, 3e-41, 2e-39, 0.0], np.float32),  # denormals
            np.array([1.0, 0.5, 0.25, 2.0 ** -60], np.float32)]
    for m in rows:
        got = O.losa_oracle._fixed_point_units(O.sanitize_masses(m)).tolist()
        assert got == _exact_units(O.sanitize_masses(m)), m
        assert max(got) <= 2 ** 51
        assert all(g >= 1 for g, x in zip(got, m) if x > 0)


def _brute_force_min_card(m32, p):
    """Minimum cardinality of a block subset whose exact mass reaches p_eff * total (all 2^n subsets)."""
    vals = [Fraction(float(x)) for x in m32]
    target = Fraction(O.p_fixed(p), 2 ** 32) * sum(vals)
    n = len(vals)
    best, best_sets = None, []
    for r in range(1, n + 1):
        for comb in itertools.combinations(range(n), r):
            if sum(vals[j] for j in comb) >= target:
                best_sets.append(comb)
        if best_sets:
            best = r
            break
    return best, best_sets, target, vals


@pytest.mark.parametrize("seed", range(6))
def test_selection_brute_force_16_blocks(seed):
    """Greedy by mass is optimal for minimum cardinality: s equals the brute-force minimum, and with
    distinct masses the kept set is the unique heaviest minimum-size set."""
    rng = np.random.default_rng(100 + seed)
    n = 12 if seed < 3 else 16
    m = (rng.random(n) ** 3 + 1e-3).astype(np.float32)
    p = [0.5, 0.9, 0.99, 0.75, 0.95, 0.6][seed]
    kept, s = O.select_contract_row(m, p)
    if n == 16:
        # full 2^16 enumeration of subset masses (exact in fp64: exponent span < 29 bits)
        masks = np.arange(1 << n, dtype=np.int64)
        bits = ((masks[:, None] >> np.arange(n)) & 1).astype(np.float64)
        sums = bits @ m.astype(np.float64)
        card = bits.sum(axis=1)
        target = float(Fraction(O.p_fixed(p), 2 ** 32) * sum(Fraction(float(x)) for x in m))
        feas = sums >= target
        min_card = int(card[feas].min())
        heaviest = masks[feas & (card == min_card)][np.argmax(sums[feas & (card == min_card)])]
        heavy_set = [j for j in range(n) if (heaviest >> j) & 1]
        assert s == min_card
        assert kept.tolist() == heavy_set
    else:
        best, sets, target, vals = _brute_force_min_card(m, p)
        assert s == best
        heaviest = max(sets, key=lambda c: sum(vals[j] for j in c))
        assert kept.tolist() == list(heaviest)


@pytest.mark.parametrize("p", [0.5, 0.9, 0.95, 0.99, 0.995])
def test_selection_minimal_prefix_invariant(p):
    """cum(s) >= target > cum(s-1): dropping the smallest kept block falls below p; retained mass >= p."""
    rng = np.random.default_rng(7)
    for _ in range(50):
        m = rng.dirichlet(np.full(64, 0.3)).astype(np.float32)
        kept, s = O.select_contract_row(m, p)
        tot = sum(Fraction(float(x)) for x in m)
        target = Fraction(O.p_fixed(p), 2 ** 32) * tot
        kept_mass = sum(Fraction(float(m[j])) for j in kept)
        assert kept_mass >= target
        smallest = min(kept, key=lambda j: (m[j], -j))
        assert kept_mass - Fraction(float(m[smallest])) < target
        # every dropped block is no heavier than every kept block
        dropped = np.setdiff1d(np.arange(64), kept)
        if dropped.size:
            assert m[dropped].max() <= m[kept].min()


def test_selection_p_one_keeps_all_and_nonfinite_policy():
    m = np.array([0.5, np.nan, -0.1, np.inf, 0.25, 0.0], np.float32)
    kept, s = O.select_contract_row(m, 1.0)
    assert kept.tolist() == list(range(6))
    kept, s = O.select_contract_row(m, 0.9)
    assert kept.tolist() == [0, 4]  # non-finite and negative masses count as 0


def test_contract_matches_float_cumsum_on_workload0():
    L = S.make_layer("0")
    M = O.block_mass(L.f64("q"), L.f64("k"), 1024, 64, 64).astype(np.float32)
    for p in (0.5, 0.9, 0.95, 0.99):
        a = O.select_contract(M, p)
        b = O.select_float(M, p)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- sparse attention

def test_sparse_p_one_equals_dense():
    """Methodology Summary (sparse attention): with every block kept the frozen-pattern output is dense attention."""
    rng = np.random.default_rng(8)
    n_valid, R, C = 200, 64, 32
    q, k, v = _rand_qkv(rng, 1, 2, 256, 16, n_valid, 2.0)
    M = O.block_mass(q, k, n_valid, R, C).astype(np.float32)
    rp, ci = O.select_contract(M, 1.0)
    assert int(rp[-1]) == 2 * 4 * 7
    Os = O.sparse_attention(q, k, v, n_valid, R, C, rp, ci)
    Od = O.dense_attention(q, k, v, n_valid)
    assert np.abs(Os - Od).max() < 1e-12


def test_sparse_single_block_is_library_softmax_attention():
    """A one-block list is plain softmax attention over that block's keys (torch SDPA on the slice)."""
    rng = np.random.default_rng(9)
    n_valid, R, C = 150, 32, 64
    q, k, v = _rand_qkv(rng, 1, 1, 192, 16, n_valid, 2.0)
    n_q = 5
    row_ptr = np.arange(n_q + 1)
    col_idx = np.array([1, 0, 2, 1, 2], np.int32)
    Os = O.sparse_attention(q, k, v, n_valid, R, C, row_ptr, col_idx)
    for i in range(n_q):
        j = col_idx[i]
        keys = slice(j * C, min((j + 1) * C, n_valid))
        r0, r1 = i * R, min((i + 1) * R, n_valid)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[0, 0, r0:r1][None]), torch.from_numpy(k[0, 0, keys][None]),
            torch.from_numpy(v[0, 0, keys][None]))[0].numpy()
        assert np.abs(Os[0, 0, r0:r1] - ref).max() < 1e-12
    assert np.all(Os[0, 0, n_valid:] == 0)


def test_sparse_zero_query_mean_of_kept_values():
    """Q = 0 => uniform weights over the retained keys => O = mean of V over the kept tokens."""
    rng = np.random.default_rng(10)
    n_valid, R, C = 100, 32, 32
    _, k, v = _rand_qkv(rng, 1, 1, 128, 8, n_valid)
    q = np.zeros_like(k)
    row_ptr = np.array([0, 2, 3, 3 + 4, 8])
    col_idx = np.array([0, 3, 1, 0, 1, 2, 3, 2], np.int32)
    Os = O.sparse_attention(q, k, v, n_valid, R, C, row_ptr, col_idx)
    toks = [np.r_[0:32, 96:100], np.r_[32:64], np.r_[0:100], np.r_[64:96]]
    for i, t in enumerate(toks):
        r1 = min((i + 1) * R, n_valid)
        assert np.abs(Os[0, 0, i * R:r1] - v[0, 0, t].mean(axis=0)).max() < 1e-14


def test_recall_at_construction_and_coverage():
    """Construction retains at least p of each block row's mass; recall and coverage follow the definitions."""
    L = S.make_layer("0")
    q, k = L.f64("q"), L.f64("k")
    M = O.block_mass(q, k, 1024, 64, 64)
    for p in (0.5, 0.9):
        rp, ci = O.select_contract(M.astype(np.float32), p)
        flat = M.reshape(-1, 16)
        for r in range(flat.shape[0]):
            assert flat[r, ci[rp[r]:rp[r + 1]]].sum() >= p * flat[r].sum() - 1e-6
        rec = O.recall(M, rp, ci, 1024, 64)
        assert rec >= p - 1e-6
        assert O.coverage(rp, 1, 2, 16, 16) == rp[-1] / 512.0


def test_recall_ragged_query_block_hand_worked():
    """Motivation Summary (Recall): the page's block mass sums over a query
    block's rows, so a block of 36 valid rows weighs 36/64 of a full one.
    N = 100, R = 64 (rows 64 and 36), C = 50, two heads; masses in row-mean
    form (dyadic, exact in fp64):
      head 0: block 0 [3/4, 1/4] keeps {0}; block 1 [1/2, 1/2] keeps {1}
      head 1: block 0 [1/8, 7/8] keeps {0, 1}; block 1 [1, 0] keeps {1}
    kept = 64*3/4 + 36*1/2 + 64*1 + 36*0 = 130 of 2*(64 + 36) = 200 rows of
    mass: recall = 13/20 (an unweighted mean of row recalls gives 9/16)."""
    M = np.array([[[[0.75, 0.25], [0.5, 0.5]], [[0.125, 0.875], [1.0, 0.0]]]])
    row_ptr = np.array([0, 1, 2, 4, 5])
    col_idx = np.array([0, 1, 0, 1, 1], np.int32)
    assert Fraction(O.recall(M, row_ptr, col_idx, 100, 64)).limit_denominator(1000) == Fraction(13, 20)
    assert abs(O.recall(M, row_ptr, col_idx, 100, 64) - 0.65) < 1e-15
    # a full last block (N = 128): equal weights, recall = (3/4 + 1/2 + 1 + 0) / 4
    assert abs(O.recall(M, row_ptr, col_idx, 128, 64) - 0.5625) < 1e-15


def test_recall_equals_kept_probability_over_queries():
    """Recall from its definition on the attention itself: with the page's
    un-normalised masses the total is one unit per valid query, so recall =
    (1/(H*N)) * sum over valid queries q of the attention probability on the
    keys of q's kept blocks -- computed here query by query with explicit
    exponentials (ragged query and key blocks: N = 100, R = 64, C = 32)."""
    rng = np.random.default_rng(21)
    N, Na, R, C, H, d = 100, 128, 64, 32, 2, 8
    q, k, _ = _rand_qkv(rng, 1, H, Na, d, N, scale_q=3.0)
    M = O.block_mass(q, k, N, R, C)
    rp, ci = O.select_contract(M.astype(np.float32), 0.6)
    n_q = 2
    kept_prob = 0.0
    for h in range(H):
        for qi in range(N):
            r = h * n_q + qi // R
            blocks = set(int(j) for j in ci[rp[r]:rp[r + 1]])
            s = [sum(q[0, h, qi, t] * k[0, h, kk, t] for t in range(d)) / math.sqrt(d) for kk in range(N)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = sum(e)
            kept_prob += sum(e[kk] for kk in range(N) if kk // C in blocks) / z
    assert abs(O.recall(M, rp, ci, N, R) - kept_prob / (H * N)) < 1e-12


def test_coverage_rectangular_blocks_hand_worked():
    """Motivation Summary (Coverage): the kept share of the n_q x n_k block
    pairs, averaged over heads.  N = 256, R = 128, C = 64: n_q = 2, n_k = 4;
    head 0 keeps 3 and 1 blocks, head 1 keeps 4 and 2: (4/8 + 6/8) / 2 = 5/8."""
    rp = np.array([0, 3, 4, 8, 10])
    assert O.coverage(rp, 1, 2, 2, 4) == 0.625
    # the same rows as two batches of one head: the average runs over both
    assert O.coverage(rp, 2, 1, 2, 4) == 0.625
    # one head, one query block of 4 key blocks, 1 kept: 1/4
    assert O.coverage(np.array([0, 1]), 1, 1, 1, 4) == 0.25


def test_p_fixed_hand_worked():
    """The selection target's p in 32-bit fixed point, floor(p * 2^32 + 1/2)
    (round half up), worked by hand from the exact binary values of p:
      0.99  * 2^32 = 4252017623.04...  -> 4252017623
      0.995 * 2^32 = 4273492459.52...  -> 4273492460 (floor would give ...459)
      0.9   * 2^32 = 3865470566.4...   -> 3865470566
      0.5   * 2^32 = 2^31 exactly
      5 * 2^-33 * 2^32 = 2.5 exactly    -> 3 (half rounds up; half-to-even gives 2)
      1.0 -> 2^32 (keep every block)."""
    assert O.p_fixed(0.99) == 4252017623
    assert O.p_fixed(0.995) == 4273492460
    assert O.p_fixed(0.9) == 3865470566
    assert O.p_fixed(0.5) == 2147483648
    assert O.p_fixed(5.0 * 2.0 ** -33) == 3
    assert O.p_fixed(1.0) == 4294967296
    for bad in (0.0, -0.5, 1.0000001, float("nan")):
        with pytest.raises(ValueError):
            O.p_fixed(bad)


def test_p_fixed_rounding_decides_a_cut():
    """A row where rounding p * 2^32 (rather than flooring it) changes the cut.
    p = 0.995: P = 4273492460, the floor 4273492459 = P_f.  Masses u_j * 2^-40
    with units u = (4262754816, 10737643, 10737419, 10737418) (each exact in
    fp32; sum 2^32).  The maximum lies in [2^-9, 2^-8), so e = -8 and the
    contract rule's units are u_j * 2^19, total 2^51, T = P * 2^19.  The
    first two blocks in mass order sum to exactly P_f * 2^19: they reach
    the target when P = P_f and fall one unit of P short when P = P_f + 1."""
    u = [4262754816, 10737643, 10737419, 10737418]
    assert sum(u) == 1 << 32 and u[0] + u[1] == 4273492459
    masses = np.array([x * 2.0 ** -40 for x in u], np.float32)
    assert [int(float(m) * 2.0 ** 40) for m in masses] == u  # exact in fp32
    kept, s = O.select_contract_row(masses, 0.995)
    assert s == 3 and kept.tolist() == [0, 1, 2]
    kept, s = O.select_contract_row(masses, 4273492459 / 2.0 ** 32)
    assert s == 2 and kept.tolist() == [0, 1]


def test_budget_order():
    # two heads of three rows, counts (3, 2, 3) and (1, 2, 2); each head's
    # three rows fit one group: head 0's group (first row: count 3) runs
    # before head 1's (first row: count 2); inside a group, longest first,
    # equal counts by index
    rp = np.array([0, 3, 5, 8, 9, 11, 13])
    assert O.budget_order(rp, 3).tolist() == [0, 2, 1, 4, 5, 3]
    # heads swapped: the heavier head still runs first
    rp2 = np.array([0, 1, 3, 5, 8, 10, 13])  # counts (1, 2, 2) and (3, 2, 3)
    assert O.budget_order(rp2, 3).tolist() == [3, 5, 4, 1, 2, 0]
    # equal first counts: ties by head
    rp3 = np.array([0, 2, 3, 5, 6])          # counts (2, 1) and (2, 1)
    assert O.budget_order(rp3, 2).tolist() == [0, 1, 2, 3]
    # one row per head: groups of one row, longest first, ties by index
    assert O.budget_order(rp, 1).tolist() == [0, 2, 1, 4, 5, 3]


def test_budget_order_groups_of_32():
    """A head of 70 rows is three groups (32, 32 and 6 rows); the groups of
    two heads interleave by their first counts."""
    rng = np.random.default_rng(6)
    n_q = 70
    counts = np.concatenate([rng.integers(50, 100, n_q), rng.integers(0, 80, n_q)])
    rp = np.concatenate([[0], np.cumsum(counts)])
    groups = []
    for h in range(2):
        ranked = sorted(range(h * n_q, (h + 1) * n_q), key=lambda r: (-counts[r], r))
        for g0 in range(0, n_q, 32):
            groups.append((-counts[ranked[g0]], h, g0, ranked[g0:g0 + 32]))
    ref = [r for g in sorted(groups, key=lambda t: t[:3]) for r in g[3]]
    assert O.budget_order(rp, n_q).tolist() == ref
    assert O.ORDER_GROUP == 32


def test_budget_order_brute_force():
    """Groups are up to 32 consecutive slots of one head, rows inside by
    (-count, row), and the groups' first counts never increase."""
    rng = np.random.default_rng(5)
    for n_q, heads in ((1, 7), (4, 3), (17, 5), (64, 2), (100, 3)):
        counts = rng.integers(0, 6, size=n_q * heads)
        rp = np.concatenate([[0], np.cumsum(counts)])
        order = O.budget_order(rp, n_q)
        assert sorted(order.tolist()) == list(range(counts.size))
        seen = {h: 0 for h in range(heads)}
        pos, prev = 0, None
        while pos < order.size:
            h = int(order[pos] // n_q)
            size = min(32, n_q - seen[h])
            grp = order[pos:pos + size].tolist()
            assert all(r // n_q == h for r in grp)
            ranked = sorted(range(h * n_q, (h + 1) * n_q), key=lambda r: (-counts[r], r))
            assert grp == ranked[seen[h]:seen[h] + size]
            key = (-int(counts[grp[0]]), h)
            assert prev is None or prev <= key
            prev = key
            seen[h] += size
            pos += size


# ---------------------------------------------------------------- generator

def test_generator_deterministic_and_head_subset():
    a = S.make_layer("0")
    b = S.make_layer("0")
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    c = S.make_layer("0", heads=[1])
    assert np.array_equal(c.k[:, 0], a.k[:, 1])
    assert np.all(a.q[:, :, 1024:] == 0)
    t = S.make_layer("1", tokens=300, n_heads=3)
    assert t.q.shape == (1, 3, 320, 128) and t.q.dtype == np.uint16
    assert np.all(t.q[:, :, 300:] == 0)


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5], np.float32)
    got = S.f64_from_bf16_bits(S.bf16_bits_from_f32(x))
    assert got.tolist() == [1.0, 1.0, 1.0 + 4 * 2 ** -8, 1.0, -2.5]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- pooled proxy masses
# Reading (the pages name coarse, pooled estimates but print no formula):
# P[i, j] = |B_j| exp(qbar_i . kbar_j * scale) / sum_j' |B_j'| exp(...).

def _blockwise_constant(rng, H, N, Na, d, R, C):
    """Q constant within every query block, K constant within every key block
    (ragged last blocks included), padding rows left random."""
    q = rng.standard_normal((1, H, Na, d))
    k = rng.standard_normal((1, H, Na, d))
    for i in range(-(-N // R)):
        q[:, :, i * R:min((i + 1) * R, N)] = rng.standard_normal((1, H, 1, d)) * 1.5
    for j in range(-(-N // C)):
        k[:, :, j * C:min((j + 1) * C, N)] = rng.standard_normal((1, H, 1, d)) * 1.5
    return q, k


@pytest.mark.parametrize("N,R,C", [(1000, 64, 64), (1000, 64, 32), (777, 128, 32), (512, 64, 64)])
def test_pooled_equals_exact_masses_for_blockwise_constant_scores(N, R, C):
    """With scores constant on every (query block, key block) pair, the exact
    block mass (the pinned definition) is the block-weighted softmax of the
    pooled scores: the pooled proxy must equal it, ragged blocks included."""
    rng = np.random.default_rng(N + R + C)
    Na = max(-(-N // R) * R, -(-N // C) * C)
    q, k = _blockwise_constant(rng, 2, N, Na, 16, R, C)
    P = O.pooled_mass(q, k, N, R, C)
    M = O.block_mass(q, k, N, R, C)
    assert np.abs(P - M).max() <= 1e-12


def test_pooled_zero_query_closed_form():
    """Q = 0: every pooled score is 0, so P[i, j] = |B_j| / N (as for M)."""
    N, R, C = 1000, 64, 32
    rng = np.random.default_rng(3)
    q = np.zeros((1, 2, 1024, 8))
    k = rng.standard_normal((1, 2, 1024, 8))
    P = O.pooled_mass(q, k, N, R, C)
    size = np.array([min(C, N - j * C) for j in range(-(-N // C))], np.float64)
    assert np.abs(P - size / N).max() <= 1e-15


def test_pooled_rows_sum_to_one_and_differ_from_exact_in_general():
    rng = np.random.default_rng(5)
    N, R, C = 700, 64, 64
    q = rng.standard_normal((1, 2, 704, 16)) * 2
    k = rng.standard_normal((1, 2, 704, 16)) * 2
    P = O.pooled_mass(q, k, N, R, C)
    assert np.all(P >= 0)
    assert np.abs(P.sum(axis=3) - 1).max() <= 1e-12
    assert np.abs(P - O.block_mass(q, k, N, R, C)).max() > 1e-3  # a coarse estimate, not M


def test_pooled_brute_force_loops():
    """Explicit loops over tokens and blocks on a tiny case."""
    rng = np.random.default_rng(11)
    N, R, C, d = 70, 16, 8, 4
    q = rng.standard_normal((1, 1, 80, d))
    k = rng.standard_normal((1, 1, 80, d))
    P = O.pooled_mass(q, k, N, R, C)
    nq, nk = -(-N // R), -(-N // C)
    sc = 1.0 / math.sqrt(d)
    for i in range(nq):
        rows = range(i * R, min((i + 1) * R, N))
        qb = [sum(q[0, 0, t, e] for t in rows) / len(rows) for e in range(d)]
        w = []
        for j in range(nk):
            keys = range(j * C, min((j + 1) * C, N))
            kb = [sum(k[0, 0, t, e] for t in keys) / len(keys) for e in range(d)]
            w.append(len(keys) * math.exp(sc * sum(qb[e] * kb[e] for e in range(d))))
        for j in range(nk):
            assert abs(P[0, 0, i, j] - w[j] / sum(w)) <= 1e-13


# ---------------------------------------------------------------- masses within candidate lists
# Reading (GSRS card: reduced search with exact weights inside the attention
# pass; no formula printed): the softmax over the listed blocks' valid tokens,
# summed per listed block and averaged over the query block's valid rows.

def _random_lists(rng, rows, n_k, keep):
    row_ptr, cols = [0], []
    for _ in range(rows):
        sel = np.flatnonzero(rng.random(n_k) < keep)
        cols.append(sel)
        row_ptr.append(row_ptr[-1] + sel.size)
    return np.asarray(row_ptr, np.int64), (np.concatenate(cols) if cols else np.zeros(0, np.int64))


@pytest.mark.parametrize("N,R,C", [(1000, 64, 64), (777, 128, 32), (512, 64, 64)])
def test_restricted_mass_with_every_block_listed_is_the_block_mass(N, R, C):
    """Listing every block leaves the softmax unrestricted: M_L must equal the
    pinned block mass M."""
    rng = np.random.default_rng(N + C)
    Na = max(-(-N // R) * R, -(-N // C) * C)
    q, k, _ = _rand_qkv(rng, 1, 2, Na, 16, N, scale_q=2.0)
    n_q, n_k = -(-N // R), -(-N // C)
    rows = 2 * n_q
    row_ptr = np.arange(rows + 1, dtype=np.int64) * n_k
    col_idx = np.tile(np.arange(n_k), rows)
    ML = O.restricted_mass(q, k, N, R, C, row_ptr, col_idx)
    assert np.abs(ML - O.block_mass(q, k, N, R, C)).max() <= 1e-12


def test_restricted_mass_zero_query_closed_form_and_row_sums():
    """Q = 0: the restricted softmax is uniform over the listed valid tokens,
    so M_L[i, j] = |B_j| / (sum of |B_j'| over the list) for listed j, else 0."""
    N, R, C = 1000, 64, 32
    rng = np.random.default_rng(8)
    q = np.zeros((1, 2, 1024, 8))
    k = rng.standard_normal((1, 2, 1024, 8))
    n_q, n_k = -(-N // R), -(-N // C)
    row_ptr, col_idx = _random_lists(rng, 2 * n_q, n_k, 0.4)
    ML = O.restricted_mass(q, k, N, R, C, row_ptr, col_idx).reshape(2 * n_q, n_k)
    size = np.array([min(C, N - j * C) for j in range(n_k)], np.float64)
    for r in range(2 * n_q):
        lst = col_idx[row_ptr[r]:row_ptr[r + 1]]
        want = np.zeros(n_k)
        if lst.size:
            want[lst] = size[lst] / size[lst].sum()
            assert abs(ML[r].sum() - 1.0) <= 1e-12
        assert np.abs(ML[r] - want).max() <= 1e-15


def test_restricted_mass_brute_force_loops():
    """Explicit loops over queries, listed blocks and tokens on a tiny case."""
    rng = np.random.default_rng(21)
    N, R, C, d = 70, 16, 8, 4
    q = rng.standard_normal((1, 1, 80, d)) * 1.5
    k = rng.standard_normal((1, 1, 80, d)) * 1.5
    n_q, n_k = -(-N // R), -(-N // C)
    row_ptr, col_idx = _random_lists(rng, n_q, n_k, 0.5)
    ML = O.restricted_mass(q, k, N, R, C, row_ptr, col_idx)[0, 0]
    sc = 1.0 / math.sqrt(d)
    for i in range(n_q):
        lst = [int(j) for j in col_idx[row_ptr[i]:row_ptr[i + 1]]]
        rows_i = range(i * R, min((i + 1) * R, N))
        want = [0.0] * n_k
        for qq in rows_i:
            w = {}
            for j in lst:
                for kk in range(j * C, min((j + 1) * C, N)):
                    w[kk] = math.exp(sum(q[0, 0, qq, e] * k[0, 0, kk, e] for e in range(d)) * sc)
            z = sum(w.values())
            for j in lst:
                want[j] += sum(w[kk] for kk in range(j * C, min((j + 1) * C, N))) / z / len(rows_i)
        assert np.abs(ML[i] - np.asarray(want)).max() <= 1e-12


# ------------------------------------------------------- drift-triggered refresh

def test_qk_drift_closed_forms():
    rng = np.random.default_rng(21)
    B, H, N, Na, d = 2, 3, 10, 16, 8
    q_ref = rng.standard_normal((B, H, Na, d))
    k_ref = rng.standard_normal((B, H, Na, d))
    # a scaled copy drifts by the scale change; an unchanged tensor by 0
    dr = O.qk_drift(1.25 * q_ref, k_ref, q_ref, k_ref, N)
    assert np.allclose(dr[..., 0], 0.25, rtol=0, atol=1e-14) and np.all(dr[..., 1] == 0)
    # an orthogonal change: rows 3 e_0 moved by 4 e_1 drift by 4/3
    a = np.zeros((B, H, Na, d))
    a[:, :, :, 0] = 3.0
    b = a.copy()
    b[:, :, :, 1] = 4.0
    assert np.allclose(O.qk_drift(a, b, a, a, N)[..., 1], 4.0 / 3.0, rtol=1e-15)
    # padding rows are not tokens
    qp, qrp = q_ref.copy(), q_ref.copy()
    qp[:, :, N:] = np.nan
    qrp[:, :, N:] = 1e30
    assert np.array_equal(O.qk_drift(qp, k_ref, qrp, k_ref, N), O.qk_drift(q_ref, k_ref, q_ref, k_ref, N))
    # a zero reference: 0 if still zero, inf otherwise
    z = np.zeros_like(q_ref)
    dz = O.qk_drift(z, q_ref, z, z, N)
    assert np.all(dz[..., 0] == 0) and np.all(np.isinf(dz[..., 1]))
    # heads are measured separately
    q2 = q_ref.copy()
    q2[1, 0, :N] += 0.5
    d2 = O.qk_drift(q2, k_ref, q_ref, k_ref, N)
    assert d2[1, 0, 0] > 0 and np.count_nonzero(d2) == 1


def test_qk_drift_brute_force():
    rng = np.random.default_rng(22)
    B, H, N, Na, d = 1, 2, 5, 8, 4
    x = [rng.standard_normal((B, H, Na, d)) for _ in range(4)]
    got = O.qk_drift(x[0], x[1], x[2], x[3], N)
    for h in range(H):
        for t, (cur, ref) in enumerate(((x[0], x[2]), (x[1], x[3]))):
            num = den = 0.0
            for n in range(N):
                for c in range(d):
                    num += (cur[0, h, n, c] - ref[0, h, n, c]) ** 2
                    den += ref[0, h, n, c] ** 2
            assert abs(got[0, h, t] - math.sqrt(num) / math.sqrt(den)) <= 1e-14 * got[0, h, t]


def test_refresh_rule():
    dr = np.array([[[0.1, 0.3], [0.3, 0.1], [0.2, 0.2], [0.0, np.inf], [np.nan, 0.25], [np.nan, 0.0]]])
    assert O.refresh_heads(dr, 0.2).tolist() == [[True, True, False, True, True, False]]
    assert O.refresh_heads(dr, 0.3).tolist() == [[False, False, False, True, False, False]]


def test_qk_drift_nan_tokens():
    rng = np.random.default_rng(23)
    q = rng.standard_normal((1, 2, 6, 4))
    q2 = q.copy()
    q2[0, 0, 1, 2] = np.nan  # a NaN in a valid token of head 0 only
    d = O.qk_drift(q2, q, q, q, 6)
    assert np.isnan(d[0, 0, 0]) and d[0, 1, 0] == 0 and np.all(d[..., 1] == 0)
    assert np.isnan(O.qk_drift(q, q, q2, q, 6)[0, 0, 0])


def test_merge_lists():
    # two heads of two rows each
    rp_a, ci_a = np.array([0, 2, 3, 3, 5]), np.array([0, 1, 2, 0, 3])
    rp_b, ci_b = np.array([0, 1, 1, 4, 5]), np.array([3, 0, 1, 2, 1])
    rp, ci = O.merge_lists(rp_a, ci_a, rp_b, ci_b, np.array([False, True]), 2)
    assert rp.tolist() == [0, 2, 3, 6, 7] and ci.tolist() == [0, 1, 2, 0, 1, 2, 1]
    rp, ci = O.merge_lists(rp_a, ci_a, rp_b, ci_b, np.array([True, False]), 2)
    assert rp.tolist() == [0, 1, 1, 1, 3] and ci.tolist() == [3, 0, 3]
    for take, (r0, c0) in (([0, 0], (rp_a, ci_a)), ([1, 1], (rp_b, ci_b))):
        rp, ci = O.merge_lists(rp_a, ci_a, rp_b, ci_b, np.array(take, bool), 2)
        assert np.array_equal(rp, r0) and np.array_equal(ci, c0)


# ------------------------------------------------------------ online thresholding

def test_threshold_hand_worked():
    m = np.array([0.1, 0.5, 0.2, 0.6, 0.05], np.float32)
    assert O.select_threshold_row(m, 0.5).tolist() == [0, 1, 3]     # 0.2 < 0.25, 0.05 < 0.3
    assert O.select_threshold_row(m, 0.3).tolist() == [0, 1, 2, 3]  # 0.2 >= 0.15
    assert O.select_threshold_row(m, 1.0).tolist() == [0, 1, 3]     # the running maxima
    assert O.select_threshold_row(m, 1e-9).tolist() == [0, 1, 2, 3, 4]
    # sanitised: NaN and negatives count as 0; equality keeps
    bad = np.array([np.nan, 0.0, 0.2, -1.0, 0.1], np.float32)
    assert O.select_threshold_row(bad, 0.5).tolist() == [0, 1, 2, 4]
    # a flat row keeps everything, a one-hot row keeps the blocks up to its peak
    assert O.select_threshold_row(np.full(6, 0.25, np.float32), 0.9).tolist() == list(range(6))
    assert O.select_threshold_row(np.eye(1, 6, 3, dtype=np.float32)[0], 0.5).tolist() == [0, 1, 2, 3]


def test_threshold_log_domain_and_monotone():
    """On softmax masses, keeping m_j >= theta * running max is keeping scores
    within ln(1/theta) of the running maximum score; a larger theta keeps a
    subset."""
    rng = np.random.default_rng(41)
    for _ in range(50):
        n = int(rng.integers(1, 200))
        s = rng.standard_normal(n) * rng.uniform(0.5, 6.0)
        m = np.exp(s - s.max())
        m32 = (m / m.sum()).astype(np.float32)
        s32 = np.log(m32.astype(np.float64))            # the scores the fp32 masses carry
        for theta in (0.01, 0.1, 0.5):
            run = np.maximum.accumulate(s32)
            margin = s32 - (run + math.log(theta))
            if np.min(np.abs(margin)) < 1e-9:
                continue
            assert O.select_threshold_row(m32, theta).tolist() == np.flatnonzero(margin > 0).tolist()
        a, b = O.select_threshold_row(m32, 0.05), O.select_threshold_row(m32, 0.4)
        assert set(b.tolist()) <= set(a.tolist()) and 0 in b.tolist()


def test_threshold_csr_and_per_head():
    rng = np.random.default_rng(42)
    M = rng.random((2, 3, 4, 7)).astype(np.float32)
    rp, ci = O.select_threshold(M, [0.2, 0.6, 0.9])
    assert rp[0] == 0 and len(rp) == 2 * 3 * 4 + 1
    for b in range(2):
        for h in range(3):
            for i in range(4):
                r = O.row_id(b, h, i, 3, 4)
                assert ci[rp[r]:rp[r + 1]].tolist() == O.select_threshold_row(M[b, h, i], [0.2, 0.6, 0.9][h]).tolist()


# ---------------------------------------------------------------- on-the-fly thresholding (pooled proxy)

def _blocky_qk(xs, C, R, n_valid, n_q):
    """Queries all (1, 0); key block j all (x_j, 0): sbar_ij = scale * x_j."""
    Na = max(n_q * R, len(xs) * C)
    q = np.zeros((1, 1, Na, 2))
    k = np.zeros((1, 1, Na, 2))
    q[0, 0, :n_valid, 0] = 1.0
    for j, x in enumerate(xs):
        k[0, 0, j * C:min((j + 1) * C, n_valid), 0] = x
    return q, k


def test_threshold_inpass_hand_worked():
    """Sol-Attn page, on-the-fly thresholding (reading in the oracle's header).
    Scale 1, C = 4, block scores x = (0, 2, 0.5, 1.5), theta = e^-1:
    a = x + ln|B_j|; full blocks: a = x + ln 4; running max after block 1 is
    2 + ln 4; block 2: 0.5 + ln 4 < -1 + 2 + ln 4 -> dropped; block 3 (full):
    1.5 + ln 4 >= 1 + ln 4 -> kept: {0, 1, 3}.  With N = 14 the last block has
    2 valid keys: a_3 = 1.5 + ln 2 = 2.19 < 1 + ln 4 = 2.39 -> dropped: {0, 1}."""
    theta = math.exp(-1.0)
    q, k = _blocky_qk([0.0, 2.0, 0.5, 1.5], 4, 4, 16, 4)
    rp, ci, margin = O.threshold_inpass_lists(q, k, 16, 4, 4, theta, scale=1.0)
    assert rp.tolist() == [0, 3, 6, 9, 12] and ci.tolist() == [0, 1, 3] * 4
    assert abs(margin - 0.5) < 1e-12   # blocks 2 and 3 lie 0.5 below and above the line
    q, k = _blocky_qk([0.0, 2.0, 0.5, 1.5], 4, 4, 14, 4)
    rp, ci, margin = O.threshold_inpass_lists(q, k, 14, 4, 4, theta, scale=1.0)
    assert ci[:rp[1]].tolist() == [0, 1]
    assert abs(margin - (math.log(2.0) - 0.5)) < 1e-12   # block 3: ln 2 - 0.5 below the line


def test_threshold_inpass_is_the_online_rule_on_pooled_masses():
    """Log-domain decision == the online-thresholding rule applied to the
    pooled proxy masses P (Z cancels), wherever no decision is a near tie."""
    rng = np.random.default_rng(31)
    for n_valid, R, C, theta in ((300, 64, 32, 0.05), (777, 128, 64, 0.2), (1000, 64, 64, 0.01)):
        Na = max(-(-n_valid // R) * R, -(-n_valid // C) * C)
        q, k, _ = _rand_qkv(rng, 1, 2, Na, 16, n_valid, scale_q=4.0)
        rp, ci, margin = O.threshold_inpass_lists(q, k, n_valid, R, C, theta)
        assert margin > 1e-6
        P = O.pooled_mass(q, k, n_valid, R, C, scale=float(np.float32(1.0 / 4.0)))
        rp2, ci2 = O.select_threshold(P.astype(np.float32), theta)
        assert np.array_equal(rp, rp2) and np.array_equal(ci, ci2)


def test_threshold_inpass_limits():
    """theta tiny keeps every block; theta = 1 keeps exactly the running-maximum
    records (blocks whose weighted proxy is >= every earlier one)."""
    rng = np.random.default_rng(32)
    n_valid, R, C = 500, 64, 32
    q, k, _ = _rand_qkv(rng, 1, 2, 512, 8, n_valid, scale_q=3.0)
    n_q, n_k = 8, 16
    rp, ci, _ = O.threshold_inpass_lists(q, k, n_valid, R, C, 1e-300)
    assert int(rp[-1]) == 2 * n_q * n_k
    rp, ci, _ = O.threshold_inpass_lists(q, k, n_valid, R, C, 1.0)
    sbar = O.pooled_scores(q, k, n_valid, R, C)
    sizes = [min(C, n_valid - j * C) for j in range(n_k)]
    for r in range(2 * n_q):
        h, i = divmod(r, n_q)
        a = [sbar[0, h, i, j] + math.log(sizes[j]) for j in range(n_k)]
        records = [j for j in range(n_k) if all(a[j] >= a[t] for t in range(j))]
        assert ci[rp[r]:rp[r + 1]].tolist() == records


def test_pooled_scores_explicit_loops():
    """sbar by explicit loops over valid tokens (ragged query and key blocks)."""
    rng = np.random.default_rng(33)
    n_valid, R, C, d = 45, 16, 8, 3
    q, k, _ = _rand_qkv(rng, 1, 1, 48, d, n_valid, 2.0)
    q[0, 0, n_valid:] = 7.0   # padding must not enter the means
    k[0, 0, n_valid:] = -5.0
    sbar = O.pooled_scores(q, k, n_valid, R, C, scale=0.5)
    for i in range(3):
        rows = range(i * R, min((i + 1) * R, n_valid))
        qb = [sum(q[0, 0, r, t] for r in rows) / len(rows) for t in range(d)]
        for j in range(6):
            keys = range(j * C, min((j + 1) * C, n_valid))
            kb = [sum(k[0, 0, c, t] for c in keys) / len(keys) for t in range(d)]
            assert abs(sbar[0, 0, i, j] - 0.5 * sum(qb[t] * kb[t] for t in range(d))) < 1e-13


def test_threshold_inpass_blockwise_constant_is_exact_thresholding():
    """Scores constant on every block pair: the pooled proxy equals the exact
    masses, so the in-pass lists are the online rule on the exact masses."""
    rng = np.random.default_rng(34)
    n_valid, R, C = 200, 32, 64
    n_q, n_k = 7, 4
    q = np.zeros((1, 1, 256, 2))
    k = np.zeros((1, 1, 256, 2))
    for i in range(n_q):
        q[0, 0, i * R:min((i + 1) * R, n_valid)] = rng.standard_normal(2) * 3
    for j in range(n_k):
        k[0, 0, j * C:min((j + 1) * C, n_valid)] = rng.standard_normal(2) * 3
    rp, ci, margin = O.threshold_inpass_lists(q, k, n_valid, R, C, 0.1)
    assert margin > 1e-6
    M = O.block_mass(q, k, n_valid, R, C, scale=float(np.float32(1.0 / math.sqrt(2))))
    rp2, ci2 = O.select_threshold(M.astype(np.float32), 0.1)
    assert np.array_equal(rp, rp2) and np.array_equal(ci, ci2)
