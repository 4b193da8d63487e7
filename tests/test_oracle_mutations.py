"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case replaces one oracle function with a plausible wrong version --
a dropped weight, a swapped dimension, the wrong rounding -- and checks
that at least one of the pins written against the pages' definitions
(LoSA page, Motivation Summary: Recall and Coverage; Methodology Summary:
the target theta times the block's total mass) then fails.  The oracle's
own code is untouched outside this module's monkeypatching.
"""
import math

import numpy as np
import pytest

import oracle as O
import oracle.losa_oracle as OL
import test_oracle_pins as pins


def _recall_unweighted(M, row_ptr, col_idx, n_valid, R):
    flat = M.reshape(-1, M.shape[-1])
    kept = sum(flat[r, col_idx[int(row_ptr[r]):int(row_ptr[r + 1])]].sum() for r in range(flat.shape[0]))
    return float(kept / flat.sum())


def _recall_one(M, row_ptr, col_idx, n_valid, R):
    return 1.0


def _coverage_nq_squared(row_ptr, batch, heads, n_q, n_k):
    return int(np.asarray(row_ptr)[-1]) / float(batch * heads * n_q * n_q)


def _coverage_nk_squared(row_ptr, batch, heads, n_q, n_k):
    return int(np.asarray(row_ptr)[-1]) / float(batch * heads * n_k * n_k)


def _coverage_no_batch(row_ptr, batch, heads, n_q, n_k):
    return int(np.asarray(row_ptr)[-1]) / float(heads * n_q * n_k)


def _p_floor(p):
    if not (0.0 < p <= 1.0):
        raise ValueError("p must lie in (0, 1]")
    return int(math.floor(p * 4294967296.0))


def _p_half_even(p):
    if not (0.0 < p <= 1.0):
        raise ValueError("p must lie in (0, 1]")
    return int(round(p * 4294967296.0))


RECALL_PINS = [pins.test_recall_ragged_query_block_hand_worked, pins.test_recall_equals_kept_probability_over_queries]
COVERAGE_PINS = [pins.test_coverage_rectangular_blocks_hand_worked]
P_PINS = [pins.test_p_fixed_hand_worked, pins.test_p_fixed_rounding_decides_a_cut]


def _some_pin_fails(pin_fns):
    for fn in pin_fns:
        try:
            fn()
        except (AssertionError, ValueError):
            return True
    return False


def test_pins_pass_on_the_oracle_as_it_is():
    assert not _some_pin_fails(RECALL_PINS + COVERAGE_PINS + P_PINS)


@pytest.mark.parametrize("wrong", [_recall_unweighted, _recall_one])
def test_planted_recall_mistakes_fail(monkeypatch, wrong):
    monkeypatch.setattr(O, "recall", wrong)
    monkeypatch.setattr(OL, "recall", wrong)
    assert _some_pin_fails(RECALL_PINS)


@pytest.mark.parametrize("wrong", [_coverage_nq_squared, _coverage_nk_squared, _coverage_no_batch])
def test_planted_coverage_mistakes_fail(monkeypatch, wrong):
    monkeypatch.setattr(O, "coverage", wrong)
    monkeypatch.setattr(OL, "coverage", wrong)
    assert _some_pin_fails(COVERAGE_PINS)


@pytest.mark.parametrize("wrong", [_p_floor, _p_half_even])
def test_planted_p_fixed_mistakes_fail(monkeypatch, wrong):
    monkeypatch.setattr(O, "p_fixed", wrong)
    monkeypatch.setattr(OL, "p_fixed", wrong)
    assert _some_pin_fails(P_PINS)


# ---- on-the-fly thresholding against the pooled proxy

def _inpass_without_block_sizes(q, k, n_valid, R, C, theta, scale=None):
    sbar = O.pooled_scores(q, k, n_valid, R, C, scale)
    B, H, n_q, n_k = sbar.shape
    t_h = np.broadcast_to(np.asarray(theta, dtype=np.float64), (H,))
    rp, cols, margin = [0], [], math.inf
    for b in range(B):
        for h in range(H):
            for i in range(n_q):
                run, kept = -math.inf, []
                for j in range(n_k):
                    run = max(run, float(sbar[b, h, i, j]))
                    if sbar[b, h, i, j] >= math.log(t_h[h]) + run:
                        kept.append(j)
                cols.append(np.asarray(kept, np.int32))
                rp.append(rp[-1] + len(kept))
    return np.asarray(rp, np.int64), np.concatenate(cols), margin


def _pooled_scores_padding_included(q, k, n_valid, R, C, scale=None):
    B, H, Na, d = q.shape
    sc = float(np.float32(O.softmax_scale(d, scale)))
    n_q, n_k = -(-n_valid // R), -(-n_valid // C)
    qbar = np.stack([q[:, :, i * R:(i + 1) * R].mean(axis=2) for i in range(n_q)], axis=2)
    kbar = np.stack([k[:, :, j * C:(j + 1) * C].mean(axis=2) for j in range(n_k)], axis=2)
    return np.einsum("bhid,bhjd->bhij", qbar, kbar) * sc


INPASS_PINS = [pins.test_threshold_inpass_hand_worked, pins.test_threshold_inpass_is_the_online_rule_on_pooled_masses,
               pins.test_pooled_scores_explicit_loops]


def test_planted_inpass_mistakes_fail(monkeypatch):
    assert not _some_pin_fails(INPASS_PINS)
    with monkeypatch.context() as m:
        m.setattr(O, "threshold_inpass_lists", _inpass_without_block_sizes)
        assert _some_pin_fails(INPASS_PINS)
    with monkeypatch.context() as m:
        m.setattr(O, "pooled_scores", _pooled_scores_padding_included)
        m.setattr(OL, "pooled_scores", _pooled_scores_padding_included)
        assert _some_pin_fails(INPASS_PINS)
