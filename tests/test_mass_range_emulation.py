"""The block-mass kernels' choice of reference, emulated in numpy fp32 (CPU).

The matrix-core mass and construction kernels sum 2^(t - m) per key block
against a fixed reference m (scores t in log2 units), with the exponential's
result flushed to zero below 2^-126 (fp32's smallest normal number), then
scale the sums to masses.  This module emulates both the earlier choice of
reference -- each wave's first-chunk maximum plus a 64-unit headroom, the
waves' sums merged by factors 2^(m_w - m_max) -- and the current one -- one
reference per query shared by the four waves, their first chunks' maximum
-- on one query row, and compares them with the exact masses.  It shows the
band of masses that the earlier choice lost (requirement: masses exact
rather than estimated, LoSA page, Methodology Summary) and that the current
one keeps.  No GPU code runs here.
"""
import numpy as np
import pytest

TINY = np.float32(2.0 ** -126)


def _exp2_flush(x):
    """fp32 2^x with results below the smallest normal number flushed to 0."""
    y = np.exp2(np.asarray(x, np.float32)).astype(np.float32)
    return np.where(y < TINY, np.float32(0.0), y).astype(np.float32)


def _layout(n_blocks, C):
    """Wave w owns key blocks w, w+4, ...; its first chunk is block w's first 32 keys."""
    return {w: list(range(w, n_blocks, 4)) for w in range(4)}


def exact_masses(t, C):
    t = np.asarray(t, np.float64)
    p = np.exp2(t - t.max())
    p /= p.sum()
    return p.reshape(-1, C).sum(axis=1)


def masses_headroom(t, C, headroom=64.0):
    """Earlier form: per-wave reference, first chunk's maximum + headroom."""
    t32 = np.asarray(t, np.float32).reshape(-1, C)
    own = _layout(t32.shape[0], C)
    m = {w: np.float32(t32[b[0], :32].max() + headroom) for w, b in own.items() if b}
    S = {}
    tot = {}
    for w, blocks in own.items():
        if not blocks:
            continue
        tot[w] = np.float32(0.0)
        for j in blocks:
            S[j] = _exp2_flush(t32[j] - m[w]).sum(dtype=np.float32)
            tot[w] = np.float32(tot[w] + S[j])
    mm = max(m.values())
    l = np.float32(sum(np.float32(tot[w] * _exp2_flush(m[w] - mm)) for w in m))
    out = np.zeros(t32.shape[0], np.float32)
    for w, blocks in own.items():
        f = np.float32(_exp2_flush(m[w] - mm) / l) if blocks else np.float32(0)
        for j in blocks:
            out[j] = np.float32(S[j] * f)
    return out


def masses_common(t, C):
    """Current form: one reference, the largest score of the waves' first chunks."""
    t32 = np.asarray(t, np.float32).reshape(-1, C)
    own = _layout(t32.shape[0], C)
    m = max(np.float32(t32[b[0], :32].max()) for b in own.values() if b)
    S = np.array([_exp2_flush(t32[j] - m).sum(dtype=np.float32) for j in range(t32.shape[0])], np.float32)
    l = S.sum(dtype=np.float32)
    return (S / l).astype(np.float32)


def _rel(a, b):
    return np.abs(a.astype(np.float64) - b) / b


def ladder(C, lows, first=(0.0, 0.0, 0.0, 0.0), jitter=0.25, seed=0):
    """Scores (log2 units) per key: blocks 0..3 (each wave's first block) at
    `first`, then one block per entry of `lows`, each key jittered a little."""
    rng = np.random.default_rng(seed)
    levels = list(first) + list(lows)
    return np.concatenate([lv + jitter * rng.random(C) for lv in levels])


@pytest.mark.parametrize("C", [64, 128])
def test_first_chunks_highest_later_blocks_far_below(C):
    """Later blocks 50..120 log2 units below the first chunks: masses between
    about 2^-122 and 2^-52, all normal fp32 numbers."""
    lows = -np.linspace(50.0, 120.0, 12)
    t = ladder(C, lows)
    ref = exact_masses(t, C)
    assert ref.min() > 2.0 ** -126
    old = masses_headroom(t, C)
    new = masses_common(t, C)
    assert _rel(new, ref).max() < 1e-5
    lost = _rel(old, ref) > 1e-3
    assert lost.any()                                  # the earlier form loses the band ...
    assert (ref[lost] < 2.0 ** -60).all()              # ... from about 2^-64 down
    assert (old[ref < 2.0 ** -92] == 0).all()          # and flushes it completely further down


def test_waves_first_chunks_far_apart():
    """Wave 1's first block sits 150 below wave 0's, but wave 1 also owns a
    block only 60 below: the earlier form's merge factor 2^(m_1 - m_0)
    flushes to zero and takes that block's mass (about 2^-62) with it."""
    C = 64
    first = (0.0, -150.0, -100.0, 0.0)
    lows = [-80.0, -60.0, -55.0, -90.0, -110.0, -120.0, -70.0, -65.0]
    t = ladder(C, lows, first=first)
    ref = exact_masses(t, C)
    old = masses_headroom(t, C)
    new = masses_common(t, C)
    normal = ref >= 2.0 ** -126
    assert _rel(new[normal], ref[normal]).max() < 1e-5
    assert np.abs(new[~normal] - ref[~normal]).max() <= 2.0 ** -126
    assert old[5] == 0.0 and ref[5] > 2.0 ** -64       # block 5 (wave 1) lost by the earlier form


def test_no_loss_bound_of_the_current_form():
    """Keys of probability below 2^-126 may be flushed; a block made only of
    them loses at most C * 2^-126 -- the stated absolute bound."""
    C = 64
    t = ladder(C, [-125.0, -127.0, -131.0, -140.0], jitter=0.0)
    ref = exact_masses(t, C)
    new = masses_common(t, C)
    assert np.abs(new - ref).max() <= C * 2.0 ** -126
