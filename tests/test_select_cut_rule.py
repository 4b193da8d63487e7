"""The selector's two sort-free searches against the sorted-prefix rule (CPU).

The retained-mass rule (LoSA page, Methodology Summary, one-time pattern
construction) sorts a row's key blocks by decreasing mass (ties: lower index
first) and keeps the shortest prefix whose exact integer units reach the
target T.  The GPU selector reaches the same cut without sorting: with
ku = 2^32 - 1 - (float bits of the mass) and F(v) = sum of the units of the
blocks with ku <= v, the cut value is the least v with F(v) >= T, found by
a most-significant-digit radix select: over the range of the keys of the
blocks with units, digits of at most 8 bits (one wave per row), or over the
whole 32-bit key in four 8-bit digits (one workgroup per row); among the blocks with ku = v (equal masses, equal
units) the cut falls on the ceil((T - F(v-1)) / q)-th in index order.

This file restates both searches in plain Python integers, written from that
description and not from the kernels, and checks that their kept sets equal
the oracle's on rows with ties, zeros, denormals, non-finite values and a
one-hot row.  It does not run the GPU code: the GPU tests compare the library
with the oracle directly; this pins the search schemes themselves.
"""
import math
import struct

import numpy as np
import pytest

import oracle as O


def _bits(m: float) -> int:
    """Float bits of a sanitised fp32 mass (NaN, inf, negatives and -0 count as 0)."""
    if not (m > 0.0 and math.isfinite(m)):
        return 0
    return struct.unpack("<I", struct.pack("<f", m))[0]


def _units(u: int, e: int) -> int:
    """ceil(m * 2^(51 - e)) for the fp32 value with bits u (exact rational arithmetic)."""
    if u == 0:
        return 0
    m = struct.unpack("<f", struct.pack("<I", u))[0]
    num, den = float(m).as_integer_ratio()
    sh = 51 - e
    if sh >= 0:
        num <<= sh
    else:
        den <<= -sh
    return -((-num) // den)


def _row_setup(m32, p):
    u = [_bits(float(x)) for x in m32]
    ku = [0xFFFFFFFF - x for x in u]
    umax = max(u)
    e = math.frexp(struct.unpack("<f", struct.pack("<I", umax))[0])[1] if umax else 0
    q = [_units(x, e) for x in u]
    P = O.p_fixed(p)
    T = -((-P * sum(q)) >> 32)
    return ku, q, T, P, e


def _finish(ku, q, T, v, e):
    """Kept set once the cut value v is known: blocks before v, then the ties by index."""
    below = sum(x for k, x in zip(ku, q) if k < v)
    qu = _units(0xFFFFFFFF - v, e)
    need = -((below - T) // qu) if (below < T and qu > 0) else 1
    ties = [j for j, k in enumerate(ku) if k == v]
    keep = [j for j, k in enumerate(ku) if k < v] + ties[:need]
    return np.array(sorted(keep))


def cut_range_radix(m32, p):
    """One wave per row: the least v found by a radix select over rel = ku - lo in
    [0, hi - lo] (lo, hi: least and greatest ku of the blocks with units), digits of at
    most 8 bits taken from the top of the range down."""
    ku, q, T, P, e = _row_setup(m32, p)
    if P == 1 << 32:
        return np.arange(len(ku))
    if T == 0:
        return _finish(ku, q, T, min(ku), e)
    pos = [k for k, x in zip(ku, q) if x > 0]
    lo, hi = min(pos), max(pos)
    top = (hi - lo).bit_length()
    pre, acc = 0, 0
    while top > 0:
        shift = max(top - 8, 0)
        hs = [0] * (1 << (top - shift))
        for k, x in zip(ku, q):
            r = k - lo
            if x > 0 and r >> top == pre >> top:
                hs[(r >> shift) & (len(hs) - 1)] += x
        cum = 0
        for d, h in enumerate(hs):
            if acc + cum + h >= T:
                break
            cum += h
        acc += cum
        pre |= d << shift
        top = shift
    return _finish(ku, q, T, lo + pre, e)


def cut_range_listed(m32, p):
    """One wave per row, as the GPU runs it: the same range radix select over
    rel = umax - u (u the mass bits, umax the largest, the range up to the least
    positive mass), but after each pass, when at most 64 blocks fall in the chosen
    digit's band, those blocks are listed in index order and the cut is taken
    among them directly: for each listed block its cumulative units (every block
    before the band plus the listed blocks of equal or larger mass); the cut is
    the largest listed mass whose cumulative units reach T, and the units
    before it are those of the larger masses only."""
    ku, q, T, P, e = _row_setup(m32, p)
    if P == 1 << 32:
        return np.arange(len(ku))
    u = [0xFFFFFFFF - k for k in ku]
    umax = max(u)
    if T == 0:
        return _finish(ku, q, T, 0xFFFFFFFF - umax, e)
    umin = min(x for x in u if x > 0)
    top = (umax - umin).bit_length()
    pre, acc, first = 0, 0, True
    while top > 0:
        shift = max(top - 8, 0)
        hs = [0] * (1 << (top - shift))
        for x, qq in zip(u, q):
            r = umax - x
            if first:
                hs[(r >> shift) & (len(hs) - 1)] += qq  # blocks without units add 0
            elif r >> top == pre >> top:
                hs[(r >> shift) & (len(hs) - 1)] += qq  # a zero in range adds 0
        first = False
        cum = 0
        for d, hh in enumerate(hs):
            if acc + cum + hh >= T:
                break
            cum += hh
        acc += cum
        pre |= d << shift
        top = shift
        if top == 0:
            break
        # the band ends at the width of the range, so zeros (rel = umax) stay out
        hi_rel = min(pre + (1 << top) - 1, umax - umin)
        band = [j for j, x in enumerate(u) if pre <= umax - x <= hi_rel]
        assert all(u[j] > 0 for j in band)
        if len(band) > 64:
            continue
        fle = [acc + sum(q[k] for k in band if u[k] >= u[j]) for j in band]
        hits = [u[j] for j, f in zip(band, fle) if f >= T]
        uv = max(hits)
        below = acc + sum(q[k] for k in band if u[k] > uv)
        assert below == sum(qq for x, qq in zip(u, q) if x > uv)
        return _finish(ku, q, T, 0xFFFFFFFF - uv, e)
    return _finish(ku, q, T, 0xFFFFFFFF - (umax - pre), e)


def cut_radix(m32, p):
    ku, q, T, P, e = _row_setup(m32, p)
    if P == 1 << 32:
        return np.arange(len(ku))
    prefix, below = 0, 0
    for pas in range(4):
        shift = 24 - 8 * pas
        hs, nz = [0] * 256, [False] * 256
        for k, x in zip(ku, q):
            if k >> (shift + 8) == prefix:
                d = (k >> shift) & 255
                hs[d] += x
                nz[d] = True
        cum = 0
        for d in range(256):
            cum += hs[d]
            if nz[d] and below + cum >= T:
                break
        below += cum - hs[d]
        prefix = (prefix << 8) | d
    return _finish(ku, q, T, prefix, e)


def _rows(rng, nk):
    rows = [rng.random(nk), rng.exponential(size=nk) ** 4, np.full(nk, 1.0 / nk),
            rng.integers(0, 4, nk) * 0.25, np.where(rng.random(nk) < 0.5, 0.0, rng.random(nk)),
            np.zeros(nk), np.eye(1, nk, int(rng.integers(nk)))[0]]
    out = [(r / max(r.sum(), 1e-300)).astype(np.float32) for r in rows]
    out.append((rng.random(nk) * 1e-38).astype(np.float32))  # denormal masses
    # dyadic masses 1/2, 1/4, ..., with the last repeated (sum exactly 1), shuffled: the
    # prefix sums hit the targets of p = 0.5, 0.75, ... exactly
    dy = np.array([2.0 ** -min(k + 1, nk - 1) for k in range(nk)] if nk > 1 else [1.0])
    out.append(rng.permutation(dy).astype(np.float32))
    bad = rng.random(nk).astype(np.float32)
    bad[rng.integers(nk, size=3)] = [np.nan, np.inf, -1.0]
    out.append(bad)
    # most blocks within a few ulps of one mass and a few far from it: the first
    # digit's band then holds more than 64 blocks (further radix passes)
    clu = (1.0 + rng.integers(0, 512, nk) * 2.0 ** -23).astype(np.float32)
    clu[rng.integers(nk, size=max(1, nk // 50))] = 8.0
    clu[rng.integers(nk, size=max(1, nk // 50))] = 1e-3
    out.append(clu / np.float32(clu.sum()))
    return out


@pytest.mark.parametrize("nk", [1, 2, 5, 64, 300, 1000])
@pytest.mark.parametrize("p", [1e-9, 0.5, 0.75, 0.9, 0.99, 0.995, 1.0])
def test_sort_free_cuts_equal_sorted_prefix_rule(nk, p):
    rng = np.random.default_rng(nk * 1000 + int(p * 1000))
    for m in _rows(rng, nk):
        ref = O.select_contract_row(m, p)[0]
        assert np.array_equal(cut_range_radix(m, p), ref)
        assert np.array_equal(cut_range_listed(m, p), ref)
        assert np.array_equal(cut_radix(m, p), ref)
