"""losa_select_noalloc: the selection without a workspace (its scratch in
the library's file-scope device array) against losa_select, bit for bit.

Two calls in a row on the one GPU array, the second with a smaller input
(the array keeps the first call's contents), with one p for all heads and
per-head p; the outputs are row_ptr, col_idx and the work order.  Masses are
seeded synthetic rows of the layer shapes' widths (the selector reads only
M), with ties, zeros and non-finite entries mixed in.
"""
import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

import free_block_sparse_exact_amd as F  # noqa: E402


def _masses(rng, B, H, nq, nk):
    m = rng.gamma(0.3, size=(B, H, nq, nk)).astype(np.float32)
    m /= m.sum(axis=-1, keepdims=True)
    flat = m.reshape(-1, nk)
    for r in range(0, flat.shape[0], 7):   # ties, zeros and a NaN now and then
        flat[r, :: max(1, nk // 5)] = flat[r, 0]
        flat[r, 1] = 0.0
        if r % 21 == 0:
            flat[r, 2] = np.nan
    return torch.from_numpy(m).cuda()


def _both(M, p, N, R, C):
    B, H, nq, nk = M.shape
    rows = B * H * nq
    ref = F.losa_select(M, p, N, R, C)
    rp = torch.full((rows + 1,), -1, dtype=torch.int32, device="cuda")
    ci = torch.full((rows * nk,), -1, dtype=torch.int32, device="cuda")
    order = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    F.losa_select_noalloc(M, p, N, R, C, rp, ci, order)
    torch.cuda.synchronize()
    nnz = int(ref[0][-1].item())
    assert torch.equal(rp, ref[0]), "row_ptr"
    assert torch.equal(ci[:nnz], ref[1][:nnz]), "col_idx"
    assert torch.equal(order, ref[2]), "order"
    return nnz


def test_noalloc_matches_select_two_calls_second_smaller():
    rng = np.random.default_rng(77)
    # first: the Wan2.1-1.3B 480p layer's shape (12 heads x 512 x 512 blocks)
    N1, R1 = 32760, 64
    M1 = _masses(rng, 1, 12, 512, 512)
    nnz1 = _both(M1, 0.99, N1, R1, R1)
    # second, smaller: 2 heads x 16 x 16 blocks, one p per head
    M2 = _masses(rng, 1, 2, 16, 16)
    nnz2 = _both(M2, [0.9, 0.5], 1000, 64, 64)
    # and the first shape again after the smaller one, then a wide row (n_k = 3713)
    _both(M1, 0.95, N1, R1, R1)
    M3 = _masses(rng, 1, 1, 929, 3713)   # one head of the HunyuanVideo layer with 32-token key blocks
    _both(M3, 0.99, 118800, 128, 32)
    say(f"noalloc select: identical to losa_select ({nnz1} and {nnz2} kept blocks)")


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """A layer whose selector workspace exceeds the array is refused before
    any launch (LOSA_ERR_WORKSPACE); the outputs are untouched."""
    B, H, N, R = 1, 127, 4096 * 64 - 5, 64
    g = F.Geometry(B, H, N, 4096 * 64, 128, R, R, F.LOSA_BF16)
    assert F.losa_select_workspace(g) > F.SELECT_SCRATCH_BYTES
    lib = F.load_library()
    rp = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    p = (ctypes.c_double * 1)(0.99)
    st = lib.losa_select_noalloc(ctypes.byref(g.shape()), rp.data_ptr(), p, 1, rp.data_ptr(), rp.data_ptr(),
                                 g.rows * g.n_k, None, None)
    assert st == 4  # LOSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.equal(rp.cpu(), torch.full((4,), 7, dtype=torch.int32))
