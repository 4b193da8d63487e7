"""GPU parity of sparse attention with on-the-fly block thresholding
(losa_sparse_attn_threshold) against the oracle.

Sol-Attn page (abstract): blocks are chosen while the online softmax runs,
by comparing each block's proxy score with a threshold, without a proxy map.
The oracle's reading (threshold_inpass_lists) decides in fp64 on pooled
scores; both sides then take the same decisions wherever none lies within
1e-9 of a tie, which every case here asserts first.  Checked: the kept-block
count and bit mask of every row, bit for bit, and O against the oracle's
sparse attention over those blocks (max abs error <= 1e-2).
"""
import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from tests.gpu_util import ATTN_ATOL, layer_to_device, sample_rows, say

pytestmark = pytest.mark.gpu

import free_block_sparse_exact_amd as F  # noqa: E402

TIE = 1e-9


def _pad(layer, N, R, C):
    Na = max(-(-N // R) * R, -(-N // C) * C)
    for name in ("q", "k", "v"):
        a = getattr(layer, name)
        out = np.zeros(a.shape[:2] + (Na, a.shape[3]), a.dtype)
        out[:, :, :N] = a[:, :, :N]
        setattr(layer, name, out)
    return layer


def _mask_bits(mask, n_k):
    m = np.asarray(mask).astype(np.uint32)
    bits = ((m[:, :, None] >> np.arange(32, dtype=np.uint32)) & 1).reshape(m.shape[0], -1)
    return bits[:, :n_k].astype(bool)


def _oracle_mask(rp, ci, rows, n_k):
    out = np.zeros((rows, n_k), bool)
    for r in range(rows):
        out[r, ci[rp[r]:rp[r + 1]]] = True
    return out


CASES = [
    # (name, workload, heads, tokens, R, C, theta)
    ("sparse_a11_r64", "1s", 2, 2000, 64, 64, 0.01),
    ("sparse_a11_r128", "1s", 2, 2000, 128, 128, 0.03),
    ("sparse_a11_r64_c32", "1s", 2, 1500, 64, 32, [0.05, 0.002]),
    ("sparse_a11_r128_c32", "1s", 1, 1333, 128, 32, 0.1),
    ("wan_d128_theta_one", "1", 2, 1000, 64, 64, 1.0),
    ("wan_d128_theta_tiny", "1", 1, 777, 128, 64, 1e-30),
    ("d64_ragged", "0", 2, 1000, 64, 64, 0.2),
    ("one_token", "1", 1, 1, 64, 64, 0.5),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_inpass_small(case):
    name, wid, heads, N, R, C, theta = case
    wl = S.get_workload(wid)
    if wl.dtype != "bf16":
        import dataclasses
        wl = dataclasses.replace(wl, dtype="bf16")
    layer = _pad(S.make_layer(wl, tokens=N, n_heads=heads), N, R, C)
    q64, k64, v64 = layer.f64("q"), layer.f64("k"), layer.f64("v")
    rp, ci, margin = O.threshold_inpass_lists(q64, k64, N, R, C, theta)
    say(f"{name}: closest decision {margin:.2e} from a tie, {int(rp[-1])} kept blocks")
    assert margin > TIE
    Oref = O.sparse_attention(q64, k64, v64, N, R, C, rp, ci)
    q, k, v = layer_to_device(layer)
    Og, cnt, mask = F.losa_sparse_attn_threshold(q, k, v, theta, N, R, C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    n_k = -(-N // C)
    rows = rp.size - 1
    assert np.array_equal(cnt.cpu().numpy(), np.diff(rp)), "kept counts"
    assert np.array_equal(_mask_bits(mask.cpu().numpy(), n_k), _oracle_mask(rp, ci, rows, n_k)), "kept blocks"
    err = float(np.abs(Og.cpu().numpy()[:, :, :N] - Oref[:, :, :N]).max())
    say(f"{name}: O max abs err {err:.3e}")
    assert err <= ATTN_ATOL
    assert np.all(Og.cpu().numpy()[:, :, N:-(-N // R) * R] == 0)


@pytest.mark.parametrize("wid,theta", [("1", 0.5), ("1s", 0.01)])
def test_inpass_full_layer(wid, theta):
    """Every row's kept blocks of the full Wan2.1-1.3B 480p layer (12 heads x
    32760 tokens) and its sparse variant, bit for bit; O on sampled rows."""
    wl = S.get_workload(wid)
    layer = S.make_layer(wl)
    q64, k64 = layer.f64("q"), layer.f64("k")
    N, R, C = wl.tokens, wl.block, wl.key_block
    rp, ci, margin = O.threshold_inpass_lists(q64, k64, N, R, C, theta)
    say(f"full layer {wid}: closest decision {margin:.2e} from a tie, coverage "
        f"{int(rp[-1]) / ((rp.size - 1) * (-(-N // C))):.3f}")
    assert margin > TIE
    q, k, v = layer_to_device(layer)
    Og, cnt, mask = F.losa_sparse_attn_threshold(q, k, v, theta, N, R, C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    n_k = -(-N // C)
    rows = rp.size - 1
    assert np.array_equal(cnt.cpu().numpy(), np.diff(rp))
    assert np.array_equal(_mask_bits(mask.cpu().numpy(), n_k), _oracle_mask(rp, ci, rows, n_k))
    v64 = layer.f64("v")
    n_q = -(-N // R)
    sample = sample_rows(wl.heads, n_q, seed=400, n_uniform=24)
    refs = O.sparse_attention_rows(q64, k64, v64, N, R, C, rp, ci, sample)
    Oh = Og.cpu().numpy()
    err = 0.0
    for (b, h, i), ref in zip(sample, refs):
        err = max(err, float(np.abs(Oh[b, h, i * R:i * R + ref.shape[0]] - ref).max()))
    say(f"full layer {wid}: O max abs err {err:.3e} on {len(sample)} sampled rows")
    assert err <= ATTN_ATOL
