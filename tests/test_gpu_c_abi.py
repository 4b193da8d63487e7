"""The path driven through the C ABI alone: tests/c_abi/losa_path.c (plain C,
HIP runtime and losa.h only; no Python or PyTorch in the process) runs block
masses, selection and sparse attention on a seeded layer written to a file,
and its outputs are checked against the fp64 oracle: masses within 1e-3
relative, lists and work order (selected from the oracle's fp32 masses)
bit-exact, O within 1e-2 absolute on those lists.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle as O
import synthetic as S
from tests.gpu_util import ATTN_ATOL, MASS_RTOL, mass_rel_err, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROGRAM = os.path.join(ROOT, "tests", "c_abi", "losa_path")


@pytest.mark.parametrize("N,R,C,H", [(1000, 64, 64, 2), (777, 128, 32, 1)])
def test_c_program_matches_oracle(tmp_path, N, R, C, H):
    if not os.path.exists(PROGRAM):
        pytest.fail("tests/c_abi/losa_path is not built (run __graft_entry__.build())")
    layer = S.make_layer("1", tokens=N, n_heads=H)
    d = layer.q.shape[-1]
    Na = max(-(-N // R) * R, -(-N // C) * C)

    def pad(a):
        out = np.zeros(a.shape[:2] + (Na, d), np.uint16)
        out[:, :, :N] = a[:, :, :N]
        return out
    q, k, v = (pad(getattr(layer, n)) for n in ("q", "k", "v"))
    q64, k64, v64 = (S.f64_from_bf16_bits(x) for x in (q, k, v))
    p = 0.95
    M_ref = O.block_mass(q64, k64, N, R, C)
    M32 = M_ref.astype(np.float32)
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        np.array([1, H, N, Na, d, R, C], np.int32).tofile(f)
        np.array([p], np.float64).tofile(f)
        for x in (q, k, v):
            np.ascontiguousarray(x).tofile(f)
        M32.tofile(f)
    r = subprocess.run([PROGRAM, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stderr
    n_q, n_k = M_ref.shape[2], M_ref.shape[3]
    rows = H * n_q
    buf = np.fromfile(out, np.uint8)
    pos = 0

    def take(dtype, n):
        nonlocal pos
        a = buf[pos:pos + 4 * n].view(dtype)
        pos += 4 * n
        return a
    M_c = take(np.float32, rows * n_k).reshape(M_ref.shape)
    rp = take(np.int32, rows + 1).astype(np.int64)
    ci = take(np.int32, int(rp[-1]))
    order = take(np.int32, rows)
    O_c = take(np.float32, H * Na * d).reshape(1, H, Na, d)
    assert pos == buf.size
    assert mass_rel_err(M_c, M_ref) <= MASS_RTOL
    rp_ref, ci_ref = O.select_contract(M32, p)
    assert np.array_equal(rp, rp_ref) and np.array_equal(ci, ci_ref)
    assert np.array_equal(order, O.budget_order(rp_ref, n_q))
    ref = O.sparse_attention(q64, k64, v64, N, R, C, rp_ref, ci_ref)
    err = float(np.abs(O_c[:, :, :N] - ref[:, :, :N]).max())
    say(f"C program N={N} R={R} C={C}: O max abs err {err:.2e}")
    assert err <= ATTN_ATOL
