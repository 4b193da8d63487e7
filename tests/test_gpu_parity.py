"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
seeded inputs, at sizes the oracle finishes in seconds that span several
tiles and a ragged last block.

Page cited: "LoSA: Near-Lossless Sparse Attention for Training-Free Video
Diffusion Acceleration" -- Motivation Summary (block mass), Methodology
Summary (one-time construction; sparse attention with a frozen pattern).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import synthetic as S
from tests.gpu_util import (ATTN_ATOL, MASS_RTOL, check_masses_with_floor, csr_to_device, layer_to_device,
                            mass_rel_err, row_csr, say, to_device)

pytestmark = pytest.mark.gpu

import free_block_sparse_exact_amd as F  # noqa: E402


def _wl(wid, **kw):
    return dataclasses.replace(S.get_workload(wid), **kw)


# (name, workload, heads, tokens, R, C, p)
CASES = [
    ("wl0_f32_d64", S.get_workload("0"), None, None, 64, 64, 0.9),
    ("wl0_f32_d64_p099", S.get_workload("0"), None, None, 64, 64, 0.99),  # the tiny workload as stated
    ("bf16_d128_r64_ragged", S.get_workload("1"), 2, 1000, 64, 64, 0.99),
    ("bf16_d128_r128_ragged", S.get_workload("3"), 2, 1000, 128, 128, 0.99),
    ("bf16_d128_r64_c32", S.get_workload("1"), 2, 777, 64, 32, 0.95),
    ("bf16_d128_r128_c32", S.get_workload("1"), 1, 777, 128, 32, 0.95),
    ("bf16_d64_r64", _wl("0", dtype="bf16"), 2, 700, 64, 64, 0.9),
    ("bf16_d128_r32_simt", S.get_workload("1"), 1, 500, 32, 64, 0.9),
    ("bf16_sparse_a11", S.get_workload("1s"), 2, 2000, 64, 64, 0.99),
    ("f32_d128", _wl("1", dtype="f32"), 1, 300, 64, 64, 0.9),
    ("bf16_one_token", S.get_workload("1"), 1, 1, 64, 64, 0.99),
    ("bf16_exact_multiple", S.get_workload("1"), 1, 512, 64, 64, 0.9),
]
IDS = [c[0] for c in CASES]

_cache = {}


def _case(name):
    if name in _cache:
        return _cache[name]
    _, wl, heads, tokens, R, C, p = next(c for c in CASES if c[0] == name)
    layer = S.make_layer(wl, tokens=tokens, n_heads=heads)
    wl2 = layer.wl
    N = wl2.tokens
    Na = max(-(-N // R) * R, -(-N // C) * C)
    # re-pad to this case's block geometry
    def pad(a):
        out = np.zeros(a.shape[:2] + (Na, a.shape[3]), a.dtype)
        out[:, :, :N] = a[:, :, :N]
        return out
    layer.q, layer.k, layer.v = pad(layer.q), pad(layer.k), pad(layer.v)
    q64, k64, v64 = layer.f64("q"), layer.f64("k"), layer.f64("v")
    M = O.block_mass(q64, k64, N, R, C)
    M32 = M.astype(np.float32)
    rp, ci = O.select_contract(M32, p)
    order = O.budget_order(rp, M.shape[2])
    Oref = O.sparse_attention(q64, k64, v64, N, R, C, rp, ci)
    d = dict(layer=layer, N=N, Na=Na, R=R, C=C, p=p, M=M, M32=M32, rp=rp, ci=ci, order=order, O=Oref)
    _cache[name] = d
    return d


@pytest.mark.parametrize("name", IDS)
def test_block_mass(name):
    c = _case(name)
    q, k, _ = layer_to_device(c["layer"])
    say(f"case {name}: block_mass N={c['N']} R={c['R']} C={c['C']} shape={tuple(q.shape)} {q.dtype}")
    M = F.losa_block_mass(q, k, c["N"], c["R"], c["C"])
    torch.cuda.synchronize()
    err = mass_rel_err(M.cpu().numpy(), c["M"])
    say(f"  max rel err {err:.3e}")
    assert err <= MASS_RTOL


@pytest.mark.parametrize("name", IDS)
def test_select_bit_exact_on_oracle_masses(name):
    c = _case(name)
    say(f"case {name}: select p={c['p']}")
    M = torch.from_numpy(c["M32"]).cuda()
    B, H, nq, nk = M.shape
    rp, ci, order = F.losa_select(M, c["p"], c["N"], c["R"], c["C"], tokens_alloc=c["Na"])
    torch.cuda.synchronize()
    rp = rp.cpu().numpy().astype(np.int64)
    nnz = int(rp[-1])
    assert np.array_equal(rp, c["rp"])
    assert np.array_equal(ci.cpu().numpy()[:nnz], c["ci"])
    assert np.array_equal(order.cpu().numpy(), c["order"])


@pytest.mark.parametrize("name", IDS)
def test_sparse_attn_on_oracle_lists(name):
    c = _case(name)
    q, k, v = layer_to_device(c["layer"])
    rp, ci = csr_to_device(c["rp"], c["ci"])
    order = torch.from_numpy(c["order"].astype(np.int32)).cuda()
    say(f"case {name}: sparse_attn nnz={int(c['rp'][-1])}")
    # bf16 output only where its rounding (half an ulp, 2^-8 below 2) leaves room in the tolerance
    out_dtype = torch.bfloat16 if q.dtype == torch.bfloat16 and np.abs(c["O"]).max() < 2 else torch.float32
    O_gpu = F.losa_sparse_attn(q, k, v, rp, ci, order, c["N"], c["R"], c["C"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    got = O_gpu.float().cpu().numpy().astype(np.float64)
    nqR = -(-c["N"] // c["R"]) * c["R"]
    err = np.abs(got[:, :, :nqR] - c["O"][:, :, :nqR]).max()
    say(f"  max abs err {err:.3e} (|O| max {np.abs(c['O']).max():.3f})")
    assert err <= ATTN_ATOL
    assert np.all(got[:, :, c["N"]:nqR] == 0)


@pytest.mark.parametrize("name", IDS)
def test_pipeline_lists_from_gpu_masses(name):
    """End to end: GPU masses -> GPU selection.  Lists are compared with the oracle's (from oracle
    masses); a differing row is allowed only where the oracle's cut margin is within the masses'
    fp32 error, and the recall under oracle masses must agree to 1e-5."""
    c = _case(name)
    q, k, v = layer_to_device(c["layer"])
    M = F.losa_block_mass(q, k, c["N"], c["R"], c["C"])
    rp, ci, order = F.losa_select(M, c["p"], c["N"], c["R"], c["C"], tokens_alloc=c["Na"])
    torch.cuda.synchronize()
    rp_g = rp.cpu().numpy().astype(np.int64)
    ci_g = ci.cpu().numpy()[:int(rp_g[-1])]
    rows = len(rp_g) - 1
    diff = [r for r in range(rows)
            if not np.array_equal(row_csr(rp_g, ci_g, r), row_csr(c["rp"], c["ci"], r))]
    rec_ref = O.recall(c["M"], c["rp"], c["ci"], c["N"], c["R"])
    rec_gpu = O.recall(c["M"], rp_g, ci_g, c["N"], c["R"])
    say(f"case {name}: {len(diff)} of {rows} rows differ; recall {rec_ref:.8f} vs {rec_gpu:.8f}")
    assert abs(rec_ref - rec_gpu) < 1e-5
    assert len(diff) <= max(1, rows // 100)


def test_determinism_bitwise():
    c = _case("bf16_sparse_a11")
    q, k, v = layer_to_device(c["layer"])
    outs = []
    for _ in range(2):
        M = F.losa_block_mass(q, k, c["N"], c["R"], c["C"])
        rp, ci, order = F.losa_select(M, c["p"], c["N"], c["R"], c["C"], tokens_alloc=c["Na"])
        Og = F.losa_sparse_attn(q, k, v, rp, ci, order, c["N"], c["R"], c["C"])
        torch.cuda.synchronize()
        nnz = int(rp[-1].item())
        outs.append([t.cpu().clone() for t in (M, rp, ci[:nnz], order, Og)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)


def test_p_one_keeps_all_and_equals_dense():
    c = _case("bf16_d128_r64_ragged")
    q, k, v = layer_to_device(c["layer"])
    M = torch.from_numpy(c["M32"]).cuda()
    rp, ci, order = F.losa_select(M, 1.0, c["N"], c["R"], c["C"], tokens_alloc=c["Na"])
    torch.cuda.synchronize()
    B, H, nq, nk = M.shape
    assert int(rp[-1]) == B * H * nq * nk
    Og = F.losa_sparse_attn(q, k, v, rp, ci, order, c["N"], c["R"], c["C"], out_dtype=torch.float32)
    L = c["layer"]
    dense = O.dense_attention(L.f64("q"), L.f64("k"), L.f64("v"), c["N"])
    err = np.abs(Og.cpu().numpy()[:, :, :c["N"]] - dense[:, :, :c["N"]]).max()
    say(f"p=1 vs dense max abs err {err:.3e}")
    assert err <= ATTN_ATOL


def test_empty_and_permuted_lists():
    """Rows with empty lists give 0; index order within a list and the work order do not matter."""
    c = _case("bf16_d128_r64_ragged")
    q, k, v = layer_to_device(c["layer"])
    rows = len(c["rp"]) - 1
    rng = np.random.default_rng(5)
    counts = np.diff(c["rp"]).copy()
    empty = rng.choice(rows, size=3, replace=False)
    lists = []
    for r in range(rows):
        l = row_csr(c["rp"], c["ci"], r).copy()
        if r in empty:
            l = l[:0]
        rng.shuffle(l)
        lists.append(l)
    rp = np.zeros(rows + 1, np.int64)
    rp[1:] = np.cumsum([len(l) for l in lists])
    ci = np.concatenate(lists).astype(np.int32)
    perm = rng.permutation(rows).astype(np.int32)
    rp_d, ci_d = csr_to_device(rp, ci)
    Og = F.losa_sparse_attn(q, k, v, rp_d, ci_d, torch.from_numpy(perm).cuda(), c["N"], c["R"], c["C"],
                            out_dtype=torch.float32)
    L = c["layer"]
    ref = O.sparse_attention(L.f64("q"), L.f64("k"), L.f64("v"), c["N"], c["R"], c["C"], rp, ci)
    got = Og.cpu().numpy()
    nqR = -(-c["N"] // c["R"]) * c["R"]
    assert np.abs(got[:, :, :nqR] - ref[:, :, :nqR]).max() <= ATTN_ATOL
    H, nq = q.shape[1], -(-c["N"] // c["R"])
    for r in empty:
        b, h, i = O.row_split(int(r), H, nq)
        assert np.all(got[b, h, i * c["R"]:(i + 1) * c["R"]] == 0)


def test_strided_token_major_layout():
    """Q/K/V/O as [B, N, H, d] storage viewed as [B, H, N, d] (non-default strides)."""
    c = _case("bf16_d128_r64_ragged")
    q, k, v = layer_to_device(c["layer"])
    qs, ks, vs = (t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v))
    assert qs.stride() != q.stride()
    M1 = F.losa_block_mass(q, k, c["N"], c["R"], c["C"])
    M2 = F.losa_block_mass(qs, ks, c["N"], c["R"], c["C"])
    rp, ci = csr_to_device(c["rp"], c["ci"])
    o_store = torch.empty(q.shape[0], q.shape[2], q.shape[1], q.shape[3], dtype=torch.float32, device="cuda")
    o_view = o_store.permute(0, 2, 1, 3)
    F.losa_sparse_attn(qs, ks, vs, rp, ci, None, c["N"], c["R"], c["C"], out=o_view)
    O1 = F.losa_sparse_attn(q, k, v, rp, ci, None, c["N"], c["R"], c["C"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(M1, M2)
    nqR = -(-c["N"] // c["R"]) * c["R"]
    assert torch.equal(o_view[:, :, :nqR], O1[:, :, :nqR])


def test_padding_garbage_is_ignored():
    """Padding rows (tokens >= N) may hold anything, NaN included."""
    c = _case("bf16_d128_r64_ragged")
    q, k, v = layer_to_device(c["layer"])
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    for t in (q2, k2, v2):
        t[:, :, c["N"]:] = float("nan")
    M1 = F.losa_block_mass(q, k, c["N"], c["R"], c["C"])
    M2 = F.losa_block_mass(q2, k2, c["N"], c["R"], c["C"])
    rp, ci = csr_to_device(c["rp"], c["ci"])
    O1 = F.losa_sparse_attn(q, k, v, rp, ci, None, c["N"], c["R"], c["C"], out_dtype=torch.float32)
    O2 = F.losa_sparse_attn(q2, k2, v2, rp, ci, None, c["N"], c["R"], c["C"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(M1, M2)
    nqR = -(-c["N"] // c["R"]) * c["R"]
    assert torch.equal(O1[:, :, :nqR], O2[:, :, :nqR])


def test_retained_mass_matches_recall():
    c = _case("bf16_sparse_a11")
    M = torch.from_numpy(c["M32"]).cuda()
    rp, ci = csr_to_device(c["rp"], c["ci"])
    kept = F.losa_retained_mass(M, rp, ci, c["N"], c["R"], c["C"]).cpu().numpy().astype(np.float64)
    nq = c["M"].shape[2]
    w = np.array([min(c["R"], c["N"] - i * c["R"]) for i in range(nq)], np.float64)
    wr = np.tile(w, kept.shape[0] // nq)
    rec_gpu = (kept[:, 0] * wr).sum() / (kept[:, 1] * wr).sum()
    rec_ref = O.recall(c["M32"].astype(np.float64), c["rp"], c["ci"], c["N"], c["R"])
    assert abs(rec_gpu - rec_ref) < 1e-5


def negative_logit_inputs(rng, shift, H, Na, d):
    """bf16 bit patterns of Q, K, V whose raw scores all lie near -shift: keys
    share one large direction u and queries point against it."""
    a = float(np.sqrt(shift))
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = -a * u + rng.standard_normal((1, H, Na, d)) * 0.7
    k = a * u + rng.standard_normal((1, H, Na, d)) * 0.7
    v = rng.standard_normal((1, H, Na, d))
    return [S.bf16_bits_from_f32(x.astype(np.float32)) for x in (q, k, v)]


def score_gap_inputs(rng, H, Na, d):
    """bf16 bit patterns of Q, K, V where keys [0, 256) score at least ~170
    (log2 units) below every later key."""
    a = 27.0
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    q = a * u + rng.standard_normal((1, H, Na, d)) * 0.3
    k = a * u + rng.standard_normal((1, H, Na, d)) * 0.3
    k[:, :, :256] = -a * u + rng.standard_normal((1, H, 256, d)) * 0.3
    v = rng.standard_normal((1, H, Na, d))
    return [S.bf16_bits_from_f32(x.astype(np.float32)) for x in (q, k, v)]


@pytest.mark.parametrize("shift", [225.0, 2500.0])
@pytest.mark.parametrize("N", [1000, 970])
@pytest.mark.parametrize("shuffle", [False, True])
def test_negative_logits_with_padded_tail(shift, N, shuffle):
    """All logits of a row far below zero, keys padded in the last block.

    Keys share one large direction u and queries point against it, so every
    raw score is about -shift (scaled logits about -20, or about -220 where
    2^-m of a zero score overflows fp32).  Padding keys (>= N) would score
    exactly 0, far above every real key: they must leave the softmax.  N = 970
    leaves the last 32-key chunk wholly padding; shuffled lists put the
    padded block anywhere in a row's list.
    """
    H, d, R = 2, 128, 64
    Na = -(-N // R) * R
    nq = Na // R
    rng = np.random.default_rng(int(shift) + N + 7 * shuffle)
    bits = negative_logit_inputs(rng, shift, H, Na, d)
    q64, k64, v64 = (S.f64_from_bf16_bits(b) for b in bits)
    rows = H * nq
    lists = [np.arange(nq, dtype=np.int32) for _ in range(rows)]
    if shuffle:
        for l in lists:
            rng.shuffle(l)
    rp = np.arange(rows + 1, dtype=np.int64) * nq
    ci = np.concatenate(lists)
    ref = O.sparse_attention(q64, k64, v64, N, R, R, rp, ci)
    s_max = max(float((q64[0, h, :N] @ k64[0, h, :N].T).max()) for h in range(H)) * O.softmax_scale(d)
    say(f"shift {shift}: largest scaled logit {s_max:.1f}")
    assert s_max < -10
    qd, kd, vd = (to_device(b, "bf16") for b in bits)
    rp_d, ci_d = csr_to_device(rp, ci)
    Og = F.losa_sparse_attn(qd, kd, vd, rp_d, ci_d, None, N, R, R, out_dtype=torch.float32)
    torch.cuda.synchronize()
    err = float(np.abs(Og.cpu().numpy()[:, :, :N] - ref[:, :, :N]).max())
    say(f"negative logits shift {shift} N {N} shuffle {shuffle}: max abs err {err:.3e}")
    assert err <= ATTN_ATOL


@pytest.mark.parametrize("R", [64, 128])
def test_overflow_fallback_paths(R):
    """Keys [0, 256) score at least ~170 (log2 units) below all later keys.

    Both the mass kernel and the attention kernel fix a reference at each
    wave's first chunk of keys, which here lies in the low class, so later
    chunks overflow that reference and every wave takes its exact two-pass
    fallback.  Masses of the low-class blocks (about 2^-170 of the row or less) are
    below fp32's normal range: for reference masses under 2^-126 the check is
    |M_gpu - M_ref| <= 2^-126; above, relative error <= MASS_RTOL.
    """
    H, d, N = 2, 128, 1000
    Na = -(-N // R) * R
    bits = score_gap_inputs(np.random.default_rng(2024 + R), H, Na, d)
    q64, k64, v64 = (S.f64_from_bf16_bits(b) for b in bits)
    qd, kd, vd = (to_device(b, "bf16") for b in bits)
    M_ref = O.block_mass(q64, k64, N, R, R)
    M_gpu = F.losa_block_mass(qd, kd, N, R, R).cpu().numpy().astype(np.float64)
    small = check_masses_with_floor(M_gpu, M_ref, f"fallback R={R}")
    assert small.any() and (~small).any()
    nq = Na // R
    rows = H * nq
    rp = np.arange(rows + 1, dtype=np.int64) * nq
    ci = np.tile(np.arange(nq, dtype=np.int32), rows)
    ref = O.sparse_attention(q64, k64, v64, N, R, R, rp, ci)
    rp_d, ci_d = csr_to_device(rp, ci)
    Og = F.losa_sparse_attn(qd, kd, vd, rp_d, ci_d, None, N, R, R, out_dtype=torch.float32)
    torch.cuda.synchronize()
    err = float(np.abs(Og.cpu().numpy()[:, :, :N] - ref[:, :, :N]).max())
    say(f"fallback R={R}: O max abs err {err:.3e}")
    assert err <= ATTN_ATOL


def _check_list_masses(Mg: np.ndarray, Mref: np.ndarray):
    """Masses within the lists: listed blocks (Mref > 0) within MASS_RTOL, the rest exactly 0."""
    listed = Mref > 0
    assert np.all(Mg[~listed] == 0.0)
    assert float((np.abs(Mg[listed] - Mref[listed]) / Mref[listed]).max()) <= MASS_RTOL


def test_batch_two_strided_all_calls():
    """batch = 2 with token-major storage [B, N, H, d] viewed as [B, H, N, d]:
    masses, lists, sparse attention, the construction call, the pooled proxy
    and the masses within the lists against the oracle (each batch entry is
    independent)."""
    rng = np.random.default_rng(77)
    B, H, N, d, R, C, p = 2, 2, 700, 128, 64, 64, 0.95
    Na = 704
    vals = [rng.standard_normal((B, Na, H, d)) * s for s in (1.5, 1.5, 1.0)]
    bits = [S.bf16_bits_from_f32(x.astype(np.float32)) for x in vals]
    x64 = [S.f64_from_bf16_bits(b).transpose(0, 2, 1, 3) for b in bits]  # [B, H, Na, d]
    dev = [to_device(b, "bf16").permute(0, 2, 1, 3) for b in bits]        # strided views
    q, k, v = dev
    assert not q.is_contiguous()
    M = F.losa_block_mass(q, k, N, R, C)
    M_ref = O.block_mass(x64[0], x64[1], N, R, C)
    assert mass_rel_err(M.cpu().numpy(), M_ref) <= MASS_RTOL
    rp, ci, order = F.losa_select(torch.from_numpy(M_ref.astype(np.float32)).cuda(), p, N, R, C, tokens_alloc=Na)
    rp_ref, ci_ref = O.select_contract(M_ref.astype(np.float32), p)
    rp_h = rp.cpu().numpy().astype(np.int64)
    assert np.array_equal(rp_h, rp_ref)
    assert np.array_equal(ci[:int(rp_h[-1])].cpu().numpy(), ci_ref)
    Og = F.losa_sparse_attn(q, k, v, rp, ci, order, N, R, C, out_dtype=torch.float32)
    ref = O.sparse_attention(x64[0], x64[1], x64[2], N, R, C, rp_ref, ci_ref)
    assert float(np.abs(Og.cpu().numpy()[:, :, :N] - ref[:, :, :N]).max()) <= ATTN_ATOL
    Od, Md = F.losa_dense_attn_mass(q, k, v, N, R, C, out_dtype=torch.float32)
    dense = O.dense_attention(x64[0], x64[1], x64[2], N)
    assert float(np.abs(Od.cpu().numpy()[:, :, :N] - dense[:, :, :N]).max()) <= ATTN_ATOL
    assert mass_rel_err(Md.cpu().numpy(), M_ref) <= MASS_RTOL
    P = F.losa_pooled_mass(q, k, N, R, C).cpu().numpy().astype(np.float64)
    P_ref = O.pooled_mass(x64[0], x64[1], N, R, C)
    assert float((np.abs(P - P_ref) / P_ref).max()) <= MASS_RTOL
    Os, Ms = F.losa_sparse_attn_mass(q, k, v, rp, ci, order, N, R, C, out_dtype=torch.float32)
    assert float(np.abs(Os.cpu().numpy()[:, :, :N] - ref[:, :, :N]).max()) <= ATTN_ATOL
    _check_list_masses(Ms.cpu().numpy(), O.restricted_mass(x64[0], x64[1], N, R, C, rp_ref, ci_ref))
    torch.cuda.synchronize()
    say("batch 2, strided: all calls match the oracle")


@pytest.mark.parametrize("RC", [(64, 64), (128, 32), (128, 128)])
@pytest.mark.parametrize("N", [1, 2, 31, 32, 33, 63, 64, 65, 96, 97, 127, 128, 129, 160])
def test_small_token_counts_all_calls(N, RC):
    """Token counts around every chunk and block boundary (one head, bf16, d = 128)
    through masses, selection, sparse attention on the oracle's lists in
    shuffled order, the construction call, the pooled proxy and the masses
    within the (shuffled) lists."""
    R, C = RC
    rng = np.random.default_rng(1000 * R + N)
    H, d = 1, 128
    Na = max(-(-N // R) * R, -(-N // C) * C)
    bits = [S.bf16_bits_from_f32((rng.standard_normal((1, H, Na, d)) * s).astype(np.float32))
            for s in (1.5, 1.5, 1.0)]
    q64, k64, v64 = (S.f64_from_bf16_bits(b) for b in bits)
    q, k, v = (to_device(b, "bf16") for b in bits)
    M_ref = O.block_mass(q64, k64, N, R, C)
    assert mass_rel_err(F.losa_block_mass(q, k, N, R, C).cpu().numpy(), M_ref) <= MASS_RTOL
    rp_ref, ci_ref = O.select_contract(M_ref.astype(np.float32), 0.95)
    rp, ci, order = F.losa_select(torch.from_numpy(M_ref.astype(np.float32)).cuda(), 0.95, N, R, C,
                                  tokens_alloc=Na)
    rp_h = rp.cpu().numpy().astype(np.int64)
    assert np.array_equal(rp_h, rp_ref)
    assert np.array_equal(ci[:int(rp_h[-1])].cpu().numpy(), ci_ref)
    # lists with the last (padded) block placed anywhere: shuffle each row
    lists = [row_csr(rp_ref, ci_ref, r).copy() for r in range(len(rp_ref) - 1)]
    for l in lists:
        rng.shuffle(l)
    ci_sh = np.concatenate(lists).astype(np.int32)
    rp_d, ci_d = csr_to_device(rp_ref, ci_sh)
    Og = F.losa_sparse_attn(q, k, v, rp_d, ci_d, None, N, R, C, out_dtype=torch.float32).cpu().numpy()
    ref = O.sparse_attention(q64, k64, v64, N, R, C, rp_ref, ci_ref)
    nqR = -(-N // R) * R
    assert float(np.abs(Og[:, :, :nqR] - ref[:, :, :nqR]).max()) <= ATTN_ATOL
    Od, Md = F.losa_dense_attn_mass(q, k, v, N, R, C, out_dtype=torch.float32)
    dense = O.dense_attention(q64, k64, v64, N)
    assert float(np.abs(Od.cpu().numpy()[:, :, :nqR] - dense[:, :, :nqR]).max()) <= ATTN_ATOL
    assert mass_rel_err(Md.cpu().numpy(), M_ref) <= MASS_RTOL
    P = F.losa_pooled_mass(q, k, N, R, C).cpu().numpy().astype(np.float64)
    assert float((np.abs(P - O.pooled_mass(q64, k64, N, R, C)) / P).max()) <= MASS_RTOL
    Os, Ms = F.losa_sparse_attn_mass(q, k, v, rp_d, ci_d, None, N, R, C, out_dtype=torch.float32)
    assert float(np.abs(Os.cpu().numpy()[:, :, :nqR] - ref[:, :, :nqR]).max()) <= ATTN_ATOL
    _check_list_masses(Ms.cpu().numpy(), O.restricted_mass(q64, k64, N, R, C, rp_ref, ci_ref))
