"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects every malformed argument on the host with its
status code before any HIP call (no device is touched: pointers passed here
are fake, non-null addresses that the library must never dereference)."""
import ctypes
import os
import re

import pytest

import free_block_sparse_exact_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "losa.h")

OK, NULL, INVALID, UNSUPPORTED, WORKSPACE, CAPACITY = 0, 1, 2, 3, 4, 5
FAKE = 0x10000  # 16-byte aligned fake device address; never dereferenced on these paths


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


# The argument-error tests hand the library fake device addresses and rely on
# host validation rejecting every call; they run only where no GPU is visible,
# so a validation bug can never turn into a launch on a bogus address.
no_gpu_only = pytest.mark.skipif(_gpu_visible(), reason="fake device pointers: host-only test")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(F.LIB_PATH):
        pytest.fail("liblosa.so is not built (run __graft_entry__.build())")
    return F.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[a-z_0-9]+\s*\*?\s+)+\**(losa_[a-z_0-9]+)\s*\(", text, re.M)))


def test_header_functions_exported(lib):
    names = declared_functions()
    assert {"losa_block_mass", "losa_select", "losa_sparse_attn", "losa_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.losa_abi_version() == 1
    for st in range(7):
        assert lib.losa_status_string(st)


def geom(**kw):
    base = dict(batch=1, heads=2, tokens=1000, tokens_alloc=1024, head_dim=128, q_block=64, k_block=64,
                dtype=F.LOSA_BF16)
    base.update(kw)
    return F.Geometry(**base)


def shape(**kw):
    s = geom(**{k: v for k, v in kw.items() if k in F.Geometry.__dataclass_fields__}).shape()
    for k, v in kw.items():
        if k not in F.Geometry.__dataclass_fields__:
            setattr(s, k, v)
    return s


def mass(lib, s, Q=FAKE, K=FAKE, M=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return lib.losa_block_mass(ctypes.byref(s), Q, K, M, ws, ws_bytes, None)


def test_workspace_queries(lib):
    n = ctypes.c_size_t()
    assert lib.losa_block_mass_workspace(ctypes.byref(shape()), ctypes.byref(n)) == OK and n.value > 0
    assert lib.losa_select_workspace(ctypes.byref(shape()), ctypes.byref(n)) == OK and n.value > 0
    assert lib.losa_sparse_attn_workspace(ctypes.byref(shape()), ctypes.byref(n)) == OK and n.value > 0
    assert lib.losa_sparse_attn_workspace(ctypes.byref(shape(dtype=F.LOSA_F32)), ctypes.byref(n)) == OK
    assert n.value == 0  # the f32 path needs no packed copies
    assert lib.losa_block_mass_workspace(ctypes.byref(shape()), None) == NULL
    assert lib.losa_block_mass_workspace(None, ctypes.byref(n)) == NULL


@no_gpu_only
@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), UNSUPPORTED),
    (dict(q_block=48), UNSUPPORTED),
    (dict(k_block=256), UNSUPPORTED),
    (dict(tokens=0), INVALID),
    (dict(heads=0), INVALID),
    (dict(batch=0), INVALID),
    (dict(tokens_alloc=1000), INVALID),          # below n_q * R = 1024
    (dict(dtype=7), INVALID),
    (dict(reserved=1), INVALID),
    (dict(softmax_scale=float("nan")), INVALID),
    (dict(tokens=4096 * 64 + 1, tokens_alloc=4097 * 64), UNSUPPORTED),  # n_k > 4096
])
def test_shape_errors(lib, kw, code):
    assert mass(lib, shape(**kw)) == code


@no_gpu_only
def test_pointer_and_stride_errors(lib):
    assert mass(lib, shape(), Q=None) == NULL
    assert mass(lib, shape(), M=None) == NULL
    assert mass(lib, shape(), Q=FAKE + 2) == INVALID      # misaligned
    s = shape()
    s.q_stride[2] = 100                                   # not a multiple of 8 bf16 elements
    assert mass(lib, s) == INVALID
    s = shape()
    s.k_stride[2] = 64                                    # token stride below head_dim
    assert mass(lib, s) == INVALID
    assert mass(lib, shape(), ws_bytes=16) == WORKSPACE


@no_gpu_only
def test_select_errors(lib):
    s = shape()
    rows, nk = 2 * 16, 16
    p1 = (ctypes.c_double * 1)(0.99)

    def sel(p=p1, n_p=1, cap=rows * nk, ws=0x100000, ws_bytes=1 << 40, rp=FAKE):
        return lib.losa_select(ctypes.byref(s), FAKE, p, n_p, rp, FAKE, cap, None, ws, ws_bytes, None)

    assert sel(cap=rows * nk - 1) == CAPACITY
    assert sel(p=(ctypes.c_double * 1)(0.0)) == INVALID
    assert sel(p=(ctypes.c_double * 1)(1.5)) == INVALID
    assert sel(p=(ctypes.c_double * 1)(float("nan"))) == INVALID
    assert sel(n_p=3) == INVALID
    assert sel(p=(ctypes.c_double * 2)(0.9, 2.0), n_p=2) == INVALID
    assert sel(ws=0x100010) == WORKSPACE                  # not 256-byte aligned
    assert sel(ws_bytes=8) == WORKSPACE
    assert sel(rp=None) == NULL


@no_gpu_only
def test_select_noalloc_errors(lib):
    """The allocation-free selection checks its arguments like losa_select and
    refuses shapes whose scratch exceeds its device array, all before any HIP
    call."""
    s = shape()
    rows, nk = 2 * 16, 16
    p1 = (ctypes.c_double * 1)(0.99)

    def sel(sh=s, p=p1, n_p=1, cap=rows * nk, rp=FAKE):
        return lib.losa_select_noalloc(ctypes.byref(sh), FAKE, p, n_p, rp, FAKE, cap, None, None)

    assert sel(cap=rows * nk - 1) == CAPACITY
    assert sel(p=(ctypes.c_double * 1)(0.0)) == INVALID
    assert sel(n_p=3) == INVALID
    assert sel(rp=None) == NULL
    big = geom(heads=127, tokens=4096 * 64 - 5, tokens_alloc=4096 * 64)
    assert F.losa_select_workspace(big) > F.SELECT_SCRATCH_BYTES
    assert sel(sh=big.shape(), cap=big.rows * big.n_k) == WORKSPACE


@no_gpu_only
def test_sparse_attn_errors(lib):
    s = shape()

    def attn(o_dtype=F.LOSA_BF16, ws=FAKE, ws_bytes=1 << 40, V=FAKE, O=FAKE):
        return lib.losa_sparse_attn(ctypes.byref(s), FAKE, FAKE, V, FAKE, FAKE, None, O, o_dtype, ws, ws_bytes, None)

    assert attn(o_dtype=5) == INVALID
    assert attn(V=None) == NULL
    assert attn(O=FAKE + 8) == INVALID
    assert attn(ws_bytes=1) == WORKSPACE
    assert attn(ws=None) == NULL


@no_gpu_only
def test_dense_attn_mass_errors(lib):
    s = shape()
    n = ctypes.c_size_t()
    assert lib.losa_dense_attn_mass_workspace(ctypes.byref(s), ctypes.byref(n)) == OK and n.value > 0

    def dense(M=FAKE, O=FAKE, o_dtype=F.LOSA_BF16, ws=FAKE, ws_bytes=1 << 40, V=FAKE):
        return lib.losa_dense_attn_mass(ctypes.byref(s), FAKE, FAKE, V, M, O, o_dtype, ws, ws_bytes, None)

    assert dense(M=None) == NULL
    assert dense(O=None) == NULL
    assert dense(V=None) == NULL
    assert dense(ws=None) == NULL
    assert dense(o_dtype=3) == INVALID
    assert dense(M=FAKE + 4) == INVALID
    assert dense(ws_bytes=n.value - 1) == WORKSPACE
    assert lib.losa_dense_attn_mass(ctypes.byref(shape(head_dim=96)), FAKE, FAKE, FAKE, FAKE, FAKE, F.LOSA_BF16,
                                    FAKE, 1 << 40, None) == UNSUPPORTED


@no_gpu_only
def test_pooled_mass_errors(lib):
    s = shape()
    n = ctypes.c_size_t()
    assert lib.losa_pooled_mass_workspace(ctypes.byref(s), ctypes.byref(n)) == OK and n.value > 0

    def pooled(P=FAKE, ws=FAKE, ws_bytes=1 << 40, K=FAKE):
        return lib.losa_pooled_mass(ctypes.byref(s), FAKE, K, P, ws, ws_bytes, None)

    assert pooled(P=None) == NULL
    assert pooled(K=None) == NULL
    assert pooled(ws=None) == NULL
    assert pooled(P=FAKE + 4) == INVALID
    assert pooled(ws_bytes=n.value - 1) == WORKSPACE


@no_gpu_only
def test_sparse_attn_mass_errors(lib):
    s = shape()
    n = ctypes.c_size_t()
    assert lib.losa_sparse_attn_mass_workspace(ctypes.byref(s), ctypes.byref(n)) == OK and n.value > 0

    def call(shp=s, rp=FAKE, ci=FAKE, M=FAKE, O=FAKE, o_dtype=F.LOSA_BF16, ws=FAKE, ws_bytes=1 << 40, V=FAKE):
        return lib.losa_sparse_attn_mass(ctypes.byref(shp), FAKE, FAKE, V, rp, ci, None, M, O, o_dtype, ws,
                                         ws_bytes, None)

    assert call(rp=None) == NULL
    assert call(ci=None) == NULL
    assert call(M=None) == NULL
    assert call(O=None) == NULL
    assert call(V=None) == NULL
    assert call(ws=None) == NULL
    assert call(o_dtype=3) == INVALID
    assert call(M=FAKE + 4) == INVALID
    assert call(ws_bytes=n.value - 1) == WORKSPACE
    # matrix-core shapes only: f32 inputs and 32-row query blocks are refused, query included
    for kw in (dict(dtype=F.LOSA_F32), dict(q_block=32)):
        assert lib.losa_sparse_attn_mass_workspace(ctypes.byref(shape(**kw)), ctypes.byref(n)) == UNSUPPORTED
        assert call(shp=shape(**kw)) == UNSUPPORTED


@no_gpu_only
def test_qk_drift_errors(lib):
    s = shape()
    n = ctypes.c_size_t()
    assert lib.losa_qk_drift_workspace(ctypes.byref(s), ctypes.byref(n)) == OK and n.value > 0

    def drift(Qr=FAKE, Kr=FAKE, tau=0.1, d=FAKE, refresh=FAKE, ws=FAKE, ws_bytes=1 << 40, shp=s):
        return lib.losa_qk_drift(ctypes.byref(shp), FAKE, FAKE, Qr, Kr, tau, d, refresh, ws, ws_bytes, None)

    assert drift(Qr=None) == NULL
    assert drift(Kr=None) == NULL
    assert drift(d=None) == NULL
    assert drift(ws=None) == NULL
    assert drift(Qr=FAKE + 2) == INVALID          # not 16-byte aligned
    assert drift(tau=float("nan")) == INVALID
    assert drift(d=FAKE + 4) == INVALID           # fp64 output not 8-byte aligned
    assert drift(refresh=FAKE + 2) == INVALID
    assert drift(ws_bytes=n.value - 1) == WORKSPACE
    bad = shape()
    bad.q_stride[2] = 100                         # token stride not a multiple of 8 elements
    assert drift(shp=bad) == INVALID


@no_gpu_only
def test_merge_lists_errors(lib):
    s = shape()
    rows, nk = 2 * 16, 16
    n = ctypes.c_size_t()
    assert lib.losa_merge_lists_workspace(ctypes.byref(s), ctypes.byref(n)) == OK
    sel = ctypes.c_size_t()
    assert lib.losa_select_workspace(ctypes.byref(s), ctypes.byref(sel)) == OK and n.value == sel.value

    def merge(take=FAKE, rpa=FAKE, cib=FAKE, rp=FAKE, cap=rows * nk, ws=0x100000, ws_bytes=1 << 40):
        return lib.losa_merge_lists(ctypes.byref(s), take, rpa, FAKE, FAKE, cib, rp, FAKE, cap, None, ws, ws_bytes,
                                    None)

    assert merge(take=None) == NULL
    assert merge(rpa=None) == NULL
    assert merge(cib=None) == NULL
    assert merge(rp=None) == NULL
    assert merge(cap=rows * nk - 1) == CAPACITY
    assert merge(ws=0x100010) == WORKSPACE
    assert merge(ws_bytes=n.value - 1) == WORKSPACE


def test_binding_names_match_header():
    """Every call the header declares has a Python binding of the same name."""
    for n in declared_functions():
        if n != "losa_status_string":
            assert hasattr(F, n), n
    for n in F.__all__:
        assert hasattr(F, n), n


@no_gpu_only
def test_select_threshold_errors(lib):
    s = shape()
    rows, nk = 2 * 16, 16
    n = ctypes.c_size_t()
    assert lib.losa_select_threshold_workspace(ctypes.byref(s), ctypes.byref(n)) == OK and n.value > 0
    t1 = (ctypes.c_double * 1)(0.1)

    def sel(t=t1, n_t=1, cap=rows * nk, ws=0x100000, ws_bytes=1 << 40, M=FAKE):
        return lib.losa_select_threshold(ctypes.byref(s), M, t, n_t, FAKE, FAKE, cap, None, ws, ws_bytes, None)

    assert sel(M=None) == NULL
    assert sel(t=None) == NULL
    assert sel(cap=rows * nk - 1) == CAPACITY
    for bad in (0.0, -0.5, 1.5, float("nan")):
        assert sel(t=(ctypes.c_double * 1)(bad)) == INVALID
    assert sel(n_t=3) == INVALID
    assert sel(t=(ctypes.c_double * 2)(0.1, 0.0), n_t=2) == INVALID
    assert sel(ws=0x100010) == WORKSPACE
    assert sel(ws_bytes=n.value - 1) == WORKSPACE


@no_gpu_only
def test_sparse_attn_threshold_errors(lib):
    s = shape()
    t1 = (ctypes.c_double * 1)(0.1)

    def thr(sh=s, t=t1, n_t=1, ws=0x100000, ws_bytes=1 << 40, O=FAKE, o_dtype=F.LOSA_BF16, cnt=None, mask=None):
        return lib.losa_sparse_attn_threshold(ctypes.byref(sh), FAKE, FAKE, FAKE, t, n_t, O, o_dtype, cnt, mask, ws,
                                              ws_bytes, None)

    assert thr(t=(ctypes.c_double * 1)(0.0)) == INVALID
    assert thr(t=(ctypes.c_double * 1)(1.5)) == INVALID
    assert thr(t=(ctypes.c_double * 2)(0.5, float("nan")), n_t=2) == INVALID
    assert thr(n_t=3) == INVALID
    assert thr(O=None) == NULL
    assert thr(o_dtype=7) == INVALID
    assert thr(cnt=FAKE + 2) == INVALID
    assert thr(ws_bytes=64) == WORKSPACE
    assert thr(ws=0x100010) == WORKSPACE
    assert thr(sh=shape(dtype=F.LOSA_F32)) == UNSUPPORTED
    assert thr(sh=shape(q_block=32)) == UNSUPPORTED
    n = ctypes.c_size_t()
    assert lib.losa_sparse_attn_threshold_workspace(ctypes.byref(s), ctypes.byref(n)) == OK and n.value > 0
