"""Two independent layers processed at the same time on two streams.

The library keeps no state between calls, so calls with separate buffers on
different streams may overlap: masses, selection, sparse attention, the
masses within the lists and the drift of two layers are enqueued alternately
on two streams (default priority) and each result must equal, bit for bit,
the same calls run alone on one stream.
"""
import numpy as np
import pytest
import torch

import synthetic as S
from tests.gpu_util import say, to_device

pytestmark = pytest.mark.gpu

import free_block_sparse_exact_amd as F  # noqa: E402


def _layer(seed, H, N, Na, d):
    rng = np.random.default_rng(seed)
    return [to_device(S.bf16_bits_from_f32((rng.standard_normal((1, H, Na, d)) * s).astype(np.float32)), "bf16")
            for s in (1.5, 1.5, 1.0)]


class Path:
    def __init__(self, q, k, v, N, R, C, p):
        self.q, self.k, self.v, self.N, self.R, self.C, self.p = q, k, v, N, R, C, p
        g = F.Geometry.of(q, N, R, C)
        self.g = g
        u8 = dict(dtype=torch.uint8, device=q.device)
        self.M = torch.empty((1, g.heads, g.n_q, g.n_k), dtype=torch.float32, device=q.device)
        self.ws_mass = torch.empty(F.losa_block_mass_workspace(g), **u8)
        self.rp = torch.empty(g.rows + 1, dtype=torch.int32, device=q.device)
        self.ci = torch.empty(g.rows * g.n_k, dtype=torch.int32, device=q.device)
        self.order = torch.empty(g.rows, dtype=torch.int32, device=q.device)
        self.ws_sel = torch.empty(F.losa_select_workspace(g), **u8)
        self.O = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        self.ws_attn = torch.empty(F.losa_sparse_attn_workspace(g), **u8)
        self.O2 = torch.empty_like(self.O)
        self.Ml = torch.empty_like(self.M)
        self.ws_sm = torch.empty(F.losa_sparse_attn_mass_workspace(g), **u8)
        self.drift = torch.empty((1, g.heads, 2), dtype=torch.float64, device=q.device)
        self.ws_d = torch.empty(F.losa_qk_drift_workspace(g), **u8)

    def calls(self, st):
        N, R, C = self.N, self.R, self.C
        yield lambda: F.losa_block_mass(self.q, self.k, N, R, C, out=self.M, ws=self.ws_mass, stream=st)
        yield lambda: F.losa_select(self.M, self.p, N, R, C, tokens_alloc=self.g.tokens_alloc, row_ptr=self.rp,
                                    col_idx=self.ci, order=self.order, ws=self.ws_sel, stream=st)
        yield lambda: F.losa_sparse_attn(self.q, self.k, self.v, self.rp, self.ci, self.order, N, R, C, out=self.O,
                                         ws=self.ws_attn, stream=st)
        yield lambda: F.losa_sparse_attn_mass(self.q, self.k, self.v, self.rp, self.ci, self.order, N, R, C,
                                              out=self.O2, M=self.Ml, ws=self.ws_sm, stream=st)
        yield lambda: F.losa_qk_drift(self.q, self.k, self.v, self.q, N, 0.5, R, C, drift=self.drift,
                                      refresh=None, ws=self.ws_d, stream=st)

    def results(self):
        nnz = int(self.rp[-1].item())
        return [t.cpu().clone() for t in (self.M, self.rp, self.ci[:nnz], self.order, self.O, self.O2, self.Ml,
                                          self.drift)]


def test_two_streams_match_one():
    H, d, p = 4, 128, 0.95
    A = Path(*_layer(11, H, 2000, 2048, d), 2000, 64, 64, p)
    B = Path(*_layer(12, H, 1500, 1536, d), 1500, 128, 32, p)
    cur = torch.cuda.current_stream()
    for path in (A, B):
        for call in path.calls(cur):
            call()
    torch.cuda.synchronize()
    alone = [A.results(), B.results()]
    for t in (A.M, B.M, A.O, B.O, A.O2, B.O2, A.Ml, B.Ml, A.drift, B.drift):
        t.fill_(float("nan"))
    for t in (A.rp, B.rp, A.ci, B.ci, A.order, B.order):
        t.fill_(-1)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for ca, cb in zip(A.calls(sa), B.calls(sb)):  # interleaved enqueue: the streams overlap
        ca()
        cb()
    torch.cuda.synchronize()
    for got, ref in zip((A.results(), B.results()), alone):
        for x, y in zip(got, ref):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    say("two layers on two streams: every output identical to the one-stream run")


def test_side_stream_with_library_allocated_buffers():
    """Only stream= given: the binding allocates every workspace and output
    itself, on that stream (so the caching allocator cannot hand a buffer
    freed at return to other work while the side stream still uses it).
    Meanwhile torch's current stream allocates and writes buffers of the same
    sizes.  The results equal the same calls on the current stream."""
    H, d, p, N, R, C = 4, 128, 0.95, 2000, 64, 64
    q, k, v = _layer(13, H, N, 2048, d)
    cur = torch.cuda.current_stream()
    M0 = F.losa_block_mass(q, k, N, R, C)
    rp0, ci0, or0 = F.losa_select(M0, p, N, R, C)
    O0 = F.losa_sparse_attn(q, k, v, rp0, ci0, or0, N, R, C, out_dtype=torch.float32)
    Od0, Md0 = F.losa_dense_attn_mass(q, k, v, N, R, C, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = [t.cpu() for t in (M0, rp0, or0, O0, Od0, Md0)]
    nnz = int(rp0[-1].item())
    ref.append(ci0[:nnz].cpu())
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    for rep in range(3):
        M = F.losa_block_mass(q, k, N, R, C, stream=side)
        rp, ci, order = F.losa_select(M, p, N, R, C, stream=side)
        O = F.losa_sparse_attn(q, k, v, rp, ci, order, N, R, C, out_dtype=torch.float32, stream=side)
        Od, Md = F.losa_dense_attn_mass(q, k, v, N, R, C, out_dtype=torch.float32, stream=side)
        # the current stream meanwhile takes and scribbles over fresh memory
        junk = [torch.full((n,), 249, dtype=torch.uint8, device=q.device) for n in (M0.numel() * 4, 1 << 24)]
        del junk
        side.synchronize()
        got = [t.cpu() for t in (M, rp, order, O, Od, Md)] + [ci[:nnz].cpu()]
        for x, y in zip(got, ref):
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    torch.cuda.synchronize()
    say("calls on a side stream with library-allocated buffers: identical to the current-stream run")
