"""The whole path captured in a HIP graph and replayed.

The calls allocate nothing, clear nothing with memset and keep no state, so a
caller can capture a step -- block masses, selection with its work order,
sparse attention on the new lists, the masses within them, the query-key
drift and the list merge -- in one graph.  Each replay is checked bit for bit
against the same calls run eagerly on the same inputs, with eager work that
overwrites every workspace and output between replays, and with the input
buffers refilled with new contents between replays (the graph reads the
buffers, not the values they held at capture).
"""
import numpy as np
import pytest
import torch

import synthetic as S
from tests.gpu_util import say, to_device

pytestmark = pytest.mark.gpu

import free_block_sparse_exact_amd as F  # noqa: E402


class Step:
    """Every buffer of one step, allocated once; run() enqueues the calls."""

    def __init__(self, q, k, v, N, R, C, p):
        self.q, self.k, self.v, self.N, self.R, self.C, self.p = q, k, v, N, R, C, p
        g = F.Geometry.of(q, N, R, C)
        self.g = g
        dev = q.device
        u8 = dict(dtype=torch.uint8, device=dev)
        self.M = torch.empty((g.batch, g.heads, g.n_q, g.n_k), dtype=torch.float32, device=dev)
        self.ws_mass = torch.empty(F.losa_block_mass_workspace(g), **u8)
        self.rp = torch.empty(g.rows + 1, dtype=torch.int32, device=dev)
        self.ci = torch.empty(g.rows * g.n_k, dtype=torch.int32, device=dev)
        self.order = torch.empty(g.rows, dtype=torch.int32, device=dev)
        self.ws_sel = torch.empty(F.losa_select_workspace(g), **u8)
        self.O = torch.empty(q.shape, dtype=torch.float32, device=dev)
        self.ws_attn = torch.empty(max(F.losa_sparse_attn_workspace(g), 1), **u8)
        self.O2 = torch.empty_like(self.O)
        self.Ml = torch.empty_like(self.M)
        self.ws_sm = torch.empty(F.losa_sparse_attn_mass_workspace(g), **u8)
        self.q_ref, self.k_ref = q.clone(), k.clone()
        self.drift = torch.empty((g.batch, g.heads, 2), dtype=torch.float64, device=dev)
        self.flags = torch.empty((g.batch, g.heads), dtype=torch.int32, device=dev)
        self.ws_drift = torch.empty(F.losa_qk_drift_workspace(g), **u8)
        self.rp2 = torch.empty_like(self.rp)
        self.ci2 = torch.empty_like(self.ci)
        self.order2 = torch.empty_like(self.order)

    def run(self, stream=None):
        N, R, C = self.N, self.R, self.C
        F.losa_block_mass(self.q, self.k, N, R, C, out=self.M, ws=self.ws_mass, stream=stream)
        F.losa_select(self.M, self.p, N, R, C, tokens_alloc=self.g.tokens_alloc, row_ptr=self.rp, col_idx=self.ci,
                      order=self.order, ws=self.ws_sel, stream=stream)
        F.losa_sparse_attn(self.q, self.k, self.v, self.rp, self.ci, self.order, N, R, C, out=self.O,
                           ws=self.ws_attn, stream=stream)
        F.losa_sparse_attn_mass(self.q, self.k, self.v, self.rp, self.ci, self.order, N, R, C, out=self.O2,
                                M=self.Ml, ws=self.ws_sm, stream=stream)
        F.losa_qk_drift(self.q, self.k, self.q_ref, self.k_ref, N, 0.1, R, C, drift=self.drift,
                        refresh=self.flags, ws=self.ws_drift, stream=stream)
        F.losa_merge_lists(self.flags, self.rp, self.ci, self.rp, self.ci, N, R, C,
                           tokens_alloc=self.g.tokens_alloc, row_ptr=self.rp2, col_idx=self.ci2, order=self.order2,
                           ws=self.ws_sel, stream=stream)

    def outputs(self):
        nnz = int(self.rp[-1].item())
        return [t.cpu().clone() for t in (self.M, self.rp, self.ci[:nnz], self.order, self.O, self.O2, self.Ml,
                                          self.drift, self.flags, self.rp2, self.ci2[:nnz], self.order2)]

    def scribble(self):
        """Eager work that overwrites every workspace and output."""
        for t in (self.M, self.O, self.O2, self.Ml, self.drift):
            t.fill_(float("nan"))
        for t in (self.rp, self.ci, self.order, self.flags, self.rp2, self.ci2, self.order2):
            t.fill_(-7)
        for t in (self.ws_mass, self.ws_sel, self.ws_attn, self.ws_sm, self.ws_drift):
            t.fill_(0xA5)


def _same(a, b):
    for x, y in zip(a, b):
        assert x.dtype == y.dtype and x.shape == y.shape
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.bool else x, y.view(torch.uint8)
                           if y.dtype != torch.bool else y)


def _inputs(seed, H, N, Na, d):
    rng = np.random.default_rng(seed)
    return [S.bf16_bits_from_f32((rng.standard_normal((1, H, Na, d)) * s).astype(np.float32))
            for s in (1.5, 1.5, 1.0)]


@pytest.mark.parametrize("R,C", [(64, 64), (128, 32)])
def test_graph_replay_matches_eager(R, C):
    H, N, d, p = 3, 1000, 128, 0.95
    Na = max(-(-N // R) * R, -(-N // C) * C)
    q, k, v = (to_device(b, "bf16") for b in _inputs(1, H, N, Na, d))
    st = Step(q, k, v, N, R, C, p)
    # the drift reference: a perturbed copy, so some heads are flagged
    st.q_ref.copy_(q)
    st.q_ref[0, 1].mul_(1.5)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()            # warm-up on the capture stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = st.outputs()
    assert eager[8].numpy().tolist() == [[0, 1, 0]]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.run()
    torch.cuda.synchronize()
    for rep in range(3):
        st.scribble()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(st.outputs(), eager)
        say(f"R={R} C={C}: replay {rep} identical to the eager step")
    # new contents in the same input buffers: the replay follows them
    q2, k2, v2 = (to_device(b, "bf16") for b in _inputs(2, H, N, Na, d))
    st.q.copy_(q2)
    st.k.copy_(k2)
    st.v.copy_(v2)
    st.run()
    torch.cuda.synchronize()
    eager2 = st.outputs()
    assert not torch.equal(eager2[4], eager[4])
    for rep in range(2):
        st.scribble()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(st.outputs(), eager2)
    say(f"R={R} C={C}: replays on new inputs identical to the eager step")
