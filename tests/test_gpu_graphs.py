"""HIP-graph capture of the clustering and block-sparse layers.

None of their calls allocates, synchronises or records a memset, so a layer can be captured
once and replayed.  Each replay, with fresh inputs copied into the captured buffers and eager
work and synchronisation in between, must equal the same calls run eagerly from the same state,
bit for bit.
"""
import pytest
import torch

from tests.gpu_util import note
from workloads import SEMANTIC_WORKLOADS, Geometry, Workload, init_token_indices, make_qkv, make_qkv_semantic

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # one eager run on the capture stream first
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_cluster_layer_graph_replays_equal_eager(gpu):
    wl = SEMANTIC_WORKLOADS["svg2_small"]
    g = wl.geom
    note("cluster layer graph replays")
    q, k, v = make_qkv_semantic(wl, device=DEV, step=0)
    iq = torch.from_numpy(init_token_indices(g.S, wl.Cq, wl.seed)).to(DEV)
    ik = torch.from_numpy(init_token_indices(g.S, wl.Ck, wl.seed + 1)).to(DEV)
    mk = lambda: gpu.ClusterLayer(q, g.F, g.HH, g.WW, wl.Cq, wl.Ck, wl.p, wl.iters, iq, ik)
    eager, graphed = mk(), mk()
    xq, xk, xv = q.clone(), k.clone(), v.clone()        # the graphed layer's static inputs
    eager(q, k, v)
    graphed(xq, xk, xv)                                   # both cold-started on step 0
    torch.cuda.synchronize()
    state = [t.clone() for t in (graphed.cq.centroids, graphed.ck.centroids)]
    graph = _capture(lambda: graphed(xq, xk, xv))
    # the capture's eager warm-up advanced the graphed layer's cache: restore it
    graphed.cq.centroids.copy_(state[0])
    graphed.ck.centroids.copy_(state[1])
    for step in range(1, 4):
        q, k, v = make_qkv_semantic(wl, device=DEV, step=step)
        xq.copy_(q)
        xk.copy_(k)
        xv.copy_(v)
        graph.replay()
        torch.cuda.synchronize()
        o_e = eager(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(graphed.o, o_e), step
        for a, b in ((graphed.cq, eager.cq), (graphed.ck, eager.ck)):
            for t in ("centroids", "labels", "perm", "offsets"):
                assert torch.equal(getattr(a, t), getattr(b, t)), (step, t)
        assert torch.equal(graphed.sel, eager.sel), step


def test_block_layer_graph_replays_equal_eager(gpu):
    g = Geometry(1, 2, 4, 12, 16, 128)
    wl = Workload("blocks_graph", g, 1, 3, 64, 46, 146, planted=True)
    note("block layer graph replays")
    q0, k0, v0 = make_qkv(wl, device=DEV)
    _, lse = gpu.dense_attn_lse(q0, k0, v0, g.F, g.HH, g.WW)
    nqb, nkb = gpu.block_grid(g.S)
    xq, xk, xv = (torch.empty_like(q0) for _ in range(3))
    mass = torch.empty((1, g.H, nqb, nkb), dtype=torch.float32, device=DEV)
    sel = torch.empty((1, g.H, nqb, nkb), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q0)
    ws = torch.empty(max(256, gpu.workspace_bytes(gpu.OP_BLOCK_ATTN, gpu.geometry(q0, g.F, g.HH, g.WW))),
                     dtype=torch.uint8, device=DEV)

    def layer():
        gpu.block_mass(xq, xk, lse, g.F, g.HH, g.WW, mass=mass)
        gpu.block_select(mass, g.F, g.HH, g.WW, g.D, 0.9, sel=sel)
        gpu.block_sparse_attn(xq, xk, xv, sel, g.F, g.HH, g.WW, o=o, ws=ws)

    xq.copy_(q0)
    xk.copy_(k0)
    xv.copy_(v0)
    graph = _capture(layer)
    for step in range(1, 4):
        q, k, v = make_qkv(wl, device=DEV, step=step)
        xq.copy_(q)
        xk.copy_(k)
        xv.copy_(v)
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_sel, got_m = o.clone(), sel.clone(), mass.clone()
        m_e = gpu.block_mass(q, k, lse, g.F, g.HH, g.WW)
        s_e = gpu.block_select(m_e, g.F, g.HH, g.WW, g.D, 0.9)
        o_e = gpu.block_sparse_attn(q, k, v, s_e, g.F, g.HH, g.WW)
        torch.cuda.synchronize()
        assert torch.equal(got_m, m_e) and torch.equal(got_sel, s_e) and torch.equal(got_o, o_e), step
