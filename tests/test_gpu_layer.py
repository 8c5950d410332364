"""One-call layer (svg_layer) and the step driver on the GPU.

svg_layer enqueues the same kernels as the separate calls, so its results must equal theirs
bit for bit; one small case is also checked against the oracle end to end.  The step driver
runs dense attention for the first quarter of the steps and profiling + sparse attention
after; its HIP-graph replays must equal eager runs on the same inputs, replay after replay.
"""
import numpy as np
import pytest
import torch

import oracle.svg_oracle as O
from tests.gpu_util import assert_close_attn, host64, note
from workloads import Geometry, Workload, make_qkv, norm_weights, sample_queries

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

LAYER_CASES = [  # name, geometry, (w_f, w_p), norm
    ("d128_norm", Geometry(1, 4, 6, 12, 16, 128), (1, 8), True),
    ("d128_plain", Geometry(1, 4, 5, 9, 11, 128), (1, 5), False),
    ("d64_norm_b2", Geometry(2, 3, 7, 10, 13, 64), (1, 6), True),
]


def _inputs(g, w, seed, norm):
    wl = Workload("layer", g, w[0], w[1], 64, seed, 100 + seed, planted=True)
    q, k, v = make_qkv(wl, device=DEV)
    idx = torch.from_numpy(sample_queries(g.S, 64, 100 + seed)).to(DEV)
    nt = None
    if norm:
        wq, wk = norm_weights(g.D, seed)
        nt = (torch.from_numpy(wq).to(DEV), torch.from_numpy(wk).to(DEV), 1e-6, 10000.0)
    return q, k, v, idx, nt


@pytest.mark.parametrize("case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
@pytest.mark.parametrize("dense", [False, True], ids=["sparse", "dense"])
def test_layer_equals_separate_calls(gpu, case, dense):
    name, g, w, norm = case
    note(f"svg_layer {name} dense={dense}")
    q, k, v, idx, nt = _inputs(g, w, 7, norm)
    o, kind, mse, qa, ka = gpu.layer(q, k, v, idx, g.F, g.HH, g.WW, w[0], w[1], dense=dense, norm=nt)
    # the same stages, one call each
    if norm:
        qr, kr = gpu.qknorm_rope(q, k, nt[0], nt[1], g.F, g.HH, g.WW, nt[2], nt[3])
    else:
        qr, kr = q, k
    if dense:
        o_ref = gpu.dense_attn(qr, kr, v, g.F, g.HH, g.WW)
    else:
        mse_ref, kind_ref = gpu.profile_heads(qr, kr, v, idx, g.F, g.HH, g.WW, w[0], w[1])
        o_ref, _ = gpu.sparse_attn(qr, kr, v, None, None, None, kind_ref, g.F, g.HH, g.WW, w[0], w[1])
    torch.cuda.synchronize()
    assert torch.equal(qa, qr) and torch.equal(ka, kr)
    assert torch.equal(o, o_ref)
    if not dense:
        assert torch.equal(kind, kind_ref) and torch.equal(mse, mse_ref)


def test_layer_vs_oracle(gpu):
    g, w = Geometry(1, 4, 4, 8, 10, 64), (1, 3)
    note("svg_layer vs oracle, 4 heads, S=320")
    q, k, v, idx, nt = _inputs(g, w, 11, True)
    o, kind, mse, qn, kn = gpu.layer(q, k, v, idx, g.F, g.HH, g.WW, w[0], w[1], norm=nt)
    torch.cuda.synchronize()
    wq, wk = norm_weights(g.D, 11)
    qo, ko = O.qknorm_rope(host64(q), host64(k), wq, wk, 1e-6, g.F, g.HH, g.WW, 10000.0)
    assert np.abs(host64(qn) - qo).max() < 0.05 and np.abs(host64(kn) - ko).max() < 0.05
    sc = O.default_scale(g.D)
    idx_h = idx.cpu().numpy()
    mse_o, kind_o = O.profile_heads(host64(qn), host64(kn), host64(v), idx_h, g.F, g.P, w[0], w[1], sc)
    kind_g = kind.cpu().numpy()
    assert O.choices_agree(kind_g, kind_o, mse_o).all(), (kind_g, kind_o)
    want = O.sparse_attention(host64(qn), host64(kn), host64(v), kind_g, g.F, g.P, w[0], w[1], sc)
    assert_close_attn(host64(o), want, "svg_layer")


@pytest.mark.parametrize("norm", [True, False], ids=["norm", "plain"])
def test_step_driver_graph_replays_equal_eager(gpu, norm):
    g, w = Geometry(1, 4, 6, 12, 16, 128), (1, 8)
    n_steps, n_layers = 4, 2
    note(f"step driver, graphs vs eager, norm={norm}")
    nt = _inputs(g, w, 3, norm)[4]
    mk = lambda graphs: gpu.StepDriver(g.B, g.H, g.F, g.HH, g.WW, g.D, n_steps, w[0], w[1], norm=nt, graphs=graphs,
                                       device=DEV)
    eager, graphed = mk(False), mk(True)
    assert [eager.is_dense(s) for s in range(n_steps)] == [True, False, False, False]
    for step in range(n_steps):
        for lay in range(n_layers):
            q, k, v, idx, _ = _inputs(g, w, 20 + step * n_layers + lay, False)
            for d in (eager, graphed):
                d.q.copy_(q)
                d.k.copy_(k)
                d.v.copy_(v)
                d.q_idx.copy_(idx)
            o_e, kind_e, mse_e = eager.layer(step)
            torch.cuda.synchronize()
            o_g, kind_g, mse_g = graphed.layer(step)
            torch.cuda.synchronize()
            assert torch.equal(o_g, o_e), (step, lay)
            if not eager.is_dense(step):
                assert torch.equal(kind_g, kind_e) and torch.equal(mse_g, mse_e), (step, lay)
    assert set(graphed._graph) == {True, False}
