"""svg_layer_noalloc (static per-device scratch, no workspace) against svg_layer (caller's
workspace) on the same inputs: two sparse layers in a row, the second smaller, then a dense
layer.  The kernels are the same, so kinds, errors and outputs must agree bit for bit."""
import numpy as np
import pytest
import torch

from tests.gpu_util import MAX_ABS, REL_L2, note
from workloads import Geometry, Workload, make_qkv, norm_weights, sample_queries

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CALLS = [  # name, geometry, w_p, n_q, with norm, dense
    ("large_d128_norm", Geometry(1, 4, 6, 12, 16, 128), 5, 64, True, False),
    ("small_d64", Geometry(1, 3, 3, 8, 10, 64), 2, 17, False, False),
    ("dense_d128", Geometry(1, 2, 2, 8, 9, 128), 2, 64, True, True),
]


def test_layer_noalloc_matches_layer(gpu):
    svg = gpu
    for i, (name, g, w_p, n_q, with_norm, dense) in enumerate(CALLS):
        note(f"svg_layer_noalloc call {i}: {name} {g}")
        wl = Workload(name, g, 1, w_p, n_q, 70 + i, 170 + i, planted=not dense)
        q, k, v = make_qkv(wl, device=DEV)
        idx = torch.from_numpy(sample_queries(g.S, n_q, wl.idx_seed)).to(DEV)
        norm = None
        if with_norm:
            wq, wk = norm_weights(g.D, wl.seed)
            norm = (torch.from_numpy(wq).to(DEV), torch.from_numpy(wk).to(DEV), 1e-6, 10000.0)
        got = svg.layer_noalloc(q, k, v, idx, g.F, g.HH, g.WW, 1, w_p, dense=dense, norm=norm)
        want = svg.layer(q, k, v, idx, g.F, g.HH, g.WW, 1, w_p, dense=dense, norm=norm)
        torch.cuda.synchronize()
        o, kind, mse, qn, kn = got
        o2, kind2, mse2, qn2, kn2 = want
        if not dense:
            assert torch.equal(kind, kind2), (name, kind, kind2)
            assert torch.equal(mse, mse2), (name, mse, mse2)
        if norm is not None:
            assert torch.equal(qn, qn2) and torch.equal(kn, kn2)
        a, b = o.double().cpu().numpy(), o2.double().cpu().numpy()
        assert np.isfinite(a).all()
        err = np.abs(a - b).max()
        rel = np.linalg.norm(a - b) / np.linalg.norm(b)
        assert err <= MAX_ABS and rel <= REL_L2, (name, err, rel)
        assert torch.equal(o, o2), name
