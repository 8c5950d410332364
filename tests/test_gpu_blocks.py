"""GPU parity of the head-adaptive block-sparse path (svg_dense_attn_lse, svg_block_mass,
svg_block_select, svg_block_sparse_attn) against the fp64 oracle of oracle/adaspa_oracle.py.

The block choice is a decision taken on floating-point masses: the GPU's choice is accepted
when it is the oracle's choice on the GPU's own masses, or a near tie of it; attention is then
checked given the GPU's choice, so a near tie never cascades.
"""
import numpy as np
import pytest
import torch

import oracle.adaspa_oracle as A
import oracle.svg_oracle as O
from tests.gpu_util import assert_close_attn, host64, note
from workloads import Geometry, Workload, make_qkv

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# The LSE comes from the running max and the row sum of bf16-rounded weights (each within 2^-8
# relative, half a bf16 step), so it may differ from the exact one by up to about 2^-8.
LSE_TOL = 4.5e-3
# Masses: fp32 sums of exponentials of fp32-accumulated bf16 products; each is checked to a
# relative 1e-4 plus 1e-7 of its block row's total.
MASS_RTOL = 1e-4
MASS_ATOL_ROW = 1e-7
COVER_TIE = 1e-6

CASES = [
    # name, geometry, planted, coverage
    ("d128_planted", Geometry(1, 2, 4, 12, 16, 128), True, 0.9),
    ("d64_ragged", Geometry(1, 2, 3, 13, 19, 64), False, 0.8),     # S = 741: ragged in both block sizes
    ("d128_b2_small", Geometry(2, 2, 2, 9, 11, 128), True, 0.95),   # S = 198 < one query block
    ("d64_cover1", Geometry(1, 3, 5, 10, 11, 64), True, 1.0),
]


def _inputs(g, planted, seed):
    wl = Workload("blocks", g, 1, 3, 64, seed, 100 + seed, planted=planted)
    return make_qkv(wl, device=DEV)


def _check_mass(got, want, what):
    tol = MASS_RTOL * np.abs(want) + MASS_ATOL_ROW * want.sum(axis=1, keepdims=True)
    assert (np.abs(got - want) <= tol).all(), f"{what}: worst {np.abs(got - want).max():.3e}"


def _check_selection(M, sel, cov, what):
    """sel [nqb, nkb] of the GPU against the oracle's choice on the same masses M (fp64)."""
    want = A.select_blocks(M, cov)
    rows = np.flatnonzero((sel != want).any(axis=1))
    for i in rows:
        s = sel[i].astype(bool)
        tot = M[i].sum()
        assert s.any() and (M[i, s] > 0).all(), f"{what}: row {i} chooses nothing or a zero block"
        assert M[i, s].min() >= M[i, ~s].max(initial=0.0) - COVER_TIE * tot, f"{what}: row {i} is not a prefix"
        assert M[i, s].sum() >= cov * tot - COVER_TIE * tot, f"{what}: row {i} falls short of the coverage"
        assert M[i, s].sum() - M[i, s].min() < cov * tot + COVER_TIE * tot or s.sum() == 1, \
            f"{what}: row {i} is not minimal"
    assert len(rows) <= max(1, sel.shape[0] // 10), f"{what}: {len(rows)} near-tie rows"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_lse_mass_select_attention(gpu, case):
    name, g, planted, cov = case
    note(f"block path {name}")
    q, k, v = _inputs(g, planted, 41)
    o_d, lse = gpu.dense_attn_lse(q, k, v, g.F, g.HH, g.WW)
    o_ref = gpu.dense_attn(q, k, v, g.F, g.HH, g.WW)
    mass = gpu.block_mass(q, k, lse, g.F, g.HH, g.WW)
    sel = gpu.block_select(mass, g.F, g.HH, g.WW, g.D, cov)
    o = gpu.block_sparse_attn(q, k, v, sel, g.F, g.HH, g.WW)
    torch.cuda.synchronize()
    assert torch.equal(o_d, o_ref), "dense attention with lse differs from svg_dense_attn"
    sc = O.default_scale(g.D)
    qh, kh, vh, oh = host64(q), host64(k), host64(v), host64(o)
    lh, mh = host64(lse), host64(mass)
    nqb, nkb = gpu.block_grid(g.S)
    heights = np.minimum(A.BQ, g.S - A.BQ * np.arange(nqb))
    for b in range(g.B):
        for h in range(g.H):
            what = f"{name} b{b} h{h}"
            want_lse = A.row_lse(qh[b, h], kh[b, h], sc)
            assert np.abs(lh[b, h] - want_lse).max() <= LSE_TOL, f"{what}: lse"
            # masses of the GPU's lse, against the oracle given that lse
            want_m = A.block_mass(qh[b, h], kh[b, h], lh[b, h], sc)
            _check_mass(mh[b, h], want_m, f"{what}: mass")
            # with the lse of the same inputs a block row holds its row count
            assert np.abs(mh[b, h].sum(axis=1) / heights - 1).max() < 5e-3, f"{what}: row sums"
            s = sel[b, h].cpu().numpy()
            _check_selection(mh[b, h], s, cov, what)
            want = A.block_sparse_attention(qh[b, h], kh[b, h], vh[b, h], s.astype(bool), sc)
            assert_close_attn(oh[b, h], want, what)


@pytest.mark.parametrize("D", [64, 128])
def test_all_blocks_is_dense(gpu, D):
    """Every block chosen: the key list is every key in order, the dense kernel's schedule, so
    the output equals svg_dense_attn bit for bit."""
    g = Geometry(1, 2, 3, 11, 13, D)
    note(f"all blocks, D={D}")
    q, k, v = _inputs(g, False, 42)
    nqb, nkb = gpu.block_grid(g.S)
    sel = torch.ones((g.B, g.H, nqb, nkb), dtype=torch.uint8, device=DEV)
    o = gpu.block_sparse_attn(q, k, v, sel, g.F, g.HH, g.WW)
    od = gpu.dense_attn(q, k, v, g.F, g.HH, g.WW)
    torch.cuda.synchronize()
    assert torch.equal(o, od)


def test_hand_block_mask(gpu):
    """A fixed mask with empty-but-one rows, the partial last key block and a diagonal."""
    g = Geometry(1, 1, 2, 10, 31, 64)          # S = 620: 3 query blocks, 10 key blocks (last has 44 keys)
    note("hand block mask")
    q, k, v = _inputs(g, False, 43)
    nqb, nkb = gpu.block_grid(g.S)
    m = np.zeros((nqb, nkb), dtype=np.uint8)
    m[0, 9] = 1                                  # only the partial block
    m[1, [0, 4, 9]] = 1
    m[2, :] = 1
    sel = torch.from_numpy(m).view(1, 1, nqb, nkb).to(DEV)
    o = gpu.block_sparse_attn(q, k, v, sel, g.F, g.HH, g.WW)
    torch.cuda.synchronize()
    want = A.block_sparse_attention(host64(q)[0, 0], host64(k)[0, 0], host64(v)[0, 0], m.astype(bool),
                                    O.default_scale(g.D))
    assert_close_attn(host64(o)[0, 0], want, "hand mask")


def test_stale_lse_from_another_step(gpu):
    """The search with the LSE of different inputs (an earlier step): masses scale by the LSE
    offset, and the GPU masses still match the oracle given that LSE."""
    g = Geometry(1, 2, 4, 12, 16, 128)
    note("stale lse")
    q0, k0, v0 = _inputs(g, True, 44)
    q1, k1, _ = _inputs(g, True, 45)
    _, lse0 = gpu.dense_attn_lse(q0, k0, v0, g.F, g.HH, g.WW)
    mass = gpu.block_mass(q1, k1, lse0, g.F, g.HH, g.WW)
    torch.cuda.synchronize()
    sc = O.default_scale(g.D)
    for h in range(g.H):
        want = A.block_mass(host64(q1)[0, h], host64(k1)[0, h], host64(lse0)[0, h], sc)
        got = host64(mass)[0, h]
        _check_mass(got, want, f"h{h}")


def test_720p_sampled(gpu):
    """The 720p planted layer as the benchmark runs it: lse and outputs on sampled rows, masses
    of sampled query blocks, and every selection row of three heads."""
    wl = Workload("hunyuan720p", Geometry(1, 24, 33, 45, 80, 128), 1, 64, 64, 4, 104, planted=True)
    g = wl.geom
    note("720p block path, sampled parity")
    q, k, v = make_qkv(wl, device=DEV)
    _, lse = gpu.dense_attn_lse(q, k, v, g.F, g.HH, g.WW)
    mass = gpu.block_mass(q, k, lse, g.F, g.HH, g.WW)
    sel = gpu.block_select(mass, g.F, g.HH, g.WW, g.D, 0.9)
    o = gpu.block_sparse_attn(q, k, v, sel, g.F, g.HH, g.WW)
    torch.cuda.synchronize()
    sc = O.default_scale(g.D)
    rng = np.random.default_rng(7)
    nqb, nkb = gpu.block_grid(g.S)
    dens = []
    for h in (0, 11, 23):
        what = f"720p h{h}"
        qh, kh, vh = host64(q[0, h]), host64(k[0, h]), host64(v[0, h])
        rows = np.sort(rng.choice(g.S, 256, replace=False))
        lh = host64(lse[0, h])
        assert np.abs(lh[rows] - A.row_lse(qh[rows], kh, sc)).max() <= LSE_TOL, what
        blocks = [0, int(rng.integers(1, nqb - 1)), nqb - 1]
        want_m = A.block_mass(qh, kh, lh, sc, q_blocks=blocks)
        mh = host64(mass[0, h])
        _check_mass(mh[blocks], want_m[blocks], what)
        s = sel[0, h].cpu().numpy()
        _check_selection(mh, s, 0.9, what)
        dens.append(float((s.astype(np.float64).sum(axis=1) * 64).mean() / g.S))
        want = A.block_sparse_attention_rows(qh, kh, vh, s.astype(bool), rows, sc)
        assert_close_attn(host64(o[0, h][torch.from_numpy(rows).to(DEV)]), want, what)
    note(f"720p block density (3 heads) {np.round(dens, 4).tolist()}")
