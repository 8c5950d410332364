"""GPU parity of the semantic clustering path (svg_kmeans, svg_centroid_topp, svg_cluster_attn)
against the fp64 oracle of oracle/svg2_oracle.py.

Where floating point picks an integer (a row's nearest centroid, the cut of a top-p prefix), the
GPU's choice is accepted when it is the oracle's or within the rounding of the GPU's arithmetic
of it (a near tie); everything downstream is then checked given the GPU's choices, so a near tie
never cascades.  Integer outputs (permutation, offsets) are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle.svg2_oracle as O2
from tests.gpu_util import assert_close_attn, host64, note
from workloads import (SEMANTIC_WORKLOADS, Geometry, SemanticWorkload, init_token_indices, make_qkv_semantic,
                       semantic_classes)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# The assignment keeps the larger of x.c - |c|^2/2 in fp32 from bf16 products; a row may pick
# another centroid only if the two squared distances agree to this fraction of their scale.
ASSIGN_TIE = 2e-5
# Top-p shares are fp64 on both sides; only sums and exponentials round differently.
SHARE_TIE = 1e-10


def _semantic(name, geom, n_classes, Cq, Ck, p, iters, seed):
    return SemanticWorkload(name, geom, n_classes, 0.8, Cq, Ck, p, iters, seed, region=3, frames_per_draw=2)


CASES = [
    # name, workload
    ("d64_small", _semantic("d64_small", Geometry(1, 2, 4, 8, 10, 64), 4, 8, 16, 0.9, 3, 31)),
    ("d128_ragged", _semantic("d128_ragged", Geometry(1, 2, 5, 9, 13, 128), 5, 12, 40, 0.9, 3, 32)),
    ("d128_b2_many_clusters", _semantic("d128_b2", Geometry(2, 2, 3, 11, 17, 128), 3, 20, 100, 0.8, 2, 33)),
    ("d64_p1", _semantic("d64_p1", Geometry(1, 3, 4, 7, 9, 64), 4, 6, 20, 1.0, 2, 34)),
]


def _inputs(wl):
    q, k, v = make_qkv_semantic(wl, device=DEV)
    g = wl.geom
    iq = torch.from_numpy(init_token_indices(g.S, wl.Cq, wl.seed)).to(DEV)
    ik = torch.from_numpy(init_token_indices(g.S, wl.Ck, wl.seed + 1)).to(DEV)
    return q, k, v, iq, ik


def _check_assignment(x64, cent, labels, what):
    """labels [S] of the GPU against the oracle's nearest (bf16-rounded) centroids of cent."""
    want = O2.kmeans_assign(x64, cent)
    diff = np.flatnonzero(labels != want)
    if len(diff):
        cb = O2.round_bf16_from_f32(cent)
        xr = x64[diff]
        d_got = ((xr - cb[labels[diff]]) ** 2).sum(axis=1)
        d_want = ((xr - cb[want[diff]]) ** 2).sum(axis=1)
        scale = (xr ** 2).sum(axis=1) + (cb ** 2).sum(axis=1).max()
        bad = d_got - d_want > ASSIGN_TIE * scale
        assert not bad.any(), f"{what}: {bad.sum()} rows not at their nearest centroid"
    assert len(diff) <= max(2, len(labels) // 200), f"{what}: {len(diff)} near ties of {len(labels)} rows"


def _check_sort(labels, perm, offsets, C, what):
    p_want, o_want = O2.cluster_permutation(labels, C)
    assert np.array_equal(offsets, o_want), f"{what}: offsets"
    assert np.array_equal(perm, p_want), f"{what}: permutation"


def _check_update(x64, labels, cent_before, cent_after, what):
    want, _ = O2.kmeans_update(x64, labels, cent_before)
    want = O2.round_f32(want)
    got = cent_after.astype(np.float64)
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert (np.abs(got - want) <= ulp).all(), f"{what}: centroid means off by more than 1 fp32 ulp"


def _check_topp(w, sel, p, what):
    """GPU selection sel [Cq, Ck] against shares w: a valid top-p prefix for every row."""
    want = O2.topp_select(w, p)
    rows = np.flatnonzero((sel != want).any(axis=1))
    for i in rows:
        s = sel[i].astype(bool)
        assert s.any() and (w[i, s] > 0).all(), f"{what}: row {i} selects nothing or a zero share"
        assert w[i, s].min() >= w[i, ~s].max(initial=0.0) - SHARE_TIE, f"{what}: row {i} is not a prefix"
        tot = w[i, s].sum()
        assert tot >= p - SHARE_TIE, f"{what}: row {i} falls short of p"
        assert tot - w[i, s].min() < p + SHARE_TIE or s.sum() == 1, f"{what}: row {i} is not minimal"
    assert len(rows) <= max(1, sel.shape[0] // 20), f"{what}: {len(rows)} near-tie rows"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_kmeans_first_iteration(gpu, case):
    name, wl = case
    g = wl.geom
    note(f"kmeans 1 iteration {name}")
    q, k, v, iq, ik = _inputs(wl)
    for x, init, C, tag in ((q, iq, wl.Cq, "Q"), (k, ik, wl.Ck, "K")):
        cl = gpu.kmeans(x, g.F, g.HH, g.WW, C, 1, init_idx=init)
        torch.cuda.synchronize()
        xh = host64(x)
        idx = init.cpu().numpy()
        for b in range(g.B):
            for h in range(g.H):
                what = f"{name} {tag} b{b} h{h}"
                x64 = xh[b, h]
                cent0 = O2.init_centroids(x64, idx)
                lab = cl.labels[b, h].cpu().numpy().astype(np.int64)
                _check_assignment(x64, cent0, lab, what)
                _check_sort(lab, cl.perm[b, h].cpu().numpy(), cl.offsets[b, h].cpu().numpy(), C, what)
                _check_update(x64, lab, cent0, cl.centroids[b, h].cpu().numpy(), what)


@pytest.mark.parametrize("case", CASES[:2], ids=[c[0] for c in CASES[:2]])
def test_kmeans_warm_start_continues_cold_run(gpu, case):
    """iters = 4 from a cold start equals 3 iterations, then 1 more from the cached centroids."""
    name, wl = case
    g = wl.geom
    note(f"kmeans warm start {name}")
    q, k, v, iq, ik = _inputs(wl)
    a = gpu.kmeans(k, g.F, g.HH, g.WW, wl.Ck, 4, init_idx=ik)
    b = gpu.kmeans(k, g.F, g.HH, g.WW, wl.Ck, 3, init_idx=ik)
    before = b.centroids.clone()
    b = gpu.kmeans(k, g.F, g.HH, g.WW, wl.Ck, 1, out=b)
    torch.cuda.synchronize()
    for t in ("centroids", "labels", "perm", "offsets"):
        assert torch.equal(getattr(a, t), getattr(b, t)), t
    # and the last iteration is Lloyd's step from the cached centroids
    kh = host64(k)
    for h in range(g.H):
        lab = b.labels[0, h].cpu().numpy().astype(np.int64)
        cent = before[0, h].cpu().numpy().astype(np.float64)
        _check_assignment(kh[0, h], cent, lab, f"{name} warm h{h}")
        _check_update(kh[0, h], lab, cent, b.centroids[0, h].cpu().numpy(), f"{name} warm h{h}")


def test_kmeans_duplicate_starts_leave_empty_clusters(gpu):
    """Duplicate cold-start rows: the higher copies lose every tie, stay empty and keep their centroid."""
    wl = CASES[0][1]
    g = wl.geom
    note("kmeans duplicate starts")
    q, k, v, iq, ik = _inputs(wl)
    idx = iq.clone()
    idx[1] = idx[0]
    idx[5] = idx[0]
    cl = gpu.kmeans(q, g.F, g.HH, g.WW, wl.Cq, 1, init_idx=idx)
    torch.cuda.synchronize()
    off = cl.offsets.cpu().numpy()
    counts = np.diff(off, axis=-1)
    assert (counts[..., 1] == 0).all() and (counts[..., 5] == 0).all()
    start = host64(q)[:, :, idx[0].item()]
    got = cl.centroids.cpu().numpy().astype(np.float64)
    assert np.array_equal(got[:, :, 1], start) and np.array_equal(got[:, :, 5], start)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_topp_and_cluster_attention(gpu, case):
    name, wl = case
    g = wl.geom
    note(f"top-p + cluster attention {name}")
    q, k, v, iq, ik = _inputs(wl)
    cq = gpu.kmeans(q, g.F, g.HH, g.WW, wl.Cq, wl.iters, init_idx=iq)
    ck = gpu.kmeans(k, g.F, g.HH, g.WW, wl.Ck, wl.iters, init_idx=ik)
    sc = 1.0 / np.sqrt(g.D)
    sel = gpu.centroid_topp(cq, ck, g.F, g.HH, g.WW, wl.p)
    o = gpu.cluster_attn(q, k, v, cq, ck, sel, g.F, g.HH, g.WW)
    torch.cuda.synchronize()
    qh, kh, vh, oh = host64(q), host64(k), host64(v), host64(o)
    for b in range(g.B):
        for h in range(g.H):
            what = f"{name} b{b} h{h}"
            counts_k = np.diff(ck.offsets[b, h].cpu().numpy())
            w = O2.centroid_weights(cq.centroids[b, h].cpu().numpy(), ck.centroids[b, h].cpu().numpy(), counts_k, sc)
            s = sel[b, h].cpu().numpy()
            _check_topp(w, s, wl.p, what)
            if wl.p == 1.0:
                assert (s.astype(bool) == (w > 0)).all()
            lq = cq.labels[b, h].cpu().numpy()
            lk = ck.labels[b, h].cpu().numpy()
            want = O2.semantic_attention(qh[b, h], kh[b, h], vh[b, h], lq, lk, s.astype(bool), sc)
            assert_close_attn(oh[b, h], want, what)


def test_cluster_layer_warm_steps(gpu):
    """The layer object: a cold first step, then warm steps from its centroid cache."""
    wl = SEMANTIC_WORKLOADS["svg2_small"]
    g = wl.geom
    note("cluster layer, 3 steps")
    q, k, v, iq, ik = _inputs(wl)
    layer = gpu.ClusterLayer(q, g.F, g.HH, g.WW, wl.Cq, wl.Ck, wl.p, wl.iters, iq, ik)
    for step in range(3):
        q, k, v = make_qkv_semantic(wl, device=DEV, step=step)
        o = layer(q, k, v)
        torch.cuda.synchronize()
        qh, kh, vh, oh = host64(q), host64(k), host64(v), host64(o)
        for h in range(g.H):
            what = f"step {step} h{h}"
            if step > 0:
                lab = layer.cq.labels[0, h].cpu().numpy().astype(np.int64)
                # the last of the iterations started from the cache: check the chain's invariants
                _check_sort(lab, layer.cq.perm[0, h].cpu().numpy(), layer.cq.offsets[0, h].cpu().numpy(), wl.Cq, what)
            s = layer.sel[0, h].cpu().numpy().astype(bool)
            want = O2.semantic_attention(qh[0, h], kh[0, h], vh[0, h], layer.cq.labels[0, h].cpu().numpy(),
                                         layer.ck.labels[0, h].cpu().numpy(), s, 1.0 / np.sqrt(g.D))
            assert_close_attn(oh[0, h], want, what)


def test_full_720p_sampled(gpu):
    """The 720p workload as the benchmark runs it: sorts and lengths in full, centroids, the
    assignment, the selection and the outputs on samples the oracle computes one by one."""
    wl = SEMANTIC_WORKLOADS["hunyuan720p_svg2"]
    g = wl.geom
    note("720p clustering path, sampled parity")
    q, k, v, iq, ik = _inputs(wl)
    layer = gpu.ClusterLayer(q, g.F, g.HH, g.WW, wl.Cq, wl.Ck, wl.p, wl.iters, iq, ik)
    # the assignment of the last iteration is checked against the centroids it started from:
    # run iters - 1 iterations, keep the centroids, then the last one
    cq = gpu.kmeans(q, g.F, g.HH, g.WW, wl.Cq, wl.iters - 1, init_idx=iq)
    ck = gpu.kmeans(k, g.F, g.HH, g.WW, wl.Ck, wl.iters - 1, init_idx=ik)
    cq_prev, ck_prev = cq.centroids.clone(), ck.centroids.clone()
    gpu.kmeans(q, g.F, g.HH, g.WW, wl.Cq, 1, out=cq)
    gpu.kmeans(k, g.F, g.HH, g.WW, wl.Ck, 1, out=ck)
    o = layer(q, k, v)
    torch.cuda.synchronize()
    for t in ("centroids", "labels", "perm", "offsets"):
        assert torch.equal(getattr(cq, t), getattr(layer.cq, t)) and torch.equal(getattr(ck, t), getattr(layer.ck, t))
    rng = np.random.default_rng(5)
    sc = 1.0 / np.sqrt(g.D)
    heads = [0, g.H // 2, g.H - 1]
    for h in heads:
        what = f"720p h{h}"
        qh = host64(q[0, h])
        kh = host64(k[0, h])
        for x64, cl, prev, C, tag in ((qh, cq, cq_prev, wl.Cq, "Q"), (kh, ck, ck_prev, wl.Ck, "K")):
            lab = cl.labels[0, h].cpu().numpy().astype(np.int64)
            _check_sort(lab, cl.perm[0, h].cpu().numpy(), cl.offsets[0, h].cpu().numpy(), C, f"{what} {tag}")
            rows = rng.choice(g.S, 512, replace=False)
            cent = prev[0, h].cpu().numpy().astype(np.float64)
            _check_assignment(x64[rows], cent, lab[rows], f"{what} {tag} assignment")
            _check_update(x64, lab, cent, cl.centroids[0, h].cpu().numpy(), f"{what} {tag} means")
        counts_k = np.diff(ck.offsets[0, h].cpu().numpy())
        w = O2.centroid_weights(cq.centroids[0, h].cpu().numpy(), ck.centroids[0, h].cpu().numpy(), counts_k, sc)
        s = layer.sel[0, h].cpu().numpy()
        _check_topp(w, s, wl.p, what)
        rows = rng.choice(g.S, 256, replace=False)
        lq = cq.labels[0, h].cpu().numpy()
        lk = ck.labels[0, h].cpu().numpy()
        want = O2.semantic_attention_rows(qh, kh, host64(v[0, h]), rows, lq, lk, s.astype(bool), sc)
        assert_close_attn(host64(o[0, h, torch.from_numpy(rows).to(DEV)]), want, what)
    # the planted classes are recovered well enough that the selection is sparse
    dens = []
    for h in range(g.H):
        nq = np.diff(cq.offsets[0, h].cpu().numpy())
        nk = np.diff(ck.offsets[0, h].cpu().numpy())
        s = layer.sel[0, h].cpu().numpy().astype(bool)
        dens.append(sum(nq[i] * nk[s[i]].sum() for i in range(wl.Cq)) / g.S ** 2)
    note(f"720p density {np.mean(dens):.4f} (min {np.min(dens):.4f}, max {np.max(dens):.4f})")
    assert 0.0 < np.mean(dens) < 0.5


@pytest.mark.parametrize("D", [64, 128])
def test_one_cluster_each_is_dense_attention(gpu, D):
    """C_q = C_k = 1: every query attends every key in token order, the dense kernel's own
    schedule, so the output equals svg_dense_attn bit for bit."""
    g = Geometry(1, 2, 3, 9, 11, D)
    wl = _semantic("one_cluster", g, 3, 1, 1, 0.5, 2, 35)
    note(f"one cluster each, D={D}")
    q, k, v, iq, ik = _inputs(wl)
    cq = gpu.kmeans(q, g.F, g.HH, g.WW, 1, 2, init_idx=iq)
    ck = gpu.kmeans(k, g.F, g.HH, g.WW, 1, 2, init_idx=ik)
    sel = gpu.centroid_topp(cq, ck, g.F, g.HH, g.WW, 0.5)
    o = gpu.cluster_attn(q, k, v, cq, ck, sel, g.F, g.HH, g.WW)
    od = gpu.dense_attn(q, k, v, g.F, g.HH, g.WW)
    torch.cuda.synchronize()
    assert (sel == 1).all()
    assert torch.equal(cq.perm[0, 0].cpu(), torch.arange(g.S, dtype=torch.int32))
    assert torch.equal(o, od)


def test_one_token_per_cluster(gpu):
    """C = S: every token is its own cluster, so the estimated shares are the exact attention
    weights of each query, and top-p keeps each query's top-p keys."""
    g = Geometry(1, 2, 4, 7, 9, 64)
    wl = _semantic("token_clusters", g, 4, g.S, g.S, 0.6, 1, 36)
    note("one token per cluster")
    q, k, v, _, _ = _inputs(wl)
    every = torch.arange(g.S, dtype=torch.int32, device=DEV)
    cq = gpu.kmeans(q, g.F, g.HH, g.WW, g.S, 1, init_idx=every)
    ck = gpu.kmeans(k, g.F, g.HH, g.WW, g.S, 1, init_idx=every)
    sel = gpu.centroid_topp(cq, ck, g.F, g.HH, g.WW, wl.p)
    o = gpu.cluster_attn(q, k, v, cq, ck, sel, g.F, g.HH, g.WW)
    torch.cuda.synchronize()
    qh, kh, vh, oh = host64(q), host64(k), host64(v), host64(o)
    sc = 1.0 / np.sqrt(g.D)
    for h in range(g.H):
        lq = cq.labels[0, h].cpu().numpy()
        lk = ck.labels[0, h].cpu().numpy()
        # distinct random rows: each token is nearest to its own start
        assert np.array_equal(lq, np.arange(g.S)) and np.array_equal(lk, np.arange(g.S))
        w = O2.centroid_weights(cq.centroids[0, h].cpu().numpy(), ck.centroids[0, h].cpu().numpy(),
                                np.ones(g.S), sc)
        s = sel[0, h].cpu().numpy()
        _check_topp(w, s, wl.p, f"h{h}")
        want = O2.semantic_attention(qh[0, h], kh[0, h], vh[0, h], lq, lk, s.astype(bool), sc)
        assert_close_attn(oh[0, h], want, f"h{h}")


def test_more_than_1024_clusters(gpu):
    """Cluster counts past one scan block (C > 1024): the counting sort's and the work items'
    multi-pass scans, and attention over 1100 query clusters."""
    g = Geometry(1, 1, 4, 24, 24, 64)                     # S = 2304
    wl = _semantic("many_clusters", g, 6, 1100, 1000, 0.9, 2, 37)
    note("C = 2000 / 1100 / 1000 clusters")
    q, k, v, iq, ik = _inputs(wl)
    i2000 = torch.from_numpy(init_token_indices(g.S, 2000, 38)).to(DEV)
    big = gpu.kmeans(q, g.F, g.HH, g.WW, 2000, 1, init_idx=i2000)
    cq = gpu.kmeans(q, g.F, g.HH, g.WW, wl.Cq, 2, init_idx=iq)
    ck = gpu.kmeans(k, g.F, g.HH, g.WW, wl.Ck, 2, init_idx=ik)
    sel = gpu.centroid_topp(cq, ck, g.F, g.HH, g.WW, wl.p)
    o = gpu.cluster_attn(q, k, v, cq, ck, sel, g.F, g.HH, g.WW)
    torch.cuda.synchronize()
    qh, kh, vh = host64(q)[0, 0], host64(k)[0, 0], host64(v)[0, 0]
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(g.S, 256, replace=False))
    lab = big.labels[0, 0].cpu().numpy().astype(np.int64)
    _check_sort(lab, big.perm[0, 0].cpu().numpy(), big.offsets[0, 0].cpu().numpy(), 2000, "C=2000")
    cent0 = O2.init_centroids(qh, i2000.cpu().numpy())
    _check_assignment(qh[rows], cent0, lab[rows], "C=2000 assignment")
    _check_update(qh, lab, cent0, big.centroids[0, 0].cpu().numpy(), "C=2000 means")
    for cl, C, x, tag in ((cq, wl.Cq, qh, "Q"), (ck, wl.Ck, kh, "K")):
        l = cl.labels[0, 0].cpu().numpy().astype(np.int64)
        _check_sort(l, cl.perm[0, 0].cpu().numpy(), cl.offsets[0, 0].cpu().numpy(), C, tag)
    s = sel[0, 0].cpu().numpy()
    sc = 1.0 / np.sqrt(g.D)
    w = O2.centroid_weights(cq.centroids[0, 0].cpu().numpy(), ck.centroids[0, 0].cpu().numpy(),
                            np.diff(ck.offsets[0, 0].cpu().numpy()), sc)
    _check_topp(w, s, wl.p, "top-p")
    want = O2.semantic_attention_rows(qh, kh, vh, rows, cq.labels[0, 0].cpu().numpy(), ck.labels[0, 0].cpu().numpy(),
                                      s.astype(bool), sc)
    assert_close_attn(host64(o[0, 0])[rows], want, "1100 query clusters")


def test_inconsistent_key_offsets_stay_in_bounds(gpu):
    """Key offsets that are non-monotone, negative or far beyond S: every key list is clamped
    to S entries of in-range rows, so the call writes nothing outside its buffers and every
    output row is a finite mean of V rows."""
    svg = gpu
    g = Geometry(1, 2, 3, 5, 7, 64)
    S = g.S
    note(f"cluster attention with inconsistent key offsets, S={S}")
    gen = torch.Generator(device="cpu").manual_seed(77)
    q, k, v = (torch.randn((g.B, g.H, S, g.D), generator=gen).to(torch.bfloat16).to(DEV) for _ in range(3))
    Cq, Ck = 3, 5
    q_off = torch.tensor([0, 40, 70, S], dtype=torch.int32).repeat(g.B, g.H, 1).contiguous()
    # non-monotone, negative and oversized key offsets
    k_off = torch.tensor([0, S, 3, 4 * S, -5, 2 * S], dtype=torch.int32).repeat(g.B, g.H, 1).contiguous()
    perm = torch.arange(S, dtype=torch.int32).repeat(g.B, g.H, 1).contiguous()
    cq = svg.Clusters(torch.zeros((g.B, g.H, Cq, g.D)), torch.zeros_like(perm), perm, q_off)
    ck = svg.Clusters(torch.zeros((g.B, g.H, Ck, g.D)), torch.zeros_like(perm), perm, k_off)
    cq = svg.Clusters(*(t.to(DEV) for t in (cq.centroids, cq.labels, cq.perm, cq.offsets)))
    ck = svg.Clusters(*(t.to(DEV) for t in (ck.centroids, ck.labels, ck.perm, ck.offsets)))
    sel = torch.ones((g.B, g.H, Cq, Ck), dtype=torch.uint8, device=DEV)
    nbytes = svg.workspace_bytes(svg.OP_CLUSTER_ATTN, svg.geometry(q, g.F, g.HH, g.WW), Cq)
    # a guard region after the workspace must stay untouched
    guard = 1 << 16
    ws = torch.full((nbytes + guard,), 0xA5, dtype=torch.uint8, device=DEV)
    o = svg.cluster_attn(q, k, v, cq, ck, sel, g.F, g.HH, g.WW, ws=ws[:nbytes])
    torch.cuda.synchronize()
    BH = g.B * g.H
    align = lambda n: (n + 255) // 256 * 256
    klen_off = align(BH * Cq * S * 4)
    klen = ws[klen_off:klen_off + BH * Cq * 4].view(torch.int32).cpu().numpy()
    assert (klen >= 0).all() and (klen <= S).all(), klen
    assert (ws[nbytes:].cpu().numpy() == 0xA5).all(), "write past the workspace"
    klist = ws[:BH * Cq * S * 4].view(torch.int32).cpu().numpy().reshape(BH, Cq, S)
    for bh in range(BH):
        for c in range(Cq):
            rows = klist[bh, c, :klen[bh * Cq + c]]
            assert ((rows >= 0) & (rows < S)).all()
    assert torch.isfinite(o.float()).all()
