"""Pins of the Sparse VideoGen2 oracle (oracle/svg2_oracle.py) to things other than itself.

Each `pin_*` function checks the oracle against hand-derived values, brute force on
a tiny input, a library routine (torch's bf16 cast, scikit-learn's Lloyd k-means),
a closed form or an invariant, and raises AssertionError on disagreement.  They run
as tests here and, with plausible mistakes planted in the oracle, in
test_svg2_oracle_mutants.py.
"""
import itertools
import math
import warnings

import numpy as np
import pytest
import torch

import oracle.svg2_oracle as O2
import oracle.svg_oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------------------ bf16 rounding
def pin_bf16_rounding_hand_values():
    # bf16 spacing at 1 is 2^-7: ties go to the even neighbour
    vals = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -(1 + 2.0 ** -9), 3.0, 0.0])
    want = np.array([1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -1.0, 3.0, 0.0])
    assert np.array_equal(O2.round_bf16_from_f32(vals.astype(np.float32)), want)


def pin_bf16_rounding_matches_torch():
    x = (_rng(1).standard_normal(20000) * np.exp(_rng(2).uniform(-20, 20, 20000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O2.round_bf16_from_f32(x), want)


# ------------------------------------------------------------------------------ k-means
def _brute_assign(x, cent_exact):
    out = []
    for row in x:
        best, best_d = None, None
        for c, cv in enumerate(cent_exact):
            d = 0.0
            for a, b in zip(row, cv):
                d += (a - b) * (a - b)
            if best is None or d < best_d:
                best, best_d = c, d
        out.append(best)
    return np.array(out)


def pin_assign_brute_force():
    r = _rng(3)
    for n, C, D in [(40, 5, 4), (33, 7, 3), (12, 1, 6)]:
        x = r.standard_normal((n, D))
        # centroids that are bf16 numbers already, so that the rounding is the identity
        cent = O2.round_bf16_from_f32(r.standard_normal((C, D)).astype(np.float32))
        assert np.array_equal(O2.kmeans_assign(x, cent), _brute_assign(x, cent))


def pin_assign_uses_bf16_centroids_and_lowest_index():
    # x = 0; c0 = 1 + 2^-9 rounds to 1, c1 = -(1 + 2^-10) rounds to -1: a tie after rounding
    # (lowest index wins), while the exact distances would pick c1
    x = np.zeros((1, 1))
    cent = np.array([[1 + 2.0 ** -9], [-(1 + 2.0 ** -10)]])
    assert O2.kmeans_assign(x, cent)[0] == 0
    assert O2.kmeans_assign(x, cent[::-1])[0] == 0
    # duplicate centroids: every row goes to the first copy
    c2 = np.array([[0.5, 0.5], [0.5, 0.5], [4.0, 4.0]])
    assert (O2.kmeans_assign(_rng(4).uniform(0, 1, (10, 2)), c2) == 0).all()


def pin_update_brute_force_and_empty_cluster():
    r = _rng(5)
    x = r.standard_normal((30, 3))
    labels = r.integers(0, 4, 30)
    labels[labels == 2] = 1                         # cluster 2 is empty
    old = r.standard_normal((4, 3))
    new, counts = O2.kmeans_update(x, labels, old)
    for c in range(4):
        members = [x[t] for t in range(30) if labels[t] == c]
        assert counts[c] == len(members)
        if members:
            s = [0.0, 0.0, 0.0]
            for m in members:
                s = [a + b for a, b in zip(s, m)]
            assert np.allclose(new[c], [v / len(members) for v in s], rtol=0, atol=1e-14)
        else:
            assert np.array_equal(new[c], old[c])


def _dyadic_blobs(seed, C, per, D, spread=40):
    """Integer points in C well-separated blobs of `per` points (per a power of two)."""
    r = _rng(seed)
    centers = r.integers(-3, 4, (C, D)) * spread
    x = np.concatenate([centers[c] + r.integers(-3, 4, (per, D)) for c in range(C)]).astype(np.float64)
    truth = np.repeat(np.arange(C), per)
    order = r.permutation(len(x))
    return x[order], truth[order]


def pin_kmeans_recovers_separated_blobs():
    x, truth = _dyadic_blobs(6, 5, 8, 4)
    # one point of each blob as the cold start (S3)
    idx = [int(np.flatnonzero(truth == c)[0]) for c in range(5)]
    labels, cent, counts = O2.kmeans(x, O2.init_centroids(x, idx), 3)
    assert np.array_equal(labels, truth)
    assert np.array_equal(counts, np.full(5, 8))
    for c in range(5):
        assert np.array_equal(cent[c], x[truth == c].mean(axis=0))


def pin_kmeans_matches_sklearn_lloyd():
    """scikit-learn's Lloyd iteration from the same start (data whose centroids are bf16 numbers)."""
    from sklearn.cluster import KMeans
    for seed, C, per, D in [(7, 4, 4, 3), (8, 6, 8, 5), (9, 3, 16, 2)]:
        x, truth = _dyadic_blobs(seed, C, per, D)
        r = _rng(seed + 100)
        # start from one point of each blob, shuffled, so the labels are a permutation of truth
        idx = [int(r.choice(np.flatnonzero(truth == c))) for c in r.permutation(C)]
        init = x[idx]
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            km = KMeans(n_clusters=C, init=init, n_init=1, max_iter=10, tol=0.0, algorithm="lloyd").fit(x)
        labels, cent, _ = O2.kmeans(x, init, 10)
        assert np.array_equal(labels, km.labels_)
        assert np.abs(cent - km.cluster_centers_).max() < 1e-12


def pin_kmeans_fixed_point_and_objective():
    r = _rng(10)
    x = r.standard_normal((200, 6))
    c0 = O2.init_centroids(x, r.choice(200, 8, replace=False))
    l1, c1, _ = O2.kmeans(x, c0, 25)
    l2, c2, _ = O2.kmeans(x, c1, 1)
    # after convergence one more iteration changes nothing
    assert np.array_equal(l1, l2) and np.abs(c1 - c2).max() < 1e-6
    # every row sits with its nearest (bf16-rounded) centroid, brute force
    cb = O2.round_bf16_from_f32(c1)
    assert np.array_equal(l1, _brute_assign(x, cb))
    # the within-cluster sum of squares never exceeds that of the start
    obj = lambda lab, c: float(((x - c[lab]) ** 2).sum())
    la0 = _brute_assign(x, O2.round_bf16_from_f32(c0))
    assert obj(l1, c1) <= obj(la0, c0)


# ------------------------------------------------------------------------------ permutation
def pin_cluster_permutation_brute_force():
    r = _rng(11)
    for n, C in [(50, 6), (17, 1), (9, 12)]:
        labels = r.integers(0, C, n)
        perm, off = O2.cluster_permutation(labels, C)
        want = sorted(range(n), key=lambda t: (labels[t], t))
        assert list(perm) == want
        assert off[0] == 0 and off[-1] == n
        for c in range(C):
            assert off[c + 1] - off[c] == sum(1 for t in range(n) if labels[t] == c)
            assert all(labels[perm[j]] == c for j in range(off[c], off[c + 1]))


# ------------------------------------------------------------------------------ top-p
def pin_centroid_weights_closed_forms():
    r = _rng(12)
    cq, ck = r.standard_normal((3, 4)), r.standard_normal((5, 4))
    n = np.array([3, 0, 7, 1, 2])
    w = O2.centroid_weights(cq, ck, n, 0.5)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-15)
    assert (w[:, 1] == 0).all()                                     # empty key cluster
    # ratio of two clusters: (n_a / n_b) exp(scale * cq . (ck_a - ck_b))
    ratio = (7 / 3) * math.exp(0.5 * float(cq[1] @ (ck[2] - ck[0])))
    assert abs(w[1, 2] / w[1, 0] - ratio) < 1e-12 * ratio
    # equal scores: shares proportional to the cluster sizes
    w0 = O2.centroid_weights(np.zeros((1, 4)), ck, n, 1.0)
    assert np.allclose(w0[0], n / n.sum(), atol=1e-15)


def pin_topp_brute_force_minimal_subset():
    r = _rng(13)
    for trial in range(60):
        C = int(r.integers(1, 8))
        w = r.dirichlet(np.ones(C) * 0.7)[None, :]
        p = float(r.choice([0.3, 0.5, 0.8, 0.9, 0.95, 1.0]))
        sel = O2.topp_select(w, p)[0]
        # the smallest number of clusters whose weights reach p, and the largest total at that size
        best_k, best_sum = None, None
        for k in range(1, C + 1):
            sums = [sum(w[0, list(s)]) for s in itertools.combinations(range(C), k)]
            if max(sums) >= p - 1e-12:
                best_k, best_sum = k, max(sums)
                break
        if best_k is None:                          # p = 1 not reached by rounding: everything
            assert sel.all()
            continue
        assert sel.sum() == best_k, (w, p, sel)
        assert abs(w[0, sel].sum() - best_sum) < 1e-12


def pin_topp_exact_threshold_and_extremes():
    w = np.array([[0.25, 0.5, 0.25, 0.0]])
    assert O2.topp_select(w, 0.75)[0].tolist() == [True, True, False, False]   # 0.5 + 0.25 reaches 0.75
    assert O2.topp_select(w, 0.76)[0].tolist() == [True, True, True, False]
    assert O2.topp_select(w, 1e-9)[0].tolist() == [False, True, False, False]  # the largest alone
    assert O2.topp_select(w, 1.0)[0].tolist() == [True, True, True, False]     # zero weight never
    with pytest.raises(ValueError):
        O2.topp_select(w, 0.0)


# ------------------------------------------------------------------------------ attention
def pin_semantic_attention_reduces_to_dense():
    r = _rng(14)
    n, D = 40, 8
    q, k, v = r.standard_normal((3, n, D))
    lq, lk = r.integers(0, 3, n), r.integers(0, 5, n)
    full = O2.semantic_attention(q, k, v, lq, lk, np.ones((3, 5), bool), 0.3)
    assert np.abs(full - O.attention(q, k, v, np.ones((n, n), bool), 0.3)).max() < 1e-13


def pin_semantic_attention_hand_example():
    # zero queries: every allowed key has the same logit, so the output is the mean of the
    # allowed values.  Key clusters: {0, 3}, {1}, {2, 4}; query cluster 0 takes key clusters
    # 0 and 2, query cluster 1 takes key cluster 1 only.
    q = np.zeros((2, 2))
    k = np.arange(10.0).reshape(5, 2)
    v = np.array([[1.0, 0], [2, 0], [3, 0], [4, 0], [5, 1]])
    lk = np.array([0, 1, 2, 0, 2])
    lq = np.array([1, 0])
    sel = np.array([[True, False, True], [False, True, False]])
    out = O2.semantic_attention(q, k, v, lq, lk, sel, 1.0)
    assert np.abs(out[0] - [2.0, 0.0]).max() < 1e-15                      # key 1 alone
    assert np.abs(out[1] - [(1 + 3 + 4 + 5) / 4, 0.25]).max() < 1e-15       # keys 0, 2, 3, 4


def pin_semantic_attention_permuted_blocks_equal():
    r = _rng(15)
    n, D, Cq, Ck = 60, 6, 4, 7
    q, k, v = r.standard_normal((3, n, D))
    lq, lk = r.integers(0, Cq, n), r.integers(0, Ck, n)
    lq[lq == 2] = 1                                                        # an empty query cluster
    sel = r.random((Cq, Ck)) < 0.45
    sel[np.arange(Cq), r.integers(0, Ck, Cq)] = True
    # every selected set must hold a key: give each key cluster at least one key
    lk[:Ck] = np.arange(Ck)
    a = O2.semantic_attention(q, k, v, lq, lk, sel, 0.4)
    b = O2.semantic_attention_permuted(q, k, v, lq, lk, sel, 0.4)
    assert np.abs(a - b).max() < 1e-13


def pin_svg2_head_consistency():
    r = _rng(16)
    n, D = 96, 8
    q, k, v = r.standard_normal((3, n, D))
    cq0 = O2.init_centroids(q, r.choice(n, 4, replace=False))
    ck0 = O2.init_centroids(k, r.choice(n, 6, replace=False))
    lq, cq, nq, lk, ck, nk, sel, out = O2.svg2_head(q, k, v, cq0, ck0, 4, 0.9, 0.35)
    assert nq.sum() == n and nk.sum() == n
    assert np.array_equal(sel, O2.topp_select(O2.centroid_weights(cq, ck, nk, 0.35), 0.9))
    for i in range(4):
        if nq[i]:
            assert sel[i].any()
    assert np.abs(out - O2.semantic_attention_permuted(q, k, v, lq, lk, sel, 0.35)).max() < 1e-13


ALL_PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_") and callable(v)]


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()
