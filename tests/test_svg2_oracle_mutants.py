"""Plant plausible mistakes in the Sparse VideoGen2 oracle (on the CPU) and check that the pins
of test_svg2_oracle_pins.py catch each one.
"""
import numpy as np
import pytest

import oracle.svg2_oracle as O2
from tests import test_svg2_oracle_pins as pins

ORIG = {n: getattr(O2, n) for n in ("kmeans_assign", "kmeans_update", "kmeans", "cluster_permutation",
                                     "centroid_weights", "topp_select", "semantic_mask", "round_bf16_from_f32")}


def _mut_round_truncate(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    return (u & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)        # truncates


def _mut_round_ties_away(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + np.uint64(0x8000)) & np.uint64(0xFFFF0000)).astype(np.uint32)       # ties away from zero
    return r.view(np.float32).astype(np.float64)


def _mut_assign_exact_centroids(x, cent):
    x = np.asarray(x, dtype=np.float64)
    d2 = ((x[:, None, :] - np.asarray(cent)[None]) ** 2).sum(axis=2)               # no bf16 rounding
    return np.argmin(d2, axis=1)


def _mut_assign_last_tie(x, cent):
    x = np.asarray(x, dtype=np.float64)
    cb = O2.round_bf16_from_f32(cent)
    d2 = ((x[:, None, :] - cb[None]) ** 2).sum(axis=2)
    return d2.shape[1] - 1 - np.argmin(d2[:, ::-1], axis=1)                         # ties to the highest index


def _mut_assign_dot_only(x, cent):
    cb = O2.round_bf16_from_f32(cent)
    return np.argmax(np.asarray(x) @ cb.T, axis=1)                                  # forgets the centroid norms


def _mut_update_empty_zero(x, labels, cent_old):
    new, counts = ORIG["kmeans_update"](x, labels, cent_old)
    new[counts == 0] = 0.0                                                          # empty cluster collapses to 0
    return new, counts


def _mut_update_sum(x, labels, cent_old):
    new, counts = ORIG["kmeans_update"](x, labels, cent_old)
    nz = counts > 0
    new[nz] *= counts[nz, None]                                                     # sum, not mean
    return new, counts


def _mut_kmeans_stale_labels(x, cent0, iters):
    labels, cent, counts = ORIG["kmeans"](x, cent0, iters)
    return O2.kmeans_assign(x, cent0), cent, counts                                  # labels of the first pass


def _mut_perm_unstable(labels, C):
    perm, off = ORIG["cluster_permutation"](labels, C)
    out = perm.copy()
    for c in range(C):
        out[off[c]:off[c + 1]] = perm[off[c]:off[c + 1]][::-1]                    # reversed within a cluster
    return out, off


def _mut_weights_unweighted(cq, ck, counts_k, scale):
    n = (np.asarray(counts_k) > 0).astype(float)                                   # ignores cluster sizes
    return ORIG["centroid_weights"](cq, ck, n, scale)


def _mut_weights_no_scale(cq, ck, counts_k, scale):
    return ORIG["centroid_weights"](cq, ck, counts_k, 1.0)


def _mut_topp_strict(w, p):
    w = np.asarray(w, dtype=np.float64)
    sel = np.zeros(w.shape, dtype=bool)
    for i in range(w.shape[0]):
        acc = 0.0
        for j in sorted(range(w.shape[1]), key=lambda j: (-w[i, j], j)):
            if w[i, j] <= 0.0:
                break
            sel[i, j] = True
            acc += w[i, j]
            if acc > p:                                                             # strict: one cluster too many
                break
    return sel


def _mut_topp_ascending(w, p):
    return ORIG["topp_select"](-np.asarray(w) + 1.0, p)                             # smallest weights first


def _mut_mask_transposed(lq_rows, lk, sel):
    sel = np.asarray(sel, dtype=bool)
    Cq, Ck = sel.shape
    return sel.T[np.asarray(lq_rows)[:, None] % Ck, np.asarray(lk)[None, :] % Cq]  # operands swapped


MUTANTS = [
    ("round_bf16_from_f32", _mut_round_truncate),
    ("round_bf16_from_f32", _mut_round_ties_away),
    ("kmeans_assign", _mut_assign_exact_centroids),
    ("kmeans_assign", _mut_assign_last_tie),
    ("kmeans_assign", _mut_assign_dot_only),
    ("kmeans_update", _mut_update_empty_zero),
    ("kmeans_update", _mut_update_sum),
    ("kmeans", _mut_kmeans_stale_labels),
    ("cluster_permutation", _mut_perm_unstable),
    ("centroid_weights", _mut_weights_unweighted),
    ("centroid_weights", _mut_weights_no_scale),
    ("topp_select", _mut_topp_strict),
    ("topp_select", _mut_topp_ascending),
    ("semantic_mask", _mut_mask_transposed),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[f"{n}:{m.__name__}" for n, m in MUTANTS])
def test_pins_catch_mutant(monkeypatch, name, mutant):
    monkeypatch.setattr(O2, name, mutant)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as exc:  # an assertion, or the mutant breaking a shape
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught mutant {mutant.__name__} of {name}"
