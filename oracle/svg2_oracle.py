"""CPU oracle for Sparse VideoGen2's semantic-aware permutation path.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain, float64 statement of
what the second GPU path (k-means clustering of Q and K, centroid top-p block
selection, and attention over the selected clusters) computes.  Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it; the
library and its Python binding never do, and the two share no code.

Source (cited by key below):
  [svg2-gist]  "Sparse VideoGen2: Accelerate Video Generation with Sparse
               Attention via Semantic-Aware Permutation" -- explainer page at
               gist.science/zh/paper/2505.18875.  Its technical summary,
               section 2 (method): A semantic-aware permutation (k-means of Q
               and K into C_q and C_k clusters, the permutation that makes each
               cluster contiguous, equivalence of the permuted output); B
               centroid-based top-p selection; C centroid caching across
               denoising steps and a kernel with variable block sizes (sparse
               loads of the scattered keys/values, dense compute over the
               contiguous queries).

Readings of points the page leaves open (each marked READING below):
  S1 k-means is Lloyd's algorithm: assign every row to its nearest centroid in
     squared Euclidean distance, then move each centroid to the mean of its rows;
     a fixed number of iterations from given centroids.  Ties go to the lowest
     cluster index; a cluster left empty keeps its centroid.  Q and K of each
     (b, h) are clustered independently.
  S2 centroids are kept in float32; the assignment compares distances to the
     centroids rounded to bfloat16 (the storage precision of Q and K).
  S3 a cold start takes the rows at C given distinct token indices as the initial
     centroids; later denoising steps start from the previous step's centroids.
  S4 the permutation is the stable sort of tokens by cluster index: clusters in
     index order, tokens in their original order inside a cluster.
  S5 a key cluster's centroid stands for its n_j keys: the estimated share of the
     attention of query cluster i that falls on key cluster j is
     w_ij = n_j exp(s_ij) / sum_j' n_j' exp(s_ij'), s_ij = scale * c_qi . c_kj.
  S6 top-p: per query cluster, key clusters in decreasing w (ties: lower index
     first), the shortest prefix whose summed w reaches p (0 < p <= 1).
  S7 each query attends exactly to the keys of the key clusters selected for its
     query cluster (softmax scale 1/sqrt(D)); the output is in the original
     token order.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from oracle.svg_oracle import attention

ROW_CHUNK = 2048


# ----------------------------------------------------------------------------------------------
# Precision of the assignment (READING S2)
# ----------------------------------------------------------------------------------------------
def round_f32(x: np.ndarray) -> np.ndarray:
    """x rounded to float32 (round to nearest even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to bfloat16 (round to nearest, ties to even), as float64.

    bfloat16 keeps the top 16 bits of a float32; rounding adds half a unit of the
    dropped 16 bits, minus one when the kept part is even, before truncating.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_odd = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_odd) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# k-means ([svg2-gist] technical summary, section 2A; READINGS S1-S3)
# ----------------------------------------------------------------------------------------------
def kmeans_assign(x: np.ndarray, cent: np.ndarray) -> np.ndarray:
    """Index of the nearest centroid of every row of x [n, D] (int64 [n]).

    cent [C, D] holds float32 values (READING S2); distances are taken to their
    bfloat16 roundings, in float64.  np.argmin keeps the first of equal minima,
    which is the lowest cluster index.
    """
    x = np.asarray(x, dtype=np.float64)
    cb = round_bf16_from_f32(cent)
    out = np.empty(len(x), dtype=np.int64)
    for r0 in range(0, len(x), ROW_CHUNK):
        xr = x[r0:r0 + ROW_CHUNK]
        d2 = ((xr[:, None, :] - cb[None, :, :]) ** 2).sum(axis=2)
        out[r0:r0 + len(xr)] = np.argmin(d2, axis=1)
    return out


def kmeans_update(x: np.ndarray, labels: np.ndarray, cent_old: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Mean of the rows of each cluster (float64 [C, D]) and the cluster sizes (int64 [C]).

    An empty cluster keeps its old centroid (READING S1).
    """
    x = np.asarray(x, dtype=np.float64)
    C = len(cent_old)
    counts = np.bincount(labels, minlength=C).astype(np.int64)
    sums = np.zeros((C, x.shape[1]))
    np.add.at(sums, labels, x)
    new = np.asarray(cent_old, dtype=np.float64).copy()
    nz = counts > 0
    new[nz] = sums[nz] / counts[nz, None]
    return new, counts


def kmeans(x: np.ndarray, cent0: np.ndarray, iters: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """`iters` Lloyd iterations from centroids cent0 [C, D].

    Returns (labels int64 [n], centroids float64 [C, D] holding float32 values,
    counts int64 [C]): the labels of the last assignment and the centroids of the
    last update, so that every centroid is the (float32-rounded) mean of its rows.
    """
    if iters < 1:
        raise ValueError("k-means needs at least one iteration")
    cent = round_f32(cent0)
    labels = counts = None
    for _ in range(iters):
        labels = kmeans_assign(x, cent)
        cent, counts = kmeans_update(x, labels, cent)
        cent = round_f32(cent)
    return labels, cent, counts


def init_centroids(x: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Cold start (READING S3): the rows at the given distinct token indices."""
    idx = np.asarray(idx, dtype=np.int64)
    if len(np.unique(idx)) != len(idx):
        raise ValueError("initial token indices must be distinct")
    return round_f32(np.asarray(x, dtype=np.float64)[idx])


# ----------------------------------------------------------------------------------------------
# Semantic-aware permutation ([svg2-gist] technical summary, section 2A; READING S4)
# ----------------------------------------------------------------------------------------------
def cluster_permutation(labels: np.ndarray, C: int) -> Tuple[np.ndarray, np.ndarray]:
    """perm [n] (perm[j] = token at sorted position j) and offsets [C + 1].

    Cluster c occupies sorted positions offsets[c] .. offsets[c+1]-1.
    """
    labels = np.asarray(labels, dtype=np.int64)
    perm = np.argsort(labels, kind="stable")
    offsets = np.concatenate([[0], np.cumsum(np.bincount(labels, minlength=C))]).astype(np.int64)
    return perm, offsets


# ----------------------------------------------------------------------------------------------
# Centroid-based top-p selection ([svg2-gist] technical summary, section 2B; READINGS S5, S6)
# ----------------------------------------------------------------------------------------------
def centroid_weights(cq: np.ndarray, ck: np.ndarray, counts_k: np.ndarray, scale: float) -> np.ndarray:
    """w [Cq, Ck]: estimated attention share of each key cluster for each query cluster."""
    s = scale * (np.asarray(cq, dtype=np.float64) @ np.asarray(ck, dtype=np.float64).T)
    n = np.asarray(counts_k, dtype=np.float64)[None, :]
    s = np.where(n > 0, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    e = n * np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def topp_select(w: np.ndarray, p: float) -> np.ndarray:
    """bool [Cq, Ck]: per row, the shortest prefix of clusters in decreasing w reaching p."""
    if not 0.0 < p <= 1.0:
        raise ValueError("p must lie in (0, 1]")
    w = np.asarray(w, dtype=np.float64)
    sel = np.zeros(w.shape, dtype=bool)
    for i in range(w.shape[0]):
        # decreasing weight, lower index first among equals
        order = sorted(range(w.shape[1]), key=lambda j: (-w[i, j], j))
        acc = 0.0
        for j in order:
            if w[i, j] <= 0.0:
                break
            sel[i, j] = True
            acc += w[i, j]
            if acc >= p:
                break
    return sel


# ----------------------------------------------------------------------------------------------
# Attention over the selected clusters ([svg2-gist] technical summary, sections 2A, 2C; READING S7)
# ----------------------------------------------------------------------------------------------
def semantic_mask(lq_rows: np.ndarray, lk: np.ndarray, sel: np.ndarray) -> np.ndarray:
    """Token mask [len(lq_rows), n_keys]: key s is allowed for query t iff sel[lq[t], lk[s]]."""
    return np.asarray(sel, dtype=bool)[np.asarray(lq_rows)[:, None], np.asarray(lk)[None, :]]


def semantic_attention_rows(q, k, v, rows, lq, lk, sel, scale) -> np.ndarray:
    """Output rows `rows` (original token order) of one head."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), np.asarray(q).shape[1]))
    for r0 in range(0, len(rows), ROW_CHUNK // 2):
        r = rows[r0:r0 + ROW_CHUNK // 2]
        out[r0:r0 + len(r)] = attention(np.asarray(q)[r], k, v, semantic_mask(lq[r], lk, sel), scale)
    return out


def semantic_attention(q, k, v, lq, lk, sel, scale) -> np.ndarray:
    """All output rows of one head."""
    return semantic_attention_rows(q, k, v, np.arange(len(q)), lq, lk, sel, scale)


def semantic_attention_permuted(q, k, v, lq, lk, sel, scale) -> np.ndarray:
    """The same head computed in cluster-sorted order, block by block, then restored.

    Q is sorted by query cluster and K/V by key cluster; the score matrix is then
    made of (query cluster, key cluster) blocks of variable size, each computed
    whole or skipped.  Equal to semantic_attention by the equivalence of
    [svg2-gist] section 2A.
    """
    Cq, Ck = np.asarray(sel).shape
    pq, oq = cluster_permutation(lq, Cq)
    pk, ok = cluster_permutation(lk, Ck)
    qs, ks, vs = np.asarray(q)[pq], np.asarray(k)[pk], np.asarray(v)[pk]
    out_sorted = np.empty(qs.shape)
    for i in range(Cq):
        a, b = oq[i], oq[i + 1]
        if a == b:
            continue
        cols = np.concatenate([np.arange(ok[j], ok[j + 1]) for j in range(Ck) if sel[i, j]] or [np.zeros(0, int)])
        out_sorted[a:b] = attention(qs[a:b], ks[cols], vs[cols], np.ones((b - a, len(cols)), dtype=bool), scale)
    out = np.empty_like(out_sorted)
    out[pq] = out_sorted
    return out


def svg2_head(q, k, v, cq0, ck0, iters, p, scale):
    """One head of the path: cluster Q and K, select, attend.

    Returns (lq, cq, nq, lk, ck, nk, sel, out).
    """
    lq, cq, nq = kmeans(q, cq0, iters)
    lk, ck, nk = kmeans(k, ck0, iters)
    sel = topp_select(centroid_weights(cq, ck, nk, scale), p)
    out = semantic_attention(q, k, v, lq, lk, sel, scale)
    return lq, cq, nq, lk, ck, nk, sel, out
