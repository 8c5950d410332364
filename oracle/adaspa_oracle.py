"""CPU oracle for the AdaSpa-style head-adaptive block-sparse attention path.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain, float64 statement of
what the third GPU path (a dense pass that keeps each query row's log-sum-exp,
an exact search of the attention mass of every block with that cached
normaliser, a per-head adaptive choice of key blocks, and attention over the
chosen blocks) computes.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the library and its Python binding
never do, and the two share no code.

Source (cited by key below):
  [adaspa]  "Training-free and Adaptive Sparse Attention for Efficient Long Video
            Generation" -- the arxivdaily page of arXiv 2502.21079, its abstract
            (Chinese and English): a blockified sparse pattern; a search that
            uses the log-sum-exp (LSE) of attention rows cached from earlier
            denoising steps, since patterns and LSE change with input, layer and
            head but stay nearly fixed across steps; head-adaptive block-sparse
            attention over the blocks found.

The abstract names these parts and gives no formula, block size or threshold.
Readings (each marked READING below):
  A1 LSE: the natural-log log-sum-exp of a query row's scaled logits over all
     keys, LSE_q = log sum_k exp(scale * q . k), as a dense attention pass
     produces it; it is cached per (layer, head, row) and reused later.
  A2 block mass: for query block i and key block j,
     M_ij = sum over rows q of i and keys k of j of exp(scale * q . k - LSE_q),
     the attention probability the block carries, normalised by the cached LSE
     (exact when the LSE belongs to the same Q and K: each row then sums to 1).
  A3 blocks: 256 query rows by 64 keys (the attention kernel's tiles), the last
     ones clipped at the sequence end; one level of blocks.
  A4 head-adaptive choice: per (head, query block), key blocks in decreasing
     mass (ties: lower index first), the shortest prefix whose mass reaches
     `coverage` times the row's total mass; the count varies by head and block.
  A5 attention: every query of block i attends exactly the keys of its chosen
     key blocks; softmax scale 1/sqrt(D) unless given.
"""
from __future__ import annotations

import math

import numpy as np

from oracle.svg_oracle import attention

BQ = 256
BK = 64
ROW_CHUNK = 1024


def row_lse(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """LSE of every row of q [n, D] against all keys k [S, D] (READING A1), float64 [n]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    out = np.empty(len(q))
    for r0 in range(0, len(q), ROW_CHUNK):
        z = scale * (q[r0:r0 + ROW_CHUNK] @ k.T)
        m = z.max(axis=1, keepdims=True)
        out[r0:r0 + len(z)] = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
    return out


def block_mass(q: np.ndarray, k: np.ndarray, lse: np.ndarray, scale: float, bq: int = BQ,
               bk: int = BK, q_blocks=None) -> np.ndarray:
    """M [nqb, nkb] of one head (READING A2, A3).  `q_blocks` limits the rows computed."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    S = len(q)
    nqb, nkb = -(-S // bq), -(-len(k) // bk)
    M = np.zeros((nqb, nkb))
    blocks = range(nqb) if q_blocks is None else q_blocks
    pad = nkb * bk - len(k)
    for i in blocks:
        rows = slice(i * bq, min(S, (i + 1) * bq))
        p = np.exp(scale * (q[rows] @ k.T) - np.asarray(lse, dtype=np.float64)[rows, None])
        col = np.concatenate([p.sum(axis=0), np.zeros(pad)])
        M[i] = col.reshape(nkb, bk).sum(axis=1)
    return M


def select_blocks(M: np.ndarray, coverage: float) -> np.ndarray:
    """bool [nqb, nkb]: per row, the shortest prefix of blocks in decreasing mass whose mass
    reaches coverage * the row's total (READING A4)."""
    if not 0.0 < coverage <= 1.0:
        raise ValueError("coverage must lie in (0, 1]")
    M = np.asarray(M, dtype=np.float64)
    sel = np.zeros(M.shape, dtype=bool)
    for i in range(M.shape[0]):
        target = coverage * M[i].sum()
        order = sorted(range(M.shape[1]), key=lambda j: (-M[i, j], j))
        acc = 0.0
        for j in order:
            if M[i, j] <= 0.0:
                break
            sel[i, j] = True
            acc += M[i, j]
            if acc >= target:
                break
    return sel


def block_token_mask(sel: np.ndarray, rows: np.ndarray, S: int, bq: int = BQ, bk: int = BK) -> np.ndarray:
    """Token mask [len(rows), S] of the chosen blocks (READING A5)."""
    rows = np.asarray(rows, dtype=np.int64)
    kb = np.arange(S) // bk
    return np.asarray(sel, dtype=bool)[(rows // bq)[:, None], kb[None, :]]


def block_sparse_attention_rows(q, k, v, sel, rows, scale, bq: int = BQ, bk: int = BK) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), np.asarray(q).shape[1]))
    S = len(k)
    for r0 in range(0, len(rows), ROW_CHUNK):
        r = rows[r0:r0 + ROW_CHUNK]
        out[r0:r0 + len(r)] = attention(np.asarray(q)[r], k, v, block_token_mask(sel, r, S, bq, bk), scale)
    return out


def block_sparse_attention(q, k, v, sel, scale, bq: int = BQ, bk: int = BK) -> np.ndarray:
    """All output rows of one head under the chosen blocks."""
    return block_sparse_attention_rows(q, k, v, sel, np.arange(len(q)), scale, bq, bk)


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
