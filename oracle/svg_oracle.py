"""CPU oracle for Sparse VideoGen's spatial/temporal sparse 3D attention.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain, float64 statement
of what the GPU path computes.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the library and its Python binding
never do, and the two share no code.

Sources (cited by key below):
  [svg-authors]  "Sparse VideoGen: Accelerating Video Diffusion Transformers with
                 Spatial-Temporal Sparsity" -- the authors' article, reposted at
                 dtcms.com/wzjs/233309.html.  Sections: Spatial Head, Temporal
                 Head, Online Profiling Strategy, Layout Transformation, and the
                 closing "other optimisations" section.
  [svg-jqzx]     "ICML 2025 | 视频生成模型无损加速两倍，秘诀竟然是「抓住attention的时空
                 稀疏性」" -- 机器之心's article on the same paper, reposted at
                 xinfinite.net/t/topic/12021.  Sections: capturing sparsity in
                 attention; the dynamic adaptive sparsity strategy (a three-step
                 list); Layout Transformation + kernel acceleration.
  [svg2-gist]    "Sparse VideoGen2: Accelerate Video Generation with Sparse
                 Attention via Semantic-Aware Permutation" -- AI-written explainer
                 at gist.science/zh/paper/2505.18875, section 2 (method), part A.

Notation.  A video latent is F frames of an HH x WW token grid; P = HH*WW tokens
per frame, S = F*P tokens.  Frame-major order (the model's own) puts every
token of a frame together: t = f*P + p with p = y*WW + x.  Token-major order
puts every frame of one location together: u = p*F + f.  Tensors are
[B, H, S, D] float64 arrays; every function works on one (b, h) slice unless it
says otherwise.

Readings of points the pages leave open (each is marked READING below):
  R1 spatial window: same frame and +-w_f frames, clipped at the ends.
  R2 temporal band: same in-frame position +-w_p over the flattened index
     p = y*WW + x, in every frame, clipped at the ends.
  R3 masks are token-level; tiles only skip work.
  R4 softmax scale 1/sqrt(D) unless given.
  R5 the profiling error is the mean over sampled rows and channels of the
     squared difference between masked and dense attention OUTPUTS.
  R6 two candidates (spatial, temporal); ties (mse_sp <= mse_tp) go to spatial.
  R7 one shared sample of query rows for every (b, h) of a call.
  R8 Q, K and V of temporal heads are reordered; the output is restored.
  R9 QK-Norm is RMSNorm over the head dim with one weight vector [D] for all
     heads (separate vectors for Q and K).
  R10 3D RoPE splits D into t/h/w slices of widths D-4*floor(D/6), 2*floor(D/6),
     2*floor(D/6); channel pairs (2j, 2j+1) inside a slice of width n rotate by
     pos * base**(-2j/n), pos being the token's frame, row or column.

Memory: attention is evaluated a block of query rows at a time (the rows are
independent), which bounds memory without changing the arithmetic.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

SPATIAL = 0
TEMPORAL = 1
DENSE = 2

ROW_CHUNK = 1024


# ----------------------------------------------------------------------------------------------
# Token coordinates
# ----------------------------------------------------------------------------------------------
def token_coords(t: np.ndarray, HH: int, WW: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """(f, p, y, x) of frame-major token indices t."""
    t = np.asarray(t, dtype=np.int64)
    P = HH * WW
    f = t // P
    p = t % P
    return f, p, p // WW, p % WW


# ----------------------------------------------------------------------------------------------
# O1  Masks  ([svg-authors] Spatial Head / Temporal Head; [svg-jqzx] capturing sparsity)
# ----------------------------------------------------------------------------------------------
def mask_spatial(q_t: np.ndarray, k_t: np.ndarray, P: int, w_f: int) -> np.ndarray:
    """Spatial head: query and key lie in the same frame or within w_f frames (READING R1).

    q_t, k_t are frame-major token indices; result is bool [len(q_t), len(k_t)].
    """
    fq = np.asarray(q_t, dtype=np.int64)[:, None] // P
    fk = np.asarray(k_t, dtype=np.int64)[None, :] // P
    return np.abs(fq - fk) <= w_f


def mask_temporal(q_t: np.ndarray, k_t: np.ndarray, P: int, w_p: int) -> np.ndarray:
    """Temporal head: key sits at (nearly) the same in-frame location, any frame (READING R2).

    The map of such a head is a set of slash lines whose stride is the frame size P.
    """
    pq = np.asarray(q_t, dtype=np.int64)[:, None] % P
    pk = np.asarray(k_t, dtype=np.int64)[None, :] % P
    return np.abs(pq - pk) <= w_p


def mask_rows(kind: int, q_t: np.ndarray, S: int, P: int, w_f: int, w_p: int) -> np.ndarray:
    """Mask of frame-major query rows q_t against all S frame-major keys."""
    k_t = np.arange(S, dtype=np.int64)
    if kind == SPATIAL:
        return mask_spatial(q_t, k_t, P, w_f)
    if kind == TEMPORAL:
        return mask_temporal(q_t, k_t, P, w_p)
    if kind == DENSE:
        return np.ones((len(q_t), S), dtype=bool)
    raise ValueError(f"unknown head kind {kind}")


# ----------------------------------------------------------------------------------------------
# O2  Layout transformation ([svg-authors] Layout Transformation; [svg-jqzx] layout section)
# ----------------------------------------------------------------------------------------------
def perm_indices(F: int, P: int) -> np.ndarray:
    """pi with token_major[u] = frame_major[pi[u]]: the transpose of the [F, P] token grid."""
    return np.arange(F * P, dtype=np.int64).reshape(F, P).T.ravel()


def inverse_perm(pi: np.ndarray) -> np.ndarray:
    return np.argsort(pi, kind="stable")


def permute(x: np.ndarray, F: int, P: int) -> np.ndarray:
    """Frame-major -> token-major along the sequence axis (axis -2)."""
    return x[..., perm_indices(F, P), :]


def unpermute(y: np.ndarray, F: int, P: int) -> np.ndarray:
    """Token-major -> frame-major along the sequence axis (axis -2)."""
    return y[..., inverse_perm(perm_indices(F, P)), :]


# ----------------------------------------------------------------------------------------------
# O3  Masked softmax attention (textbook definition; the pages give no formula)
# ----------------------------------------------------------------------------------------------
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q k^T, restricted to mask) v for a block of rows, in float64.

    q [n, D], k [S, D], v [S, D], mask bool [n, S].  A row with no allowed key
    is an error (every row of the method allows at least its own token).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if not mask.any(axis=1).all():
        raise ValueError("attention row with no allowed key")
    logits = scale * (q @ k.T)
    logits = np.where(mask, logits, -np.inf)
    logits -= logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w /= w.sum(axis=1, keepdims=True)
    return w @ v


def default_scale(D: int) -> float:
    """READING R4: 1/sqrt(D)."""
    return 1.0 / math.sqrt(D)


def head_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows: np.ndarray, kind: int,
                        F: int, P: int, w_f: int, w_p: int, scale: float) -> np.ndarray:
    """Frame-major output rows `rows` of one head under its token mask (q, k, v: [S, D])."""
    S = F * P
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), q.shape[1]), dtype=np.float64)
    for c0 in range(0, len(rows), ROW_CHUNK):
        r = rows[c0:c0 + ROW_CHUNK]
        out[c0:c0 + len(r)] = attention(q[r], k, v, mask_rows(kind, r, S, P, w_f, w_p), scale)
    return out


def head_attention(q, k, v, kind, F, P, w_f, w_p, scale) -> np.ndarray:
    """All S frame-major output rows of one head."""
    return head_attention_rows(q, k, v, np.arange(F * P), kind, F, P, w_f, w_p, scale)


def head_attention_token_major(q, k, v, kind, F, P, w_f, w_p, scale) -> np.ndarray:
    """The same head computed in token-major order: permute Q/K/V, attend under the
    permuted mask (mask(pi[u], pi[u'])), restore the output order (READING R8).

    By [svg2-gist] section 2A a permutation applied consistently to queries and
    keys leaves the attention output unchanged once the output is un-permuted.
    """
    S = F * P
    pi = perm_indices(F, P)
    qt, kt, vt = q[pi], k[pi], v[pi]
    ot = np.empty_like(qt, dtype=np.float64)
    for c0 in range(0, S, ROW_CHUNK):
        u = np.arange(c0, min(S, c0 + ROW_CHUNK))
        if kind == SPATIAL:
            m = mask_spatial(pi[u], pi, P, w_f)
        elif kind == TEMPORAL:
            m = mask_temporal(pi[u], pi, P, w_p)
        else:
            m = np.ones((len(u), S), dtype=bool)
        ot[u] = attention(qt[u], kt, vt, m, scale)
    return ot[inverse_perm(pi)]


# ----------------------------------------------------------------------------------------------
# O4  Block mask: which BM x BN tiles of a head's score matrix hold any allowed pair
# ----------------------------------------------------------------------------------------------
def head_layout_index(kind: int, F: int, P: int) -> np.ndarray:
    """Frame-major token held at each position of the head's working layout.

    Temporal heads work in token-major order (READING R8); others in frame-major.
    """
    if kind == TEMPORAL:
        return perm_indices(F, P)
    return np.arange(F * P, dtype=np.int64)


def block_mask(kind: int, F: int, P: int, w_f: int, w_p: int, bm: int, bn: int,
               q_blocks=None) -> np.ndarray:
    """uint8 [nQB, nKB]: OR of the token mask over each tile, in the head's layout.

    Tiles at the end of the sequence are clipped.  `q_blocks` limits the rows
    computed (the others are left 0) for large grids.
    """
    S = F * P
    nqb = -(-S // bm)
    nkb = -(-S // bn)
    lay = head_layout_index(kind, F, P)
    out = np.zeros((nqb, nkb), dtype=np.uint8)
    blocks = range(nqb) if q_blocks is None else q_blocks
    for i in blocks:
        rows = lay[i * bm: min(S, (i + 1) * bm)]
        # column j of m is the key held at position j of the head's layout
        m = mask_rows(kind, rows, S, P, w_f, w_p)[:, lay]
        any_key = m.any(axis=0)
        pad = nkb * bn - S
        any_key = np.concatenate([any_key, np.zeros(pad, dtype=bool)])
        out[i] = any_key.reshape(nkb, bn).any(axis=1)
    return out


# ----------------------------------------------------------------------------------------------
# O5  Online profiling ([svg-jqzx] dynamic adaptive sparsity, steps 1-3;
#     [svg-authors] Online Profiling Strategy)
# ----------------------------------------------------------------------------------------------
def profile_head(q, k, v, idx, F, P, w_f, w_p, scale) -> Tuple[float, float, int]:
    """Per-head choice of mask from a sample of query rows.

    Step 1: the sampled rows idx (frame-major).  Step 2: their attention under
    the spatial mask, the temporal mask and no mask.  Step 3: the error of each
    sparse result against the dense one, and the kind with the smaller error.
    Returns (mse_spatial, mse_temporal, kind)  (READINGS R5, R6).
    """
    idx = np.asarray(idx, dtype=np.int64)
    o_full = head_attention_rows(q, k, v, idx, DENSE, F, P, w_f, w_p, scale)
    o_sp = head_attention_rows(q, k, v, idx, SPATIAL, F, P, w_f, w_p, scale)
    o_tp = head_attention_rows(q, k, v, idx, TEMPORAL, F, P, w_f, w_p, scale)
    mse_sp = float(np.mean((o_sp - o_full) ** 2))
    mse_tp = float(np.mean((o_tp - o_full) ** 2))
    kind = SPATIAL if mse_sp <= mse_tp else TEMPORAL
    return mse_sp, mse_tp, kind


def profile_heads(q, k, v, idx, F, P, w_f, w_p, scale) -> Tuple[np.ndarray, np.ndarray]:
    """All (b, h) of [B, H, S, D] inputs with one shared sample idx (READING R7).

    Returns mse float64 [B, H, 2] (spatial, temporal) and kind uint8 [B, H].
    """
    B, H = q.shape[:2]
    mse = np.zeros((B, H, 2))
    kind = np.zeros((B, H), dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            a, c, kd = profile_head(q[b, h], k[b, h], v[b, h], idx, F, P, w_f, w_p, scale)
            mse[b, h] = (a, c)
            kind[b, h] = kd
    return mse, kind


def choices_agree(kind_a: np.ndarray, kind_b: np.ndarray, mse_ref: np.ndarray, rel_tie: float = 1e-6) -> np.ndarray:
    """Per (b, h): True where two choices agree or the reference errors are a near tie."""
    a, c = mse_ref[..., 0], mse_ref[..., 1]
    near = np.abs(a - c) <= rel_tie * np.maximum(np.maximum(a, c), 1e-300)
    return (kind_a == kind_b) | near


# ----------------------------------------------------------------------------------------------
# O6  QK-RMSNorm and O7 3D RoPE ([svg-authors] other optimisations; [svg-jqzx] layout section,
#     last paragraph: both operations are named, neither is defined -> READINGS R9, R10)
# ----------------------------------------------------------------------------------------------
def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean over the last axis of x^2 + eps) * w."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def rope_split(D: int) -> Tuple[int, int, int]:
    """Widths (dt, dh, dw) of the frame / row / column slices of the head dim."""
    third = 2 * (D // 6)
    return D - 2 * third, third, third


def rope_3d(x: np.ndarray, F: int, HH: int, WW: int, base: float, dims=None) -> np.ndarray:
    """Rotate channel pairs of x [..., S, D] (frame-major tokens) by their 3D position."""
    x = np.asarray(x, dtype=np.float64)
    S, D = x.shape[-2], x.shape[-1]
    dt, dh, dw = rope_split(D) if dims is None else dims
    assert dt + dh + dw == D and dt % 2 == 0 and dh % 2 == 0 and dw % 2 == 0
    f, _, y, xx = token_coords(np.arange(S), HH, WW)
    out = x.copy()
    off = 0
    for width, pos in ((dt, f), (dh, y), (dw, xx)):
        for j in range(width // 2):
            theta = pos.astype(np.float64) * base ** (-2.0 * j / width)
            c, s = np.cos(theta), np.sin(theta)
            a = x[..., off + 2 * j]
            b = x[..., off + 2 * j + 1]
            out[..., off + 2 * j] = a * c - b * s
            out[..., off + 2 * j + 1] = a * s + b * c
        off += width
    return out


def qknorm_rope(q, k, wq, wk, eps, F, HH, WW, base, dims=None):
    """QK-RMSNorm then 3D RoPE on Q and K ([B, H, S, D]); V is untouched."""
    return (rope_3d(rms_norm(q, wq, eps), F, HH, WW, base, dims),
            rope_3d(rms_norm(k, wk, eps), F, HH, WW, base, dims))


# ----------------------------------------------------------------------------------------------
# O8  One layer of the sparse path
# ----------------------------------------------------------------------------------------------
def sparse_attention(q, k, v, kind, F, P, w_f, w_p, scale) -> np.ndarray:
    """[B, H, S, D] output, each head under the mask of its kind (uint8 [B, H])."""
    out = np.empty(q.shape, dtype=np.float64)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            out[b, h] = head_attention(q[b, h], k[b, h], v[b, h], int(kind[b, h]), F, P, w_f, w_p, scale)
    return out


def full_step(q, k, v, idx, F, HH, WW, w_f, w_p, scale, norm=None):
    """Norm/RoPE (if `norm` = (wq, wk, eps, base) is given) -> profile -> sparse attention.

    Returns (q', k', mse, kind, out).  The layout transform does not change the
    result (see head_attention_token_major), so the output is computed directly
    in frame-major order.
    """
    P = HH * WW
    if norm is not None:
        wq, wk, eps, base = norm
        q, k = qknorm_rope(q, k, wq, wk, eps, F, HH, WW, base)
    mse, kind = profile_heads(q, k, v, idx, F, P, w_f, w_p, scale)
    out = sparse_attention(q, k, v, kind, F, P, w_f, w_p, scale)
    return q, k, mse, kind, out
