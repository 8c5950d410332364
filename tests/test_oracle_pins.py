"""Pins of the CPU oracle to things other than itself.

Each `pin_*` function checks the oracle against a hand-derived fixture, brute
force on a tiny input, a library routine, a closed form or an invariant, and
raises AssertionError on disagreement.  They are run as tests here and, with
plausible mistakes planted in the oracle, by test_oracle_mutants.py.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle.svg_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden_blocks(name):
    blocks, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = line.strip("[]")
                blocks[cur] = []
            else:
                blocks[cur].append(line)
    return blocks


def _rng(seed):
    return np.random.default_rng(seed)


def _brute_tokens(F, HH, WW):
    """(t, f, p, y, x) enumerated by nested loops, independent of integer division."""
    out = []
    t = 0
    for f in range(F):
        for y in range(HH):
            for x in range(WW):
                out.append((t, f, y * WW + x, y, x))
                t += 1
    return out


# --------------------------------------------------------------------------------------- masks
def pin_masks_golden():
    g = _read_golden_blocks("tiny_masks.txt")
    F, P = 3, 2
    t = np.arange(F * P)
    sp = O.mask_spatial(t, t, P, 1).astype(int)
    tp = O.mask_temporal(t, t, P, 0).astype(int)
    want_sp = np.array([[int(c) for c in r] for r in g["spatial w_f=1"]])
    want_tp = np.array([[int(c) for c in r] for r in g["temporal w_p=0"]])
    want_tm = np.array([[int(c) for c in r] for r in g["temporal_token_major w_p=0"]])
    assert (sp == want_sp).all(), sp
    assert (tp == want_tp).all(), tp
    pi = O.perm_indices(F, P)
    assert (tp[np.ix_(pi, pi)] == want_tm).all()


def pin_masks_brute_force():
    for (F, HH, WW) in [(3, 2, 3), (4, 1, 5), (1, 3, 2), (5, 2, 2)]:
        toks = _brute_tokens(F, HH, WW)
        S, P = F * HH * WW, HH * WW
        t = np.arange(S)
        for w in (0, 1, 2, 7):
            sp = O.mask_spatial(t, t, P, w)
            tp = O.mask_temporal(t, t, P, w)
            for (tq, fq, pq, _, _) in toks:
                for (tk, fk, pk, _, _) in toks:
                    assert sp[tq, tk] == (abs(fq - fk) <= w)
                    assert tp[tq, tk] == (abs(pq - pk) <= w)


def _nnz_closed(n_groups, group, w):
    """Pairs allowed by a band of +-w groups, each group `group` tokens."""
    per = sum(min(n_groups - 1, g + w) - max(0, g - w) + 1 for g in range(n_groups))
    return group * group * per


def pin_mask_nnz_closed_form():
    for (F, HH, WW, w_f, w_p) in [(13, 6, 9, 1, 8), (7, 5, 5, 2, 3), (4, 8, 8, 1, 2)]:
        P, S = HH * WW, F * HH * WW
        t = np.arange(S)
        nsp = sum(int(O.mask_rows(O.SPATIAL, t[i:i + 512], S, P, w_f, w_p).sum()) for i in range(0, S, 512))
        ntp = sum(int(O.mask_rows(O.TEMPORAL, t[i:i + 512], S, P, w_f, w_p).sum()) for i in range(0, S, 512))
        assert nsp == _nnz_closed(F, P, w_f)
        assert ntp == _nnz_closed(P, F, w_p)
        if w_f == 1 and F >= 2:
            assert nsp == P * P * (3 * F - 2)


def pin_mask_row_counts_720p():
    """Sampled rows of the 720p grid (F=33, 45x80): per-row counts equal the band widths."""
    F, HH, WW, w_f, w_p = 33, 45, 80, 1, 64
    P, S = HH * WW, F * HH * WW
    rows = _rng(5).choice(S, 64, replace=False)
    rows = np.concatenate([rows, [0, S - 1, P - 1, P, S - P]])
    sp = O.mask_rows(O.SPATIAL, rows, S, P, w_f, w_p).sum(axis=1)
    tp = O.mask_rows(O.TEMPORAL, rows, S, P, w_f, w_p).sum(axis=1)
    for r, a, b in zip(rows, sp, tp):
        f, p = divmod(int(r), P)
        assert a == P * (min(F - 1, f + w_f) - max(0, f - w_f) + 1)
        assert b == F * (min(P - 1, p + w_p) - max(0, p - w_p) + 1)
    # whole-grid densities from the closed form: about 9% spatial, 3.6% temporal at this shape
    assert abs(_nnz_closed(F, P, w_f) / S ** 2 - 0.08907) < 5e-5
    assert abs(_nnz_closed(P, F, w_p) / S ** 2 - 0.03551) < 5e-5


# --------------------------------------------------------------------------------- permutation
def pin_perm_golden_and_closed_form():
    with open(os.path.join(GOLDEN, "perm_small.txt")) as fh:
        want = [int(v) for line in fh if not line.startswith("#") and line.strip() for v in line.split()]
    assert list(O.perm_indices(2, 3)) == want
    for (F, P) in [(2, 3), (5, 7), (33, 3600), (1, 9), (9, 1)]:
        pi = O.perm_indices(F, P)
        u = np.arange(F * P)
        p, f = u // F, u % F
        assert (pi == f * P + p).all()
        inv = O.inverse_perm(pi)
        t = np.arange(F * P)
        assert (inv == (t % P) * F + t // P).all()
        assert (pi[inv] == t).all() and (inv[pi] == t).all()


def pin_permute_roundtrip():
    F, P, D = 4, 6, 3
    x = _rng(1).standard_normal((2, 3, F * P, D))
    y = O.permute(x, F, P)
    pi = O.perm_indices(F, P)
    assert np.array_equal(y[..., 5, :], x[..., pi[5], :])
    assert np.array_equal(O.unpermute(y, F, P), x)
    # location-contiguity: the F rows of one location are adjacent after the reorder
    for p in range(P):
        assert np.array_equal(y[0, 0, p * F:(p + 1) * F], x[0, 0, p::P])


# ---------------------------------------------------------------------------------- attention
def _sdpa(q, k, v, mask, scale):
    """torch's own scaled-dot-product attention in float64 on the CPU."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a))[None, None] for a in (q, k, v))
    m = torch.from_numpy(np.ascontiguousarray(mask))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale)[0, 0].numpy()


def pin_attention_vs_torch_sdpa():
    F, HH, WW, D = 5, 4, 6, 16
    P, S = HH * WW, F * HH * WW
    r = _rng(2)
    q, k, v = (r.standard_normal((S, D)) * 1.5 for _ in range(3))
    scale = O.default_scale(D)
    assert abs(scale - 0.25) < 1e-15
    for kind in (O.DENSE, O.SPATIAL, O.TEMPORAL):
        got = O.head_attention(q, k, v, kind, F, P, 1, 2, scale)
        m = O.mask_rows(kind, np.arange(S), S, P, 1, 2)
        want = _sdpa(q, k, v, m, scale)
        assert np.abs(got - want).max() < 1e-12, kind


def pin_attention_brute_force():
    F, HH, WW, D = 3, 2, 2, 4
    P, S = HH * WW, F * HH * WW
    r = _rng(3)
    q, k, v = (r.standard_normal((S, D)) for _ in range(3))
    toks = _brute_tokens(F, HH, WW)
    for kind, w in ((O.SPATIAL, 1), (O.TEMPORAL, 1), (O.DENSE, 0)):
        got = O.head_attention(q, k, v, kind, F, P, w, w, 0.5)
        for (tq, fq, pq, _, _) in toks:
            num = [0.0] * D
            den = 0.0
            allowed = []
            for (tk, fk, pk, _, _) in toks:
                ok = kind == O.DENSE or (kind == O.SPATIAL and abs(fq - fk) <= w) or \
                    (kind == O.TEMPORAL and abs(pq - pk) <= w)
                if ok:
                    allowed.append((tk, 0.5 * sum(q[tq, c] * k[tk, c] for c in range(D))))
            mx = max(s for _, s in allowed)
            for tk, s in allowed:
                e = math.exp(s - mx)
                den += e
                for c in range(D):
                    num[c] += e * v[tk, c]
            for c in range(D):
                assert abs(got[tq, c] - num[c] / den) < 1e-12


def pin_attention_invariants():
    F, HH, WW, D = 4, 3, 5, 8
    P, S = HH * WW, F * HH * WW
    r = _rng(4)
    q, k, v = (r.standard_normal((S, D)) * 2 for _ in range(3))
    sc = O.default_scale(D)
    # softmax rows sum to one: with V = 1 every output is 1
    for kind in (O.SPATIAL, O.TEMPORAL, O.DENSE):
        ones = O.head_attention(q, k, np.ones((S, D)), kind, F, P, 1, 2, sc)
        assert np.abs(ones - 1).max() < 1e-12
    # uniform logits (q = 0): output is the mean of the allowed value rows
    got = O.head_attention(np.zeros((S, D)), k, v, O.TEMPORAL, F, P, 1, 1, sc)
    for tq in (0, 7, S - 1):
        m = O.mask_rows(O.TEMPORAL, np.array([tq]), S, P, 1, 1)[0]
        assert np.abs(got[tq] - v[m].mean(axis=0)).max() < 1e-12
    # one allowed key: spatial with w_f = 0 on a 1x1 grid -> each token sees only itself
    got = O.head_attention(q[:F], k[:F], v[:F], O.SPATIAL, F, 1, 0, 0, sc)
    assert np.array_equal(got, v[:F])
    # windows that cover everything reduce to dense
    dense = O.head_attention(q, k, v, O.DENSE, F, P, 0, 0, sc)
    assert np.abs(O.head_attention(q, k, v, O.SPATIAL, F, P, F - 1, 0, sc) - dense).max() < 1e-12
    assert np.abs(O.head_attention(q, k, v, O.TEMPORAL, F, P, 0, P - 1, sc) - dense).max() < 1e-12
    # a single frame: the spatial head is dense
    one = slice(0, P)
    assert np.abs(O.head_attention(q[one], k[one], v[one], O.SPATIAL, 1, P, 1, 0, sc) -
                  O.head_attention(q[one], k[one], v[one], O.DENSE, 1, P, 1, 0, sc)).max() < 1e-12


def pin_layout_equivariance():
    """Permute -> attend under the permuted mask -> un-permute equals direct attention
    (the permutation statement of the SVG2 explainer, section 2A)."""
    F, HH, WW, D = 5, 3, 4, 8
    P, S = HH * WW, F * HH * WW
    r = _rng(6)
    q, k, v = (r.standard_normal((S, D)) * 2 for _ in range(3))
    for kind in (O.SPATIAL, O.TEMPORAL, O.DENSE):
        a = O.head_attention(q, k, v, kind, F, P, 1, 2, 0.3)
        b = O.head_attention_token_major(q, k, v, kind, F, P, 1, 2, 0.3)
        assert np.abs(a - b).max() < 1e-12


# ---------------------------------------------------------------------------------- block mask
def _block_mask_brute(kind, F, HH, WW, w_f, w_p, bm, bn):
    toks = _brute_tokens(F, HH, WW)
    S = len(toks)
    order = toks if kind != O.TEMPORAL else sorted(toks, key=lambda r: (r[2], r[1]))  # location-major
    nqb, nkb = -(-S // bm), -(-S // bn)
    out = np.zeros((nqb, nkb), dtype=np.uint8)
    for i, (_, fq, pq, _, _) in enumerate(order):
        for j, (_, fk, pk, _, _) in enumerate(order):
            ok = kind == O.DENSE or (kind == O.SPATIAL and abs(fq - fk) <= w_f) or \
                (kind == O.TEMPORAL and abs(pq - pk) <= w_p)
            if ok:
                out[i // bm, j // bn] = 1
    return out


def _block_runs(kind, F, P, w_f, w_p, bm, bn):
    """Interval form: rows of a band are contiguous in the head's layout."""
    S = F * P
    G, NG, w = (P, F, w_f) if kind == O.SPATIAL else (F, P, w_p)
    nqb, nkb = -(-S // bm), -(-S // bn)
    out = np.zeros((nqb, nkb), dtype=np.uint8)
    for i in range(nqb):
        r0, r1 = i * bm, min(S, (i + 1) * bm) - 1
        if kind == O.DENSE:
            lo, hi = 0, S
        else:
            lo = max(0, r0 // G - w) * G
            hi = min(NG, r1 // G + w + 1) * G
        out[i, lo // bn: -(-hi // bn)] = 1
    return out


def pin_block_mask_brute_force():
    for (F, HH, WW) in [(3, 2, 3), (4, 3, 2)]:
        for (bm, bn) in [(1, 1), (2, 3), (4, 4), (5, 7), (7, 5)]:
            for kind in (O.SPATIAL, O.TEMPORAL, O.DENSE):
                got = O.block_mask(kind, F, HH * WW, 1, 1, bm, bn)
                assert np.array_equal(got, _block_mask_brute(kind, F, HH, WW, 1, 1, bm, bn)), (F, bm, bn, kind)


def pin_block_mask_runs():
    for (F, HH, WW, w_f, w_p) in [(13, 6, 9, 1, 8), (5, 10, 13, 2, 20)]:
        P = HH * WW
        for (bm, bn) in [(128, 128), (128, 64), (64, 96), (100, 30)]:
            for kind in (O.SPATIAL, O.TEMPORAL, O.DENSE):
                got = O.block_mask(kind, F, P, w_f, w_p, bm, bn)
                assert np.array_equal(got, _block_runs(kind, F, P, w_f, w_p, bm, bn)), (kind, bm, bn)


# ---------------------------------------------------------------------------------- profiling
def pin_profile_brute_force():
    F, HH, WW, D = 3, 2, 2, 4
    P, S = HH * WW, F * HH * WW
    r = _rng(7)
    q, k, v = (r.standard_normal((1, 1, S, D)) * 2 for _ in range(3))
    idx = np.array([0, 5, 11])
    mse, kind = O.profile_heads(q, k, v, idx, F, P, 1, 0, 0.5)

    def row(tq, allow):
        s = [(tk, 0.5 * float(np.dot(q[0, 0, tq], k[0, 0, tk]))) for tk in range(S) if allow(tk)]
        mx = max(x for _, x in s)
        e = [(tk, math.exp(x - mx)) for tk, x in s]
        den = sum(x for _, x in e)
        return [sum(w * v[0, 0, tk, c] for tk, w in e) / den for c in range(D)]

    err = [0.0, 0.0]
    for tq in idx:
        full = row(tq, lambda tk: True)
        sp = row(tq, lambda tk: abs(tk // P - tq // P) <= 1)
        tp = row(tq, lambda tk: tk % P == tq % P)
        for c in range(D):
            err[0] += (sp[c] - full[c]) ** 2
            err[1] += (tp[c] - full[c]) ** 2
    err = [e / (len(idx) * D) for e in err]
    assert abs(mse[0, 0, 0] - err[0]) < 1e-13 and abs(mse[0, 0, 1] - err[1]) < 1e-13
    assert kind[0, 0] == (O.SPATIAL if err[0] <= err[1] else O.TEMPORAL)


def pin_profile_full_cover_and_ties():
    F, HH, WW, D = 4, 3, 3, 8
    P, S = HH * WW, F * HH * WW
    r = _rng(8)
    q, k, v = (r.standard_normal((1, 1, S, D)) * 2 for _ in range(3))
    idx = np.arange(0, S, 3)
    # spatial window covers every frame: its error is exactly zero and it is chosen
    mse, kind = O.profile_heads(q, k, v, idx, F, P, F - 1, 0, 0.35)
    assert mse[0, 0, 0] == 0.0 and mse[0, 0, 1] > 0 and kind[0, 0] == O.SPATIAL
    # temporal band covers every location: temporal error is zero and it is chosen
    mse, kind = O.profile_heads(q, k, v, idx, F, P, 0, P - 1, 0.35)
    assert mse[0, 0, 1] == 0.0 and mse[0, 0, 0] > 0 and kind[0, 0] == O.TEMPORAL
    # both cover everything: an exact tie goes to spatial
    mse, kind = O.profile_heads(q, k, v, idx, F, P, F - 1, P - 1, 0.35)
    assert mse[0, 0, 0] == mse[0, 0, 1] == 0.0 and kind[0, 0] == O.SPATIAL


def pin_profile_planted():
    """Heads built to correlate within a frame / within a location pick that kind."""
    from workloads import Geometry, Workload, make_qkv, expected_planted_kinds, bf16_to_f64
    wl = Workload("planted_small", Geometry(1, 6, 6, 6, 8, 64), 1, 4, 64, 11, 111, planted=True)
    q, k, v = make_qkv(wl)
    g = wl.geom
    idx = np.sort(_rng(9).choice(g.S, 64, replace=False))
    mse, kind = O.profile_heads(bf16_to_f64(q), bf16_to_f64(k), bf16_to_f64(v), idx, g.F, g.P, 1, 4, O.default_scale(64))
    assert np.array_equal(kind[0], expected_planted_kinds(wl)), (kind, expected_planted_kinds(wl), mse)


# ---------------------------------------------------------------------------------- norm / rope
def pin_rmsnorm_vs_torch():
    r = _rng(10)
    x = r.standard_normal((3, 5, 64)) * 3
    w = r.uniform(0.5, 1.5, 64)
    got = O.rms_norm(x, w, 1e-6)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(w), eps=1e-6).numpy()
    assert np.abs(got - want).max() < 1e-12
    y = O.rms_norm(x, np.ones(64), 1e-6)
    rms = np.sqrt(np.mean(y * y, axis=-1))
    ms = np.mean(x * x, axis=-1)
    assert np.abs(rms - np.sqrt(ms / (ms + 1e-6))).max() < 1e-12


def pin_rope_golden_angles():
    F, HH, WW, D = 3, 3, 5, 12
    assert O.rope_split(12) == (4, 4, 4)
    assert O.rope_split(128) == (44, 42, 42) and O.rope_split(64) == (24, 20, 20)
    rows = []
    with open(os.path.join(GOLDEN, "rope_angles.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                rows.append([float(v) for v in line.split()])
    S, P = F * HH * WW, HH * WW
    for (f, y, x, *angles) in rows:
        t = int(f) * P + int(y) * WW + int(x)
        for pair, ang in enumerate(angles):
            e = np.zeros((S, D))
            e[t, 2 * pair] = 1.0          # unit vector on the pair's first channel
            out = O.rope_3d(e, F, HH, WW, 10000.0)
            assert abs(out[t, 2 * pair] - math.cos(ang)) < 1e-12
            assert abs(out[t, 2 * pair + 1] - math.sin(ang)) < 1e-12


def pin_rope_invariants():
    F, HH, WW, D = 4, 3, 5, 24
    P, S = HH * WW, F * HH * WW
    r = _rng(11)
    x = r.standard_normal((S, D))
    y = O.rope_3d(x, F, HH, WW, 10000.0)
    assert np.abs(y[0] - x[0]).max() < 1e-15                        # position (0,0,0) is the identity
    pn = lambda a: a[:, 0::2] ** 2 + a[:, 1::2] ** 2
    assert np.abs(pn(y) - pn(x)).max() < 1e-12                      # each pair keeps its norm
    # scores depend on position differences only: shift both tokens by (1,1,1)
    qv, kv = r.standard_normal(D), r.standard_normal(D)
    def score(tq, tk):
        a = np.zeros((S, D)); a[tq] = qv
        b = np.zeros((S, D)); b[tk] = kv
        return float(O.rope_3d(a, F, HH, WW, 10000.0)[tq] @ O.rope_3d(b, F, HH, WW, 10000.0)[tk])
    tok = lambda f, yy, xx: f * P + yy * WW + xx
    assert abs(score(tok(0, 0, 1), tok(2, 1, 3)) - score(tok(1, 1, 2), tok(3, 2, 4))) < 1e-12
    # only the slice of the axis that changes is rotated differently
    a = y[tok(1, 1, 1)]; b = y[tok(1, 1, 2)]
    dt, dh, dw = O.rope_split(D)
    xa = O.rope_3d(np.tile(x[0], (S, 1)), F, HH, WW, 10000.0)
    assert np.abs(xa[tok(1, 1, 1), :dt + dh] - xa[tok(1, 1, 2), :dt + dh]).max() < 1e-15
    assert np.abs(xa[tok(1, 1, 1), dt + dh:] - xa[tok(1, 1, 2), dt + dh:]).max() > 1e-3
    del a, b


def pin_rope_complex_form():
    """An independent formulation: pairs as complex numbers times exp(i*theta)."""
    F, HH, WW, D = 3, 4, 4, 36
    P, S = HH * WW, F * HH * WW
    x = _rng(12).standard_normal((2, S, D))
    got = O.rope_3d(x, F, HH, WW, 500.0)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = np.zeros((S, D // 2))
    dt, dh, dw = 36 - 24, 12, 12
    for t in range(S):
        f, rem = divmod(t, P)
        yy, xx = divmod(rem, WW)
        pos = [f] * (dt // 2) + [yy] * (dh // 2) + [xx] * (dw // 2)
        jj = list(range(dt // 2)) + list(range(dh // 2)) + list(range(dw // 2))
        nn = [dt] * (dt // 2) + [dh] * (dh // 2) + [dw] * (dw // 2)
        theta[t] = [p * 500.0 ** (-2.0 * j / n) for p, j, n in zip(pos, jj, nn)]
    zr = z * np.exp(1j * theta)
    want = np.empty_like(x)
    want[..., 0::2], want[..., 1::2] = zr.real, zr.imag
    assert np.abs(got - want).max() < 1e-12


def _norm_rope_row_loop(row, w, eps, f, yy, xx, D, base):
    """One token row through RMSNorm then 3D RoPE, written as plain scalar loops.

    The slice widths and pairing are restated here from the readings (frame slice
    D - 4*floor(D/6), row and column slices 2*floor(D/6) each; interleaved pairs),
    not taken from the oracle.
    """
    ss = 0.0
    for c in range(D):
        ss += float(row[c]) * float(row[c])
    inv = 1.0 / math.sqrt(ss / D + eps)
    y = [float(row[c]) * inv * float(w[c]) for c in range(D)]
    third = 2 * (D // 6)
    out = list(y)
    off = 0
    for width, pos in ((D - 2 * third, f), (third, yy), (third, xx)):
        for j in range(width // 2):
            th = pos * base ** (-2.0 * j / width)
            a, b = y[off + 2 * j], y[off + 2 * j + 1]
            out[off + 2 * j] = a * math.cos(th) - b * math.sin(th)
            out[off + 2 * j + 1] = a * math.sin(th) + b * math.cos(th)
        off += width
    return out


def pin_qknorm_rope_row_loop():
    """QK-Norm then RoPE, Q with its own weight and K with its own, against scalar loops.

    The weights differ inside every rotated pair, so rotating before normalising
    (or exchanging the two weight vectors) changes the result.
    """
    F, HH, WW, D = 3, 2, 4, 24
    P, S = HH * WW, F * HH * WW
    r = _rng(15)
    q = r.standard_normal((1, 2, S, D)) * 2.5
    k = r.standard_normal((1, 2, S, D)) * 0.7
    wq = r.uniform(0.5, 1.5, D)
    wk = r.uniform(0.5, 1.5, D)
    eps = 1e-6
    gq, gk = O.qknorm_rope(q, k, wq, wk, eps, F, HH, WW, 10000.0)
    for h in range(2):
        for t in range(S):
            f, rem = divmod(t, P)
            yy, xx = divmod(rem, WW)
            wantq = _norm_rope_row_loop(q[0, h, t], wq, eps, f, yy, xx, D, 10000.0)
            wantk = _norm_rope_row_loop(k[0, h, t], wk, eps, f, yy, xx, D, 10000.0)
            assert np.abs(gq[0, h, t] - wantq).max() < 1e-12, (h, t)
            assert np.abs(gk[0, h, t] - wantk).max() < 1e-12, (h, t)


# ----------------------------------------------------------------------------- choice checker
def pin_choices_agree_hand_cases():
    """The head-choice comparison: equal kinds agree; different kinds agree only inside
    a relative gap of 1e-6 of the larger reference error."""
    sp, tp = O.SPATIAL, O.TEMPORAL
    kinds = lambda *v: np.array(v, dtype=np.uint8)
    # equal choices agree whatever the errors
    assert O.choices_agree(kinds(sp, tp), kinds(sp, tp), np.array([[1.0, 2.0], [3.0, 0.5]])).all()
    # a clear disagreement (10% apart) is reported
    got = O.choices_agree(kinds(sp, tp), kinds(tp, tp), np.array([[1.0, 1.1], [3.0, 0.5]]))
    assert got.tolist() == [False, True]
    # 5e-7 relative apart: a near tie, either choice accepted
    assert O.choices_agree(kinds(tp), kinds(sp), np.array([[1.0, 1.0 + 5e-7]])).all()
    # 2e-6 relative apart: not a tie
    assert not O.choices_agree(kinds(tp), kinds(sp), np.array([[1.0, 1.0 + 2e-6]])).any()
    # the gap is relative to the LARGER error: d = 1.0000005e-6 is within 1e-6 of 1 + d
    # but not within 1e-6 of 1
    d = 1.0000005e-6
    assert O.choices_agree(kinds(tp), kinds(sp), np.array([[1.0, 1.0 + d]])).all()
    assert O.choices_agree(kinds(sp), kinds(tp), np.array([[1.0 + d, 1.0]])).all()
    # the relative rule scales: errors of 1e-20 and 1.1e-20 are 10% apart
    assert not O.choices_agree(kinds(sp), kinds(tp), np.array([[1e-20, 1.1e-20]])).any()
    # both errors zero: an exact tie
    assert O.choices_agree(kinds(sp), kinds(tp), np.array([[0.0, 0.0]])).all()
    # shapes [B, H] are kept
    out = O.choices_agree(np.zeros((2, 3), np.uint8), np.ones((2, 3), np.uint8), np.ones((2, 3, 2)))
    assert out.shape == (2, 3) and out.all()


# -------------------------------------------------------------------------------------- step
def pin_full_step_consistency():
    from workloads import Geometry, Workload, make_qkv, bf16_to_f64, norm_weights
    wl = Workload("step_small", Geometry(1, 4, 4, 4, 6, 64), 1, 3, 32, 13, 113, planted=True, norm_rope=True)
    g = wl.geom
    q, k, v = (bf16_to_f64(t) for t in make_qkv(wl))
    wq, wk = norm_weights(g.D, wl.seed)
    idx = np.sort(_rng(14).choice(g.S, 32, replace=False))
    sc = O.default_scale(g.D)
    q2, k2, mse, kind, out = O.full_step(q, k, v, idx, g.F, g.HH, g.WW, 1, 3, sc, norm=(wq, wk, 1e-6, 10000.0))
    qn, kn = O.qknorm_rope(q, k, wq, wk, 1e-6, g.F, g.HH, g.WW, 10000.0)
    assert np.array_equal(q2, qn) and np.array_equal(k2, kn)
    m2, k2_ = O.profile_heads(qn, kn, v, idx, g.F, g.P, 1, 3, sc)
    assert np.array_equal(kind, k2_) and np.array_equal(mse, m2)
    for h in range(g.H):
        want = O.head_attention_token_major(qn[0, h], kn[0, h], v[0, h], int(kind[0, h]), g.F, g.P, 1, 3, sc)
        assert np.abs(out[0, h] - want).max() < 1e-12


ALL_PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_") and callable(v)]


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()
