"""One full layer of the path on the GPU against the oracle, stage by stage.

Each stage is compared on the exact bf16 values the GPU stage consumed: norm/RoPE on the
layer inputs, profiling and attention on the GPU's normalised Q/K (bf16) and V.
"""
import numpy as np
import pytest
import torch

import oracle.svg_oracle as O
from tests.gpu_util import assert_close_attn, bf16_ulp, host64, note
from workloads import WORKLOADS, expected_planted_kinds, make_qkv, norm_weights, sample_queries

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _layer(gpu, wl, layer=0):
    g = wl.geom
    q, k, v = make_qkv(wl, device=DEV, layer=layer)
    idx = sample_queries(g.S, wl.n_q, wl.idx_seed + layer)
    norm = None
    if wl.norm_rope:
        wq, wk = norm_weights(g.D, wl.seed)
        norm = (torch.from_numpy(wq).to(DEV), torch.from_numpy(wk).to(DEV), wl.eps, wl.rope_base)
    o, kind, mse, qn, kn = gpu.sparse_layer(q, k, v, torch.from_numpy(idx).to(DEV), g.F, g.HH, g.WW, wl.w_f, wl.w_p,
                                            norm=norm)
    torch.cuda.synchronize()
    return q, k, v, idx, norm, o, kind.cpu().numpy(), mse.cpu().numpy(), qn, kn


def _check_layer(gpu, wl, rows_per_head, heads=None, layer=0, planted_expected=True):
    g = wl.geom
    q, k, v, idx, norm, o, kind, mse, qn, kn = _layer(gpu, wl, layer)
    sc = O.default_scale(g.D)
    heads = range(g.H) if heads is None else heads
    rng = np.random.default_rng(99 + layer)
    if norm is not None:
        wq, wk = norm_weights(g.D, wl.seed)
        for h in list(heads)[:2]:
            for src, w, out in ((q, wq, qn), (k, wk, kn)):
                want = O.rope_3d(O.rms_norm(host64(src[0, h]), w.astype(np.float64), wl.eps), g.F, g.HH, g.WW,
                                 wl.rope_base)
                pair = np.repeat(np.hypot(want[:, 0::2], want[:, 1::2]), 2, axis=1)
                assert (np.abs(host64(out[0, h]) - want) <= bf16_ulp(want) + 1e-6 + 2.0 ** -20 * pair).all()
    # profiling on what the GPU profiled
    for h in heads:
        qh, kh, vh = host64(qn[0, h]), host64(kn[0, h]), host64(v[0, h])
        a, c, kd = O.profile_head(qh, kh, vh, idx, g.F, g.P, wl.w_f, wl.w_p, sc)
        assert O.choices_agree(np.array([kind[0, h]]), np.array([kd]), np.array([[a, c]]), 1e-6).all(), \
            (h, kind[0, h], kd, a, c, mse[0, h])
        # sparse attention output under the chosen kind, rows sampled plus both ends
        rows = np.unique(np.concatenate([rng.choice(g.S, rows_per_head, replace=False), np.arange(0, 64),
                                         np.arange(g.S - 64, g.S)]))
        want = O.head_attention_rows(qh, kh, vh, rows, int(kind[0, h]), g.F, g.P, wl.w_f, wl.w_p, sc)
        assert_close_attn(host64(o[0, h])[rows], want, f"{wl.name} head {h} kind {kind[0, h]}")
    exp = expected_planted_kinds(wl, layer)
    if exp is not None and planted_expected:
        assert np.array_equal(kind[0], exp), (kind[0], exp)


def test_step_720p_subgrid_4_frames(gpu):
    wl = WORKLOADS["hunyuan720p_f4"]
    note(f"full layer {wl.name} {wl.geom}")
    # With only 4 frames the +-1 frame spatial window already holds 5/8 of all keys, so the
    # spatial mask wins for temporal-planted heads too; only agreement with the oracle counts.
    _check_layer(gpu, wl, rows_per_head=192, planted_expected=False)


def test_step_720p_full_grid(gpu):
    wl = WORKLOADS["hunyuan720p"]
    note(f"full layer {wl.name} {wl.geom}")
    _check_layer(gpu, wl, rows_per_head=24, heads=range(0, wl.geom.H, 3))


def test_step_wan_shape_with_norm(gpu):
    """The Wan-like grid (40 heads, 21 x 30 x 52 tokens, norm + RoPE): every head's profiling
    choice and sampled output rows, with the first and last 64 rows of each head."""
    wl = WORKLOADS["wan"]
    note(f"full layer {wl.name} {wl.geom}")
    _check_layer(gpu, wl, rows_per_head=24)


def test_step_cogvideox_shape(gpu):
    """The CogVideoX-like grid (48 heads, 13 x 30 x 45 tokens, D = 64): every head's profiling
    choice and sampled output rows, with the first and last 64 rows of each head."""
    wl = WORKLOADS["cogvideox"]
    note(f"full layer {wl.name} {wl.geom}")
    _check_layer(gpu, wl, rows_per_head=24)


@pytest.mark.parametrize("layer", [1, 2, 3])
def test_step_720p_subgrid_later_layers(gpu, layer):
    """Layers 1-3 of the four-layer step on fresh inputs (4-frame sub-grid of the 720p layer)."""
    wl = WORKLOADS["hunyuan720p_f4"]
    note(f"full layer {wl.name} layer {layer}")
    _check_layer(gpu, wl, rows_per_head=48, heads=range(layer, wl.geom.H, 4), layer=layer, planted_expected=False)


# The benchmarked layer itself: the 720p grid with QK-RMSNorm + 3D RoPE over 33 frames, four
# layers of fresh inputs, run through svg_layer (norm, profiling, block-sparse attention with
# the fused layout transformation), on exactly the inputs the benchmark generates.
BENCHED = [  # layer, heads, sampled output rows per head
    (0, range(0, 12), 256),
    (0, range(12, 24), 256),
    (1, range(0, 24), 64),
    (2, range(0, 24), 64),
    (3, range(0, 24), 64),
]


@pytest.mark.parametrize("layer,heads,n_rows", BENCHED,
                         ids=[f"layer{l}_heads{h.start}-{h.stop - 1}" for l, h, _ in BENCHED])
def test_benched_720p_step_layer(gpu, layer, heads, n_rows):
    wl = WORKLOADS["hunyuan720p_step"]
    g = wl.geom
    note(f"benched layer {wl.name} layer {layer} heads {heads.start}-{heads.stop - 1} {g}")
    q, k, v = make_qkv(wl, device=DEV, layer=layer)
    idx = sample_queries(g.S, wl.n_q, wl.idx_seed + layer)
    wq, wk = norm_weights(g.D, wl.seed)
    norm = (torch.from_numpy(wq).to(DEV), torch.from_numpy(wk).to(DEV), wl.eps, wl.rope_base)
    o, kind, mse, qn, kn = gpu.layer(q, k, v, torch.from_numpy(idx).to(DEV), g.F, g.HH, g.WW, wl.w_f, wl.w_p,
                                     norm=norm)
    # the benchmark's own call sequence (separate stage calls, fused layout) gives the same bits
    o2, kind2, _, _, _ = gpu.sparse_layer(q, k, v, torch.from_numpy(idx).to(DEV), g.F, g.HH, g.WW, wl.w_f, wl.w_p,
                                          norm=norm, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(kind2, kind) and torch.equal(o2, o)
    del o2
    kind, mse = kind.cpu().numpy(), mse.cpu().numpy()
    sc = O.default_scale(g.D)
    # norm + RoPE: every row of two heads, frames 0..32 of the rotation table
    if layer == 0:
        for h in list(heads)[:1] + list(heads)[-1:]:
            for src, w, out in ((q, wq, qn), (k, wk, kn)):
                want = O.rope_3d(O.rms_norm(host64(src[0, h]), w.astype(np.float64), wl.eps), g.F, g.HH, g.WW,
                                 wl.rope_base)
                pair = np.repeat(np.hypot(want[:, 0::2], want[:, 1::2]), 2, axis=1)
                bad = np.abs(host64(out[0, h]) - want) > bf16_ulp(want) + 1e-6 + 2.0 ** -20 * pair
                assert not bad.any(), f"norm/RoPE head {h}: {bad.sum()} elements off"
    pi = O.perm_indices(g.F, g.P)
    rng = np.random.default_rng(500 + layer)
    ends = np.arange(256)
    for h in heads:
        qh, kh, vh = host64(qn[0, h]), host64(kn[0, h]), host64(v[0, h])
        a, c, kd = O.profile_head(qh, kh, vh, idx, g.F, g.P, wl.w_f, wl.w_p, sc)
        assert O.choices_agree(np.array([kind[0, h]]), np.array([kd]), np.array([[a, c]]), 1e-6).all(), \
            (layer, h, kind[0, h], kd, a, c, mse[0, h])
        # the first and last 256-row query block of the head's working layout, plus random rows
        blocks = np.concatenate([ends, g.S - 256 + ends])
        if kind[0, h] == O.TEMPORAL:
            blocks = pi[blocks]
        rows = np.unique(np.concatenate([rng.choice(g.S, n_rows, replace=False), blocks]))
        want = O.head_attention_rows(qh, kh, vh, rows, int(kind[0, h]), g.F, g.P, wl.w_f, wl.w_p, sc)
        assert_close_attn(host64(o[0, h])[rows], want, f"layer {layer} head {h} kind {kind[0, h]}")
