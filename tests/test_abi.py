"""The C-ABI library loads on any machine and exports exactly what include/svg.h declares.

No call here reaches a kernel launch: every call carries an argument the host-side checks
reject before anything is enqueued.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svg.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svg_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def svg():
    import spatial_temporal_sparse_amd as m
    return m


def test_header_declares_the_path():
    names = _declared_functions()
    for n in ("svg_qknorm_rope", "svg_profile_heads", "svg_permute", "svg_unpermute", "svg_build_block_mask",
              "svg_sparse_attn", "svg_dense_attn", "svg_layer", "svg_dense_step", "svg_workspace_bytes",
              "svg_tile_shape", "svg_status_string", "svg_last_error", "svg_kmeans", "svg_centroid_topp",
              "svg_cluster_attn", "svg_dense_attn_lse", "svg_block_mass", "svg_block_select",
              "svg_block_sparse_attn"):
        assert n in names


def test_library_exports_every_declared_symbol(svg):
    lib = ctypes.CDLL(svg.LIB_PATH)
    for n in _declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", svg.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(_declared_functions()) <= exported
    assert not [s for s in exported if s.startswith("svg_") and s not in _declared_functions()]


def test_status_strings(svg):
    for code, tag in ((0, "SVG_OK"), (-1, "SVG_ERR_INVALID"), (-2, "SVG_ERR_UNSUPPORTED"), (-3, "SVG_ERR_HIP"),
                      (-4, "SVG_ERR_WORKSPACE")):
        assert svg.lib.svg_status_string(code).decode().startswith(tag)
    assert "unknown" in svg.lib.svg_status_string(7).decode()


def test_tile_shape(svg):
    assert svg.tile_shape() == (128, 64)


def test_workspace_sizes(svg):
    g = svg.Geom(1, 24, 33, 45, 80, 128)
    # the head order (24 int32, padded to 256 bytes), then 256 bytes of per-XCD work counters
    assert svg.workspace_bytes(svg.OP_SPARSE_ATTN, g) == 512
    ws = svg.workspace_bytes(svg.OP_PROFILE, g, 64)
    assert ws > 0 and ws % 256 == 0
    assert svg.workspace_bytes(svg.OP_PROFILE, g, 0) == 0                  # n_q out of range
    assert svg.workspace_bytes(svg.OP_PROFILE, svg.Geom(1, 24, 33, 45, 80, 96), 64) == 0   # D unsupported
    assert svg.workspace_bytes(99, g, 64) == 0
    # a layer runs profiling and attention one after the other on one workspace
    assert svg.workspace_bytes(svg.OP_LAYER, g, 64) == max(ws, 512)
    assert svg.workspace_bytes(svg.OP_LAYER, g, 0) == 0


def test_dense_step_schedule(svg):
    # the first quarter of the steps (step < 0.25 * n_steps) run dense
    assert [svg.dense_step(s, 4) for s in range(4)] == [True, False, False, False]
    assert [s for s in range(50) if svg.dense_step(s, 50)] == list(range(13))
    assert not any(svg.dense_step(s, 8, 0.0) for s in range(8))
    assert all(svg.dense_step(s, 8, 1.0) for s in range(8))
    for bad in ((4, 4, 0.25), (-1, 4, 0.25), (0, 0, 0.25), (0, 4, 1.5), (0, 4, -0.1)):
        assert svg.lib.svg_dense_step(*bad) == -1


FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: each call below fails a host check first


def test_argument_checks(svg):
    L = svg.lib
    W = svg.Windows
    good = svg.Geom(1, 2, 4, 8, 8, 64)
    # null pointers
    assert L.svg_permute(None, FAKE, 2, None, 1, good, None) == -1
    assert "src" in L.svg_last_error().decode()
    # geometry fields must be positive
    assert L.svg_permute(FAKE, ctypes.c_void_p(0x200000), 2, None, 1, svg.Geom(1, 2, 0, 8, 8, 64), None) == -1
    # element size
    assert L.svg_permute(FAKE, ctypes.c_void_p(0x800000), 3, None, 1, good, None) == -1
    # misaligned pointer
    assert L.svg_permute(ctypes.c_void_p(0x100002), ctypes.c_void_p(0x800000), 2, None, 1, good, None) == -1
    # overlapping src / dst
    assert L.svg_unpermute(FAKE, ctypes.c_void_p(0x100010), 2, None, 1, good, None) == -1
    # unsupported head dim
    assert L.svg_dense_attn(FAKE, FAKE, FAKE, svg.Geom(1, 2, 4, 8, 8, 96), 0.1, FAKE, None) == -2
    # non-positive scale
    assert L.svg_dense_attn(FAKE, FAKE, FAKE, good, 0.0, FAKE, None) == -1
    # negative window
    assert L.svg_build_block_mask(FAKE, good, W(-1, 2), 128, 64, FAKE, None) == -1
    # empty tile
    assert L.svg_build_block_mask(FAKE, good, W(1, 2), 0, 64, FAKE, None) == -1
    # n_q out of range and missing workspace
    assert L.svg_profile_heads(FAKE, FAKE, FAKE, FAKE, 0, good, W(1, 2), 0.125, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert L.svg_profile_heads(FAKE, FAKE, FAKE, FAKE, 64, good, W(1, 2), 0.125, FAKE, FAKE, None, 0, None) == -4
    assert L.svg_profile_heads(FAKE, FAKE, FAKE, FAKE, 64, good, W(1, 2), 0.125, FAKE, FAKE, FAKE, 16, None) == -4
    # sparse attention with kinds needs the token-major tensors and a workspace
    assert L.svg_sparse_attn(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, good, W(1, 2), 0.125, FAKE, FAKE, FAKE, 256,
                             None) == -1
    assert L.svg_sparse_attn(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, good, W(1, 2), 0.125, FAKE, FAKE, None, 0,
                             None) == -4
    # all four token-major tensors NULL selects the fused layout transformation: only the
    # workspace is missing here
    assert L.svg_sparse_attn(FAKE, FAKE, FAKE, None, None, None, FAKE, good, W(1, 2), 0.125, FAKE, None, None, 0,
                             None) == -4
    # a head must fit in 4 GB (S * D * 2 bytes)
    big = svg.Geom(1, 1, 1 << 5, 1 << 10, 1 << 10, 128)
    assert L.svg_dense_attn(FAKE, FAKE, FAKE, big, 0.1, FAKE, None) == -2
    assert L.svg_sparse_attn(FAKE, FAKE, FAKE, None, None, None, FAKE, big, W(1, 2), 0.125, FAKE, None, FAKE,
                             1 << 20, None) == -2
    assert L.svg_profile_heads(FAKE, FAKE, FAKE, FAKE, 64, big, W(1, 2), 0.125, FAKE, FAKE, FAKE, 1 << 20,
                               None) == -2
    # svg_layer checks every stage before it enqueues any: here the norm stage is valid and the
    # profiling stage is not, and the call returns that stage's status
    F2, F3, F4 = (ctypes.c_void_p(a) for a in (0x200000, 0x300000, 0x400000))
    assert L.svg_layer(FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, 1e4, 24, 20, 20, F2, F3, FAKE, 0, good, W(1, 2), 0.125, 0,
                       F4, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert L.svg_layer(FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, 1e4, 24, 20, 20, F2, F3, FAKE, 64, good, W(1, 2), 0.125, 0,
                       F4, FAKE, FAKE, FAKE, 16, None) == -4
    # normalised outputs are required when the norm runs, and the rope slices must fit D
    assert L.svg_layer(FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, 1e4, 24, 20, 20, None, F3, FAKE, 64, good, W(1, 2), 0.125, 1,
                       F4, None, None, None, 0, None) == -1
    assert L.svg_layer(FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, 1e4, 24, 22, 20, F2, F3, FAKE, 64, good, W(1, 2), 0.125, 1,
                       F4, None, None, None, 0, None) == -1
    # a dense layer still needs its output and a positive scale
    assert L.svg_layer(FAKE, FAKE, FAKE, None, None, 0.0, 0.0, 0, 0, 0, None, None, None, 0, good, W(0, 0), 0.125, 1,
                       None, None, None, None, 0, None) == -1
    assert L.svg_layer(FAKE, FAKE, FAKE, None, None, 0.0, 0.0, 0, 0, 0, None, None, None, 0, good, W(0, 0), 0.0, 1,
                       F4, None, None, None, 0, None) == -1
    # rope slices must be even and add up to D; eps must be positive
    assert L.svg_qknorm_rope(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, 1e4, 24, 21, 19, good, None) == -1
    assert L.svg_qknorm_rope(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.0, 1e4, 24, 20, 20, good, None) == -1
    # sequence too long
    assert L.svg_dense_attn(FAKE, FAKE, FAKE, svg.Geom(1, 1, 1 << 16, 1 << 8, 1 << 8, 64), 0.1, FAKE, None) == -1


def test_binding_rejects_host_tensors(svg):
    import torch
    x = torch.zeros((1, 2, 256, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        svg.permute(x, 4, 8, 8)
    with pytest.raises(ValueError):
        svg.geometry(x, 4, 8, 9)


def test_clustering_workspace_sizes(svg):
    g = svg.Geom(1, 24, 33, 45, 80, 128)
    S = 33 * 45 * 80
    km = svg.workspace_bytes(svg.OP_KMEANS, g, 512)
    # bf16 centroids + half norms + per-chunk counts, each rounded up to 256 bytes
    want = 24 * 512 * 128 * 2 + 24 * 512 * 4 + -(-(24 * (-(-S // 256)) * 512 * 4) // 256) * 256
    assert km == want
    assert svg.workspace_bytes(svg.OP_KMEANS, g, 0) == 0
    assert svg.workspace_bytes(svg.OP_KMEANS, g, 4097) == 0
    ca = svg.workspace_bytes(svg.OP_CLUSTER_ATTN, g, 128)
    assert ca >= 24 * 128 * S * 4                                      # one key list per query cluster
    assert svg.workspace_bytes(svg.OP_CLUSTER_ATTN, g, 0) == 0


def test_clustering_argument_checks(svg):
    L = svg.lib
    good = svg.Geom(1, 2, 4, 8, 8, 64)
    F2 = ctypes.c_void_p(0x200000)
    big_ws = 1 << 30
    # cluster count out of range, iterations out of range, workspace missing
    assert L.svg_kmeans(FAKE, good, 0, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, big_ws, None) == -1
    assert L.svg_kmeans(FAKE, good, 257, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, big_ws, None) == -1
    assert L.svg_kmeans(FAKE, good, 16, 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, big_ws, None) == -1
    assert L.svg_kmeans(FAKE, good, 16, 3, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -4
    assert L.svg_kmeans(FAKE, good, 16, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, 64, None) == -4
    assert L.svg_kmeans(None, good, 16, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, big_ws, None) == -1
    assert L.svg_kmeans(FAKE, svg.Geom(1, 2, 4, 8, 8, 96), 16, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, big_ws, None) == -2
    # top-p: p in (0, 1], at most 1024 key clusters
    assert L.svg_centroid_topp(FAKE, FAKE, FAKE, good, 8, 16, 0.125, 0.0, FAKE, None) == -1
    assert L.svg_centroid_topp(FAKE, FAKE, FAKE, good, 8, 16, 0.125, 1.5, FAKE, None) == -1
    assert L.svg_centroid_topp(FAKE, FAKE, FAKE, svg.Geom(1, 2, 40, 8, 8, 64), 8, 1025, 0.125, 0.9, FAKE, None) == -1
    assert L.svg_centroid_topp(FAKE, FAKE, FAKE, good, 8, 16, -1.0, 0.9, FAKE, None) == -1
    # cluster attention: cluster counts and workspace
    assert L.svg_cluster_attn(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, good, 0, 16, 0.125, F2, FAKE, big_ws,
                              None) == -1
    assert L.svg_cluster_attn(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, good, 8, 16, 0.125, F2, None, 0,
                              None) == -4
    assert L.svg_cluster_attn(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, good, 8, 16, 0.125, F2, FAKE, big_ws,
                              None) == -1


def test_block_path_workspace_and_checks(svg):
    L = svg.lib
    g = svg.Geom(1, 24, 33, 45, 80, 128)
    nqb, nkb = svg.block_grid(118800)
    assert (nqb, nkb) == (465, 1857)
    assert svg.workspace_bytes(svg.OP_BLOCK_ATTN, g) == -(-(24 * nqb * nkb * 4) // 256) * 256 + -(-(24 * nqb * 4) // 256) * 256
    # more than 4096 key blocks
    big = svg.Geom(1, 1, 8, 256, 129, 64)
    assert svg.workspace_bytes(svg.OP_BLOCK_ATTN, big) == 0
    small = svg.Geom(1, 2, 4, 8, 8, 64)
    F2 = ctypes.c_void_p(0x200000)
    assert L.svg_block_mass(FAKE, FAKE, FAKE, big, 0.125, F2, None) == -2
    assert L.svg_block_mass(FAKE, FAKE, None, small, 0.125, F2, None) == -1
    assert L.svg_block_select(FAKE, small, 0.0, F2, None) == -1
    assert L.svg_block_select(FAKE, small, 1.5, F2, None) == -1
    assert L.svg_block_sparse_attn(FAKE, FAKE, FAKE, FAKE, small, 0.125, F2, None, 0, None) == -4
    assert L.svg_block_sparse_attn(FAKE, FAKE, FAKE, FAKE, small, 0.0, F2, FAKE, 1 << 20, None) == -1
    assert L.svg_dense_attn_lse(FAKE, FAKE, FAKE, small, 0.125, F2, None, None) == -1


def test_layer_noalloc_rejects_oversized_requests(svg):
    """svg_layer_noalloc refuses, on the host and before any device call, a layer whose
    workspace would not fit its static scratch, and a bad sample size."""
    from ctypes import c_void_p
    fake = c_void_p(1 << 20)       # aligned, never dereferenced: the checks fail first
    big = svg.Geom(1, 4096, 1, 8, 8, 128)
    need = svg.workspace_bytes(svg.OP_LAYER, big, 64)
    assert need > svg.NOALLOC_SCRATCH_BYTES
    st = svg.lib.svg_layer_noalloc(fake, fake, fake, None, None, 1e-6, 1e4, 44, 42, 42, None, None, fake, 64, big,
                                   svg.Windows(1, 2), 0.088, 0, fake, fake, fake, None)
    assert st == -4 and b"scratch" in svg.lib.svg_last_error()
    small = svg.Geom(1, 2, 2, 8, 8, 128)
    assert svg.workspace_bytes(svg.OP_LAYER, small, 64) <= svg.NOALLOC_SCRATCH_BYTES
    st = svg.lib.svg_layer_noalloc(fake, fake, fake, None, None, 1e-6, 1e4, 44, 42, 42, None, None, fake, 0, small,
                                   svg.Windows(1, 2), 0.088, 0, fake, fake, fake, None)
    assert st == -1
    bad_d = svg.Geom(1, 2, 2, 8, 8, 96)
    st = svg.lib.svg_layer_noalloc(fake, fake, fake, None, None, 1e-6, 1e4, 32, 32, 32, None, None, fake, 64, bad_d,
                                   svg.Windows(1, 2), 0.088, 0, fake, fake, fake, None)
    assert st == -2


def test_noalloc_scratch_size_matches_header(svg):
    text = open(HEADER).read()
    m = re.search(r"#define SVG_LAYER_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == svg.NOALLOC_SCRATCH_BYTES


def test_rope_split_and_default_scale(svg):
    assert svg.rope_split(128) == (44, 42, 42) and svg.rope_split(64) == (24, 20, 20)
    assert svg.rope_split(6) == (2, 2, 2) and svg.rope_split(12) == (4, 4, 4)
    for D in range(6, 257, 2):
        dt, dh, dw = svg.rope_split(D)
        assert dt + dh + dw == D and dt % 2 == dh % 2 == dw % 2 == 0 and dh == dw and 0 <= dt - dh <= 4
    import ctypes
    x = ctypes.c_int32()
    for bad in (4, 7, 0, -2):
        assert svg.lib.svg_rope_split(bad, ctypes.byref(x), ctypes.byref(x), ctypes.byref(x)) == -1
    assert svg.lib.svg_rope_split(128, None, ctypes.byref(x), ctypes.byref(x)) == -1
    assert abs(svg.default_scale(128) - 128 ** -0.5) < 1e-8 and svg.default_scale(64) == 0.125
    assert svg.default_scale(0) == 0.0
