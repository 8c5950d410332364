"""Seeded synthetic inputs for the spatial/temporal sparse attention path.

This module only draws random numbers and arranges them into tensors of the
video-DiT shapes below; it holds none of the method's arithmetic (no masks,
no softmax, no norm, no rotary embedding, no profiling).  Both the CPU oracle
side and the GPU side of the tests, and the benchmark, take their inputs from
here, so the two sides always see identical bf16 values.

Shapes follow the token grids of the models the Sparse VideoGen pages name
(CogVideoX, Wan 2.1, HunyuanVideo at 720p).  No model weights, prompts or
videos exist here: Q/K/V are random activations with a planted per-head
structure so that some heads prefer the spatial mask and others the temporal
mask:

* a "spatial-planted" head adds one shared random vector per (head, frame) to
  every Q and K row of that frame, so queries correlate with keys of their own
  frame;
* a "temporal-planted" head adds one shared random vector per (head, in-frame
  position) to every Q and K row at that position, so queries correlate with
  keys at the same location in every frame.

V is unstructured N(0, 1).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

SPATIAL = 0
TEMPORAL = 1
DENSE = 2


@dataclasses.dataclass(frozen=True)
class Geometry:
    """Batch B, heads H, a token grid of F frames x HH rows x WW columns, head dim D."""
    B: int
    H: int
    F: int
    HH: int
    WW: int
    D: int

    @property
    def P(self) -> int:
        return self.HH * self.WW

    @property
    def S(self) -> int:
        return self.F * self.HH * self.WW


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    geom: Geometry
    w_f: int              # spatial window: frames either side
    w_p: int              # temporal band: in-frame positions either side
    n_q: int              # profiled query count
    seed: int             # Q/K/V seed
    idx_seed: int         # query-sample seed
    planted: bool         # plant spatial/temporal structure
    plant_scale: float = 2.0
    norm_rope: bool = False
    rope_base: float = 10000.0
    eps: float = 1e-6


# The five workloads: the tiny case the oracle finishes in seconds, three
# model-shaped token grids, and the full per-layer step at the 720p grid.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", Geometry(1, 2, 4, 8, 8, 64), 1, 2, 64, 1, 101, planted=False),
    "cogvideox": Workload("cogvideox", Geometry(1, 48, 13, 30, 45, 64), 1, 8, 64, 2, 102, planted=True),
    "wan": Workload("wan", Geometry(1, 40, 21, 30, 52, 128), 1, 8, 64, 3, 103, planted=True, norm_rope=True),
    "hunyuan720p": Workload("hunyuan720p", Geometry(1, 24, 33, 45, 80, 128), 1, 64, 64, 4, 104, planted=True),
    "hunyuan720p_step": Workload("hunyuan720p_step", Geometry(1, 24, 33, 45, 80, 128), 1, 64, 64, 50, 150,
                                 planted=True, norm_rope=True),
    # the 4-frame sub-grid of the 720p step, small enough for the oracle in full
    "hunyuan720p_f4": Workload("hunyuan720p_f4", Geometry(1, 24, 4, 45, 80, 128), 1, 64, 64, 60, 160,
                               planted=True, norm_rope=True),
}


def planted_kinds(H: int, seed: int) -> np.ndarray:
    """Seeded half/half assignment of heads to planted kinds (uint8 [H])."""
    rng = np.random.default_rng(seed + 7919)
    order = rng.permutation(H)
    kinds = np.full(H, TEMPORAL, dtype=np.uint8)
    kinds[order[: H // 2]] = SPATIAL
    return kinds


def sample_queries(S: int, n_q: int, seed: int) -> np.ndarray:
    """Uniform sample of n_q distinct query rows of [0, S), int32, one set per call."""
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(S, size=n_q, replace=False)).astype(np.int32)


def norm_weights(D: int, seed: int):
    """Two learned-weight stand-ins ~ U(0.5, 1.5), fp32 [D] each (for Q and for K)."""
    rng = np.random.default_rng(seed + 31)
    wq = rng.uniform(0.5, 1.5, size=D).astype(np.float32)
    wk = rng.uniform(0.5, 1.5, size=D).astype(np.float32)
    return wq, wk


def _plant(x: torch.Tensor, geom: Geometry, kinds: np.ndarray, u_sp: torch.Tensor, u_tp: torch.Tensor,
           scale: float) -> None:
    """In place: x[b, h] += scale * shared vector of the row's group (frame or position)."""
    B, H, F, P, D = geom.B, geom.H, geom.F, geom.P, geom.D
    xv = x.view(B, H, F, P, D)
    for h in range(H):
        if kinds[h] == SPATIAL:
            xv[:, h] += scale * u_sp[h].view(1, F, 1, D)
        else:
            xv[:, h] += scale * u_tp[h].view(1, 1, P, D)


def make_qkv(wl: Workload, device: str = "cpu", layer: int = 0, dtype=torch.bfloat16, step: int = 0):
    """Q, K, V as [B, H, S, D] tensors of `dtype` (bf16 by default; RNE from fp32).

    Values are drawn in fp32 with a seeded generator on `device` and cast once.
    On "cpu" the draw is bit-reproducible everywhere; on a GPU it is
    reproducible for a given device type.  `layer` offsets the seed so that
    each layer of a multi-layer step gets fresh activations.  `step` > 0 redraws
    the N(0, 1) part (a later denoising step of the same layer) and keeps the
    planted per-head vectors and kinds.
    """
    g = wl.geom
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed * 1000 + layer)
    shape = (g.B, g.H, g.S, g.D)
    q = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    k = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if wl.planted:
        kinds = planted_kinds(g.H, wl.seed * 1000 + layer)
        u_sp = torch.randn((g.H, g.F, g.D), generator=gen, device=device, dtype=torch.float32)
        u_tp = torch.randn((g.H, g.P, g.D), generator=gen, device=device, dtype=torch.float32)
    if step > 0:
        gen.manual_seed((wl.seed * 1000 + layer) * 7919 + step)
        q.normal_(generator=gen)
        k.normal_(generator=gen)
        v.normal_(generator=gen)
    if wl.planted:
        _plant(q, g, kinds, u_sp, u_tp, wl.plant_scale)
        _plant(k, g, kinds, u_sp, u_tp, wl.plant_scale)
        del u_sp, u_tp
    return q.to(dtype), k.to(dtype), v.to(dtype)


def expected_planted_kinds(wl: Workload, layer: int = 0) -> Optional[np.ndarray]:
    if not wl.planted:
        return None
    return planted_kinds(wl.geom.H, wl.seed * 1000 + layer)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16 (or fp32) tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


# ----------------------------------------------------------------------------------------------
# Semantic workloads (Sparse VideoGen2): tokens carry a hidden semantic class
# ----------------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class SemanticWorkload:
    """Q/K/V whose rows belong to hidden semantic classes, for the clustering path.

    Every token gets one of `n_classes` classes from a seeded map of coarse
    image regions (blocks of `region` rows x columns) that is redrawn every
    `frames_per_draw` frames, so a class is a set of scattered patches, as an
    object's tokens are.  Q and K rows of class z are N(0, I) plus `strength`
    times one shared random vector of (head, z); V is N(0, I).
    """
    name: str
    geom: Geometry
    n_classes: int
    strength: float
    Cq: int               # query clusters
    Ck: int               # key clusters
    p: float              # top-p threshold
    iters: int            # k-means iterations of one call
    seed: int
    region: int = 5
    frames_per_draw: int = 4


SEMANTIC_WORKLOADS: Dict[str, SemanticWorkload] = {
    # small enough for the oracle in full
    "svg2_small": SemanticWorkload("svg2_small", Geometry(1, 2, 4, 8, 10, 64), 4, 0.8, 8, 16, 0.9, 4, 21,
                                   region=3, frames_per_draw=2),
    # the 720p token grid of the spatial/temporal workloads
    "hunyuan720p_svg2": SemanticWorkload("hunyuan720p_svg2", Geometry(1, 24, 33, 45, 80, 128), 8, 0.8, 128, 512,
                                         0.9, 3, 22),
}


def semantic_classes(wl: SemanticWorkload) -> np.ndarray:
    """int64 [H, S]: hidden class of every frame-major token of each head."""
    g = wl.geom
    rng = np.random.default_rng(wl.seed + 4099)
    nfd = -(-g.F // wl.frames_per_draw)
    ny, nx = -(-g.HH // wl.region), -(-g.WW // wl.region)
    draw = rng.integers(0, wl.n_classes, size=(g.H, nfd, ny, nx))
    f = np.arange(g.F) // wl.frames_per_draw
    y = np.arange(g.HH) // wl.region
    x = np.arange(g.WW) // wl.region
    z = draw[:, f[:, None, None], y[None, :, None], x[None, None, :]]
    return z.reshape(g.H, g.S).astype(np.int64)


def make_qkv_semantic(wl: SemanticWorkload, device: str = "cpu", step: int = 0, dtype=torch.bfloat16):
    """Q, K, V [B, H, S, D] (bf16 by default) with the hidden classes of semantic_classes().

    `step` redraws the noise (a later denoising step) while the classes and their
    vectors stay, so that centroids of one step are a warm start for the next.
    """
    g = wl.geom
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed * 1000)
    mu = torch.randn((g.H, wl.n_classes, g.D), generator=gen, device=device, dtype=torch.float32)
    gen.manual_seed(wl.seed * 1000 + 1 + step)
    shape = (g.B, g.H, g.S, g.D)
    q = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    k = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    z = torch.from_numpy(semantic_classes(wl)).to(device)
    for h in range(g.H):
        add = wl.strength * mu[h][z[h]]
        q[:, h] += add
        k[:, h] += add
        del add
    return q.to(dtype), k.to(dtype), v.to(dtype)


def init_token_indices(S: int, C: int, seed: int) -> np.ndarray:
    """C distinct token indices of [0, S) (int32, sorted) whose rows start a cold k-means."""
    rng = np.random.default_rng(seed + 7)
    return np.sort(rng.choice(S, size=C, replace=False)).astype(np.int32)
