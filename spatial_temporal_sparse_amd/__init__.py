"""Python binding of libsvg: Sparse VideoGen's spatial/temporal sparse 3D attention on MI355X.

Argument marshalling only.  Every step of the path runs in the HIP kernels of libsvg.so;
PyTorch supplies device memory and the current HIP stream.  Importing this package loads
the library and raises ImportError if it has not been built
(``python spatial_temporal_sparse_amd/build.py``); there is no fallback.

Tensors are [B, H, S, D] bf16, contiguous, on one HIP device, with S = F * HH * WW tokens
in frame-major order (t = f*HH*WW + y*WW + x) unless a function says token-major.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvg.so")

SPATIAL = 0
TEMPORAL = 1
DENSE = 2
OP_PROFILE = 1
OP_SPARSE_ATTN = 2
OP_LAYER = 3
OP_KMEANS = 4
OP_CLUSTER_ATTN = 5
# size of svg_layer_noalloc's static per-device scratch (SVG_LAYER_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20
OP_BLOCK_ATTN = 6
BLOCK_Q = 256
BLOCK_K = 64

_c_i32 = ctypes.c_int32
_c_vp = ctypes.c_void_p


class Geom(ctypes.Structure):
    _fields_ = [("B", _c_i32), ("H", _c_i32), ("F", _c_i32), ("HH", _c_i32), ("WW", _c_i32), ("D", _c_i32)]


class Windows(ctypes.Structure):
    _fields_ = [("frames", _c_i32), ("positions", _c_i32)]


class SvgError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} [status {status}]")
        self.status = status


_st = _c_i32
# result and argument types of every exported call
_SIGNATURES = {
    "svg_qknorm_rope": (_st, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_float, ctypes.c_float,
                             _c_i32, _c_i32, _c_i32, Geom, _c_vp]),
    "svg_profile_heads": (_st, [_c_vp, _c_vp, _c_vp, _c_vp, _c_i32, Geom, Windows, ctypes.c_float, _c_vp, _c_vp,
                               _c_vp, ctypes.c_size_t, _c_vp]),
    "svg_permute": (_st, [_c_vp, _c_vp, _c_i32, _c_vp, _c_i32, Geom, _c_vp]),
    "svg_unpermute": (_st, [_c_vp, _c_vp, _c_i32, _c_vp, _c_i32, Geom, _c_vp]),
    "svg_build_block_mask": (_st, [_c_vp, Geom, Windows, _c_i32, _c_i32, _c_vp, _c_vp]),
    "svg_sparse_attn": (_st, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, Geom, Windows, ctypes.c_float,
                             _c_vp, _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "svg_dense_attn": (_st, [_c_vp, _c_vp, _c_vp, Geom, ctypes.c_float, _c_vp, _c_vp]),
    "svg_layer": (_st, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_float, ctypes.c_float, _c_i32, _c_i32, _c_i32,
                       _c_vp, _c_vp, _c_vp, _c_i32, Geom, Windows, ctypes.c_float, _c_i32, _c_vp, _c_vp, _c_vp,
                       _c_vp, ctypes.c_size_t, _c_vp]),
    "svg_layer_noalloc": (_st, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_float, ctypes.c_float, _c_i32, _c_i32,
                               _c_i32, _c_vp, _c_vp, _c_vp, _c_i32, Geom, Windows, ctypes.c_float, _c_i32, _c_vp,
                               _c_vp, _c_vp, _c_vp]),
    "svg_dense_step": (_c_i32, [_c_i32, _c_i32, ctypes.c_float]),
    "svg_kmeans": (_st, [_c_vp, Geom, _c_i32, _c_i32, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, ctypes.c_size_t,
                        _c_vp]),
    "svg_centroid_topp": (_st, [_c_vp, _c_vp, _c_vp, Geom, _c_i32, _c_i32, ctypes.c_float, ctypes.c_float, _c_vp,
                               _c_vp]),
    "svg_cluster_attn": (_st, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, Geom, _c_i32, _c_i32,
                              ctypes.c_float, _c_vp, _c_vp, ctypes.c_size_t, _c_vp]),
    "svg_dense_attn_lse": (_st, [_c_vp, _c_vp, _c_vp, Geom, ctypes.c_float, _c_vp, _c_vp, _c_vp]),
    "svg_block_mass": (_st, [_c_vp, _c_vp, _c_vp, Geom, ctypes.c_float, _c_vp, _c_vp]),
    "svg_block_select": (_st, [_c_vp, Geom, ctypes.c_float, _c_vp, _c_vp]),
    "svg_block_sparse_attn": (_st, [_c_vp, _c_vp, _c_vp, _c_vp, Geom, ctypes.c_float, _c_vp, _c_vp, ctypes.c_size_t,
                                   _c_vp]),
    "svg_workspace_bytes": (ctypes.c_size_t, [_c_i32, ctypes.POINTER(Geom), _c_i32]),
    "svg_tile_shape": (None, [ctypes.POINTER(_c_i32), ctypes.POINTER(_c_i32)]),
    "svg_rope_split": (_st, [_c_i32, ctypes.POINTER(_c_i32), ctypes.POINTER(_c_i32), ctypes.POINTER(_c_i32)]),
    "svg_default_scale": (ctypes.c_float, [_c_i32]),
    "svg_status_string": (ctypes.c_char_p, [_c_i32]),
    "svg_last_error": (ctypes.c_char_p, []),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python {os.path.join(_HERE, 'build.py')}`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(status: int) -> None:
    if status != 0:
        raise SvgError(status, f"{lib.svg_status_string(status).decode()}: {lib.svg_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else _c_vp(t.data_ptr())


def _stream(t: torch.Tensor):
    return _c_vp(torch.cuda.current_stream(t.device).cuda_stream)


def _check_qkv(name: str, t: torch.Tensor, shape, dtype=torch.bfloat16, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def geometry(x: torch.Tensor, F: int, HH: int, WW: int) -> Geom:
    """The svg_geom of a [B, H, S, D] tensor laid out on an F x HH x WW token grid."""
    if x.dim() != 4:
        raise ValueError("expected a [B, H, S, D] tensor")
    B, H, S, D = x.shape
    if S != F * HH * WW:
        raise ValueError(f"S={S} does not equal F*HH*WW={F * HH * WW}")
    return Geom(B, H, F, HH, WW, D)


def _shape(g: Geom):
    return (g.B, g.H, g.F * g.HH * g.WW, g.D)


def default_scale(D: int) -> float:
    """The library's default softmax scale (svg_default_scale)."""
    return float(lib.svg_default_scale(int(D)))


def rope_split(D: int) -> Tuple[int, int, int]:
    """The library's default frame / row / column slice widths of the head dim (svg_rope_split)."""
    dt, dh, dw = _c_i32(), _c_i32(), _c_i32()
    _check(lib.svg_rope_split(int(D), ctypes.byref(dt), ctypes.byref(dh), ctypes.byref(dw)))
    return dt.value, dh.value, dw.value


def workspace_bytes(op: int, g: Geom, n_q: int = 0) -> int:
    return int(lib.svg_workspace_bytes(op, ctypes.byref(g), n_q))


def tile_shape() -> Tuple[int, int]:
    bm, bn = _c_i32(), _c_i32()
    lib.svg_tile_shape(ctypes.byref(bm), ctypes.byref(bn))
    return bm.value, bn.value


def _workspace(op: int, g: Geom, n_q: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    need = workspace_bytes(op, g, n_q)
    if ws is None:
        return torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    if ws.dtype != torch.uint8 or ws.device != device or not ws.is_contiguous() or ws.numel() < need:
        raise ValueError(f"workspace must be a contiguous uint8 tensor of >= {need} bytes on {device}")
    return ws


def qknorm_rope(q, k, wq, wk, F, HH, WW, eps=1e-6, rope_base=10000.0, dims=None, q_out=None, k_out=None):
    """QK-RMSNorm + 3D RoPE of q and k (svg_qknorm_rope). Returns (q_out, k_out)."""
    g = geometry(q, F, HH, WW)
    shp = _shape(g)
    _check_qkv("q", q, shp)
    _check_qkv("k", k, shp, device=q.device)
    _check_qkv("wq", wq, (g.D,), torch.float32, q.device)
    _check_qkv("wk", wk, (g.D,), torch.float32, q.device)
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    _check_qkv("q_out", q_out, shp, device=q.device)
    _check_qkv("k_out", k_out, shp, device=q.device)
    dt, dh, dw = rope_split(g.D) if dims is None else dims
    _check(lib.svg_qknorm_rope(_ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), _ptr(wq), _ptr(wk), float(eps),
                               float(rope_base), dt, dh, dw, g, _stream(q)))
    return q_out, k_out


def profile_heads(q, k, v, q_idx, F, HH, WW, w_f, w_p, scale=None, mse=None, kind=None, ws=None):
    """Per-head spatial/temporal choice from sampled query rows (svg_profile_heads).

    q_idx: int32 [n_q] device tensor of frame-major rows.  Returns (mse [B, H, 2] fp32,
    kind [B, H] uint8).
    """
    g = geometry(q, F, HH, WW)
    shp = _shape(g)
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_qkv(n, t, shp, device=q.device)
    if q_idx.dtype != torch.int32 or q_idx.dim() != 1 or q_idx.device != q.device or not q_idx.is_contiguous():
        raise ValueError("q_idx must be a contiguous int32 [n_q] tensor on the same device")
    n_q = q_idx.numel()
    mse = torch.empty((g.B, g.H, 2), dtype=torch.float32, device=q.device) if mse is None else mse
    kind = torch.empty((g.B, g.H), dtype=torch.uint8, device=q.device) if kind is None else kind
    _check_qkv("mse", mse, (g.B, g.H, 2), torch.float32, q.device)
    _check_qkv("kind", kind, (g.B, g.H), torch.uint8, q.device)
    ws = _workspace(OP_PROFILE, g, n_q, q.device, ws)
    sc = default_scale(g.D) if scale is None else scale
    _check(lib.svg_profile_heads(_ptr(q), _ptr(k), _ptr(v), _ptr(q_idx), n_q, g, Windows(w_f, w_p), float(sc),
                                 _ptr(mse), _ptr(kind), _ptr(ws), ws.numel(), _stream(q)))
    return mse, kind


def _perm(fn, x, F, HH, WW, kind, select, out):
    g = geometry(x, F, HH, WW)
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("permute supports bf16 and fp32 rows")
    _check_qkv("x", x, _shape(g), x.dtype)
    out = torch.empty_like(x) if out is None else out
    _check_qkv("out", out, _shape(g), x.dtype, x.device)
    if kind is not None:
        _check_qkv("kind", kind, (g.B, g.H), torch.uint8, x.device)
    fn(_ptr(x), _ptr(out), x.element_size(), _ptr(kind), int(select), g, _stream(x))
    return out


def permute(x, F, HH, WW, kind=None, select=TEMPORAL, out=None):
    """Frame-major -> token-major (svg_permute) for heads with kind == select (all if kind is None)."""
    return _perm(lambda *a: _check(lib.svg_permute(*a)), x, F, HH, WW, kind, select, out)


def unpermute(x, F, HH, WW, kind=None, select=TEMPORAL, out=None):
    """Token-major -> frame-major (svg_unpermute) for heads with kind == select (all if kind is None)."""
    return _perm(lambda *a: _check(lib.svg_unpermute(*a)), x, F, HH, WW, kind, select, out)


def build_block_mask(kind, F, HH, WW, w_f, w_p, bm, bn):
    """uint8 [B, H, ceil(S/bm), ceil(S/bn)] tile mask in each head's layout (svg_build_block_mask)."""
    if kind.dtype != torch.uint8 or kind.dim() != 2 or kind.device.type != "cuda" or not kind.is_contiguous():
        raise ValueError("kind must be a contiguous uint8 [B, H] device tensor")
    B, H = kind.shape
    g = Geom(B, H, F, HH, WW, 64)
    S = F * HH * WW
    out = torch.empty((B, H, -(-S // bm), -(-S // bn)), dtype=torch.uint8, device=kind.device)
    _check(lib.svg_build_block_mask(_ptr(kind), g, Windows(w_f, w_p), bm, bn, _ptr(out), _stream(kind)))
    return out


def sparse_attn(q, k, v, qt, kt, vt, kind, F, HH, WW, w_f, w_p, scale=None, o=None, ot=None, ws=None):
    """Block-sparse attention (svg_sparse_attn): spatial/dense heads read q/k/v and write o
    (frame-major); temporal heads read qt/kt/vt and write ot (token-major).  With qt, kt, vt
    all None the layout transformation is fused: temporal heads read q/k/v and write o too,
    and ot is None.  Returns (o, ot)."""
    g = geometry(q, F, HH, WW)
    shp = _shape(g)
    fused = qt is None and kt is None and vt is None
    if fused and ot is not None:
        raise ValueError("ot must be None when qt, kt and vt are None (fused layout transformation)")
    for n, t in (("q", q), ("k", k), ("v", v)) + (() if fused else (("qt", qt), ("kt", kt), ("vt", vt))):
        _check_qkv(n, t, shp, device=q.device)
    _check_qkv("kind", kind, (g.B, g.H), torch.uint8, q.device)
    o = torch.empty_like(q) if o is None else o
    if not fused:
        ot = torch.empty_like(q) if ot is None else ot
        _check_qkv("ot", ot, shp, device=q.device)
    _check_qkv("o", o, shp, device=q.device)
    ws = _workspace(OP_SPARSE_ATTN, g, 0, q.device, ws)
    sc = default_scale(g.D) if scale is None else scale
    _check(lib.svg_sparse_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(qt), _ptr(kt), _ptr(vt), _ptr(kind), g,
                               Windows(w_f, w_p), float(sc), _ptr(o), _ptr(ot), _ptr(ws), ws.numel(), _stream(q)))
    return o, ot


def dense_attn(q, k, v, F, HH, WW, scale=None, o=None):
    """Unmasked attention with the same kernel (svg_dense_attn)."""
    g = geometry(q, F, HH, WW)
    shp = _shape(g)
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_qkv(n, t, shp, device=q.device)
    o = torch.empty_like(q) if o is None else o
    _check_qkv("o", o, shp, device=q.device)
    sc = default_scale(g.D) if scale is None else scale
    _check(lib.svg_dense_attn(_ptr(q), _ptr(k), _ptr(v), g, float(sc), _ptr(o), _stream(q)))
    return o


class LayerBuffers:
    """Device buffers one sparse layer reuses across calls (token-major copies, outputs, workspaces)."""

    def __init__(self, like: torch.Tensor, n_q: int, F: int, HH: int, WW: int):
        g = geometry(like, F, HH, WW)
        dev = like.device
        self.qt, self.kt, self.vt, self.ot = (torch.empty_like(like) for _ in range(4))
        self.o = torch.empty_like(like)
        self.qn = torch.empty_like(like)
        self.kn = torch.empty_like(like)
        self.mse = torch.empty((g.B, g.H, 2), dtype=torch.float32, device=dev)
        self.kind = torch.empty((g.B, g.H), dtype=torch.uint8, device=dev)
        self.ws_profile = torch.empty(max(256, workspace_bytes(OP_PROFILE, g, n_q)), dtype=torch.uint8, device=dev)
        self.ws_attn = torch.empty(max(256, workspace_bytes(OP_SPARSE_ATTN, g, 0)), dtype=torch.uint8, device=dev)


def sparse_layer(q, k, v, q_idx, F, HH, WW, w_f, w_p, norm=None, scale=None, bufs: Optional[LayerBuffers] = None,
                 fused=False):
    """One layer of the path, all on the current stream with no host synchronisation:
    [QK-RMSNorm + 3D RoPE] -> profile heads -> token-major copies of temporal heads' Q/K/V ->
    block-sparse attention -> frame-major output.  fused=True leaves the layout transformation
    to the attention kernel's loads and stores (same result, no copies).

    norm: None or (wq, wk, eps, rope_base).  Returns (o, kind, mse, q', k').
    """
    if bufs is None:
        bufs = LayerBuffers(q, q_idx.numel(), F, HH, WW)
    if norm is not None:
        wq, wk, eps, base = norm
        q, k = qknorm_rope(q, k, wq, wk, F, HH, WW, eps, base, q_out=bufs.qn, k_out=bufs.kn)
    profile_heads(q, k, v, q_idx, F, HH, WW, w_f, w_p, scale, mse=bufs.mse, kind=bufs.kind, ws=bufs.ws_profile)
    if fused:
        sparse_attn(q, k, v, None, None, None, bufs.kind, F, HH, WW, w_f, w_p, scale, o=bufs.o, ws=bufs.ws_attn)
        return bufs.o, bufs.kind, bufs.mse, q, k
    permute(q, F, HH, WW, bufs.kind, TEMPORAL, out=bufs.qt)
    permute(k, F, HH, WW, bufs.kind, TEMPORAL, out=bufs.kt)
    permute(v, F, HH, WW, bufs.kind, TEMPORAL, out=bufs.vt)
    sparse_attn(q, k, v, bufs.qt, bufs.kt, bufs.vt, bufs.kind, F, HH, WW, w_f, w_p, scale, o=bufs.o, ot=bufs.ot,
                ws=bufs.ws_attn)
    unpermute(bufs.ot, F, HH, WW, bufs.kind, TEMPORAL, out=bufs.o)
    return bufs.o, bufs.kind, bufs.mse, q, k


def dense_step(step: int, n_steps: int, dense_fraction: float = 0.25) -> bool:
    """True if denoising step `step` of `n_steps` runs dense attention (svg_dense_step): the
    first dense_fraction of the steps do, i.e. steps with step < dense_fraction * n_steps."""
    r = int(lib.svg_dense_step(int(step), int(n_steps), float(dense_fraction)))
    if r < 0:
        _check(r)
    return r == 1


def _layer_args(q, k, v, q_idx, F, HH, WW, w_f, w_p, dense, norm, dims, scale, o, qn, kn, mse, kind):
    """Checked ctypes arguments of svg_layer / svg_layer_noalloc up to the workspace, and the
    outputs (o, kind, mse, q', k') the call writes."""
    g = geometry(q, F, HH, WW)
    shp = _shape(g)
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_qkv(n, t, shp, device=dev)
    if q_idx.dtype != torch.int32 or q_idx.dim() != 1 or q_idx.device != dev or not q_idx.is_contiguous():
        raise ValueError("q_idx must be a contiguous int32 [n_q] tensor on the same device")
    n_q = q_idx.numel()
    o = torch.empty_like(q) if o is None else o
    _check_qkv("o", o, shp, device=dev)
    mse = torch.empty((g.B, g.H, 2), dtype=torch.float32, device=dev) if mse is None else mse
    kind = torch.empty((g.B, g.H), dtype=torch.uint8, device=dev) if kind is None else kind
    _check_qkv("mse", mse, (g.B, g.H, 2), torch.float32, dev)
    _check_qkv("kind", kind, (g.B, g.H), torch.uint8, dev)
    wq = wk = None
    eps, base = 1e-6, 10000.0
    if norm is not None:
        wq, wk, eps, base = norm
        _check_qkv("wq", wq, (g.D,), torch.float32, dev)
        _check_qkv("wk", wk, (g.D,), torch.float32, dev)
        qn = torch.empty_like(q) if qn is None else qn
        kn = torch.empty_like(k) if kn is None else kn
        _check_qkv("qn", qn, shp, device=dev)
        _check_qkv("kn", kn, shp, device=dev)
    dt, dh, dw = rope_split(g.D) if dims is None else dims
    sc = default_scale(g.D) if scale is None else scale
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(wq), _ptr(wk), float(eps), float(base), dt, dh, dw, _ptr(qn), _ptr(kn),
            _ptr(q_idx), n_q, g, Windows(w_f, w_p), float(sc), int(bool(dense)), _ptr(o), _ptr(mse), _ptr(kind))
    outs = (o, kind, mse, (qn if norm is not None else q), (kn if norm is not None else k))
    return g, n_q, args, outs


def layer(q, k, v, q_idx, F, HH, WW, w_f, w_p, dense=False, norm=None, dims=None, scale=None, o=None, qn=None,
          kn=None, mse=None, kind=None, ws=None):
    """One attention layer in one library call (svg_layer): [QK-RMSNorm + 3D RoPE], then dense
    attention (dense=True) or profiling + block-sparse attention with the fused layout
    transformation.  norm: None or (wq, wk, eps, rope_base).  Returns (o, kind, mse, q', k'),
    where q', k' are what attention read; kind and mse are not written by a dense layer."""
    g, n_q, args, outs = _layer_args(q, k, v, q_idx, F, HH, WW, w_f, w_p, dense, norm, dims, scale, o, qn, kn, mse,
                                     kind)
    ws = _workspace(OP_LAYER, g, n_q, q.device, ws)
    _check(lib.svg_layer(*args, _ptr(ws), ws.numel(), _stream(q)))
    return outs


def layer_noalloc(q, k, v, q_idx, F, HH, WW, w_f, w_p, dense=False, norm=None, dims=None, scale=None, o=None,
                  qn=None, kn=None, mse=None, kind=None):
    """layer() through svg_layer_noalloc: the library's static per-device scratch instead of a
    workspace, so the call allocates nothing when every output buffer is passed in.  Calls
    that overlap on one device share that scratch and must not run concurrently."""
    _, _, args, outs = _layer_args(q, k, v, q_idx, F, HH, WW, w_f, w_p, dense, norm, dims, scale, o, qn, kn, mse,
                                   kind)
    _check(lib.svg_layer_noalloc(*args, _stream(q)))
    return outs


class StepDriver:
    """The attention layers of a denoising loop on one device.

    Each layer is one svg_layer call on the driver's static buffers: the caller writes the
    layer's inputs into `q`, `k`, `v` (bf16 [B, H, S, D], frame-major) and `q_idx` (int32
    [n_q] sampled rows), then calls `layer(step)`, which leaves the output in `o` (and, for a
    sparse step, the head kinds and errors in `kind`, `mse`).  Steps with
    dense_step(step, n_steps, dense_fraction) run dense attention, the others profile and run
    sparse attention.  With graphs=True the dense and the sparse layer are each captured once
    in a HIP graph (torch.cuda.CUDAGraph) on first use and replayed afterwards; nothing is
    allocated per layer either way.
    """

    def __init__(self, B, H, F, HH, WW, D, n_steps, w_f, w_p, n_q=64, norm=None, dense_fraction=0.25, scale=None,
                 graphs=False, device="cuda"):
        self.F, self.HH, self.WW = F, HH, WW
        self.n_steps, self.dense_fraction = int(n_steps), float(dense_fraction)
        self.w_f, self.w_p, self.scale = w_f, w_p, scale
        self.graphs = bool(graphs)
        dev = torch.device(device)
        shp = (B, H, F * HH * WW, D)
        self.q, self.k, self.v, self.o = (torch.zeros(shp, dtype=torch.bfloat16, device=dev) for _ in range(4))
        self.q_idx = torch.zeros((n_q,), dtype=torch.int32, device=dev)
        self.mse = torch.zeros((B, H, 2), dtype=torch.float32, device=dev)
        self.kind = torch.zeros((B, H), dtype=torch.uint8, device=dev)
        self.norm = None
        self.qn = self.kn = None
        if norm is not None:
            wq, wk, eps, base = norm
            self.norm = (wq.to(dev).contiguous(), wk.to(dev).contiguous(), float(eps), float(base))
            self.qn, self.kn = torch.empty_like(self.q), torch.empty_like(self.k)
        g = geometry(self.q, F, HH, WW)
        self.ws = torch.empty(max(256, workspace_bytes(OP_LAYER, g, n_q)), dtype=torch.uint8, device=dev)
        self._graph = {}

    def is_dense(self, step: int) -> bool:
        return dense_step(step, self.n_steps, self.dense_fraction)

    def _run(self, dense: bool) -> None:
        layer(self.q, self.k, self.v, self.q_idx, self.F, self.HH, self.WW, self.w_f, self.w_p, dense=dense,
              norm=self.norm, scale=self.scale, o=self.o, qn=self.qn, kn=self.kn, mse=self.mse, kind=self.kind,
              ws=self.ws)

    def layer(self, step: int):
        """Runs one layer of denoising step `step` on the static inputs; returns (o, kind, mse)."""
        dense = self.is_dense(step)
        if not self.graphs:
            self._run(dense)
            return self.o, self.kind, self.mse
        g = self._graph.get(dense)
        if g is None:
            self._run(dense)                      # eager first run (the graph is captured after it)
            torch.cuda.current_stream(self.q.device).synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._run(dense)
            self._graph[dense] = g
        g.replay()
        return self.o, self.kind, self.mse


# ----------------------------------------------------------------------------------------------
# Semantic clustering path (Sparse VideoGen2)
# ----------------------------------------------------------------------------------------------
class Clusters:
    """Output of kmeans(): centroids [B, H, C, D] fp32, labels / perm [B, H, S] int32 and
    offsets [B, H, C + 1] int32 (cluster c holds perm[..., offsets[c]:offsets[c + 1]])."""

    def __init__(self, centroids, labels, perm, offsets):
        self.centroids, self.labels, self.perm, self.offsets = centroids, labels, perm, offsets

    @property
    def C(self) -> int:
        return self.centroids.shape[2]


def kmeans(x, F, HH, WW, C, iters, init_idx=None, centroids=None, out: Optional[Clusters] = None, ws=None):
    """Lloyd k-means of the rows of x per (b, h) (svg_kmeans).

    Cold start from the rows at init_idx (int32 [C] device tensor), or a warm start from
    `centroids` (fp32 [B, H, C, D], updated in place) or from out.centroids.  Returns a
    Clusters (out, if given).
    """
    g = geometry(x, F, HH, WW)
    _check_qkv("x", x, _shape(g))
    dev = x.device
    S = g.F * g.HH * g.WW
    if init_idx is None and centroids is None and out is None:
        raise ValueError("kmeans needs init_idx (cold start), centroids or out (warm start)")
    if out is None:
        cent = centroids if centroids is not None else torch.empty((g.B, g.H, C, g.D), dtype=torch.float32, device=dev)
        out = Clusters(cent, torch.empty((g.B, g.H, S), dtype=torch.int32, device=dev),
                       torch.empty((g.B, g.H, S), dtype=torch.int32, device=dev),
                       torch.empty((g.B, g.H, C + 1), dtype=torch.int32, device=dev))
    elif centroids is not None and centroids.data_ptr() != out.centroids.data_ptr():
        out.centroids.copy_(centroids)
    _check_qkv("centroids", out.centroids, (g.B, g.H, C, g.D), torch.float32, dev)
    _check_qkv("labels", out.labels, (g.B, g.H, S), torch.int32, dev)
    _check_qkv("perm", out.perm, (g.B, g.H, S), torch.int32, dev)
    _check_qkv("offsets", out.offsets, (g.B, g.H, C + 1), torch.int32, dev)
    if init_idx is not None:
        _check_qkv("init_idx", init_idx, (C,), torch.int32, dev)
    ws = _workspace(OP_KMEANS, g, C, dev, ws)
    _check(lib.svg_kmeans(_ptr(x), g, C, iters, _ptr(init_idx), _ptr(out.centroids), _ptr(out.labels), _ptr(out.perm),
                          _ptr(out.offsets), _ptr(ws), ws.numel(), _stream(x)))
    return out


def centroid_topp(cq: Clusters, ck: Clusters, F, HH, WW, p, scale=None, sel=None):
    """Key clusters selected per query cluster (svg_centroid_topp): uint8 [B, H, Cq, Ck]."""
    B, H, Cq, D = cq.centroids.shape
    Ck = ck.C
    g = Geom(B, H, F, HH, WW, D)
    dev = cq.centroids.device
    _check_qkv("ck.centroids", ck.centroids, (B, H, Ck, D), torch.float32, dev)
    _check_qkv("ck.offsets", ck.offsets, (B, H, Ck + 1), torch.int32, dev)
    sel = torch.empty((B, H, Cq, Ck), dtype=torch.uint8, device=dev) if sel is None else sel
    _check_qkv("sel", sel, (B, H, Cq, Ck), torch.uint8, dev)
    sc = default_scale(D) if scale is None else scale
    _check(lib.svg_centroid_topp(_ptr(cq.centroids), _ptr(ck.centroids), _ptr(ck.offsets), g, Cq, Ck, float(sc),
                                 float(p), _ptr(sel), _stream(cq.centroids)))
    return sel


def cluster_attn(q, k, v, cq: Clusters, ck: Clusters, sel, F, HH, WW, scale=None, o=None, ws=None):
    """Attention of every query to the keys of its query cluster's selected key clusters
    (svg_cluster_attn).  Returns o [B, H, S, D] bf16 in the original token order."""
    g = geometry(q, F, HH, WW)
    shp = _shape(g)
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_qkv(n, t, shp, device=q.device)
    dev = q.device
    Cq, Ck = cq.C, ck.C
    S = shp[2]
    for n, t, sh in (("cq.perm", cq.perm, (g.B, g.H, S)), ("cq.offsets", cq.offsets, (g.B, g.H, Cq + 1)),
                     ("ck.perm", ck.perm, (g.B, g.H, S)), ("ck.offsets", ck.offsets, (g.B, g.H, Ck + 1))):
        _check_qkv(n, t, sh, torch.int32, dev)
    _check_qkv("sel", sel, (g.B, g.H, Cq, Ck), torch.uint8, dev)
    o = torch.empty_like(q) if o is None else o
    _check_qkv("o", o, shp, device=dev)
    ws = _workspace(OP_CLUSTER_ATTN, g, Cq, dev, ws)
    sc = default_scale(g.D) if scale is None else scale
    _check(lib.svg_cluster_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(cq.perm), _ptr(cq.offsets), _ptr(ck.perm),
                                _ptr(ck.offsets), _ptr(sel), g, Cq, Ck, float(sc), _ptr(o), _ptr(ws), ws.numel(),
                                _stream(q)))
    return o


class ClusterLayer:
    """One attention layer of the clustering path with its centroid cache.

    The first call clusters from the rows at the given token indices (a cold start); later
    calls start k-means from the previous call's centroids, the cache that carries from one
    denoising step to the next.  Buffers are allocated once.
    """

    def __init__(self, like: torch.Tensor, F, HH, WW, Cq, Ck, p, iters, init_q, init_k, scale=None):
        g = geometry(like, F, HH, WW)
        self.g, self.F, self.HH, self.WW = g, F, HH, WW
        self.Cq, self.Ck, self.p, self.iters = Cq, Ck, p, iters
        self.init_q, self.init_k = init_q, init_k
        self.scale = default_scale(g.D) if scale is None else scale
        dev = like.device
        S = F * HH * WW
        mk = lambda C: Clusters(torch.empty((g.B, g.H, C, g.D), dtype=torch.float32, device=dev),
                                torch.empty((g.B, g.H, S), dtype=torch.int32, device=dev),
                                torch.empty((g.B, g.H, S), dtype=torch.int32, device=dev),
                                torch.empty((g.B, g.H, C + 1), dtype=torch.int32, device=dev))
        self.cq, self.ck = mk(Cq), mk(Ck)
        self.sel = torch.empty((g.B, g.H, Cq, Ck), dtype=torch.uint8, device=dev)
        self.o = torch.empty_like(like)
        self.ws_km = torch.empty(max(256, workspace_bytes(OP_KMEANS, g, max(Cq, Ck))), dtype=torch.uint8, device=dev)
        self.ws_attn = torch.empty(max(256, workspace_bytes(OP_CLUSTER_ATTN, g, Cq)), dtype=torch.uint8, device=dev)
        self.warm = False

    def __call__(self, q, k, v):
        iq = None if self.warm else self.init_q
        ik = None if self.warm else self.init_k
        kmeans(q, self.F, self.HH, self.WW, self.Cq, self.iters, init_idx=iq, out=self.cq, ws=self.ws_km)
        kmeans(k, self.F, self.HH, self.WW, self.Ck, self.iters, init_idx=ik, out=self.ck, ws=self.ws_km)
        centroid_topp(self.cq, self.ck, self.F, self.HH, self.WW, self.p, self.scale, sel=self.sel)
        cluster_attn(q, k, v, self.cq, self.ck, self.sel, self.F, self.HH, self.WW, self.scale, o=self.o,
                     ws=self.ws_attn)
        self.warm = True
        return self.o


# ----------------------------------------------------------------------------------------------
# Head-adaptive block-sparse path with an LSE-cached block search
# ----------------------------------------------------------------------------------------------
def block_grid(S: int) -> Tuple[int, int]:
    """(query blocks, key blocks) of a sequence of S tokens."""
    return -(-S // BLOCK_Q), -(-S // BLOCK_K)


def dense_attn_lse(q, k, v, F, HH, WW, scale=None, o=None, lse=None):
    """Dense attention and each row's natural-log log-sum-exp (svg_dense_attn_lse).
    Returns (o [B, H, S, D] bf16, lse [B, H, S] fp32)."""
    g = geometry(q, F, HH, WW)
    shp = _shape(g)
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_qkv(n, t, shp, device=q.device)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(shp[:3], dtype=torch.float32, device=q.device) if lse is None else lse
    _check_qkv("o", o, shp, device=q.device)
    _check_qkv("lse", lse, shp[:3], torch.float32, q.device)
    sc = default_scale(g.D) if scale is None else scale
    _check(lib.svg_dense_attn_lse(_ptr(q), _ptr(k), _ptr(v), g, float(sc), _ptr(o), _ptr(lse), _stream(q)))
    return o, lse


def block_mass(q, k, lse, F, HH, WW, scale=None, mass=None):
    """Attention mass of every (256-row, 64-key) block under the cached lse (svg_block_mass).
    Returns fp32 [B, H, nqb, nkb]."""
    g = geometry(q, F, HH, WW)
    shp = _shape(g)
    _check_qkv("q", q, shp)
    _check_qkv("k", k, shp, device=q.device)
    _check_qkv("lse", lse, shp[:3], torch.float32, q.device)
    nqb, nkb = block_grid(shp[2])
    mass = torch.empty((g.B, g.H, nqb, nkb), dtype=torch.float32, device=q.device) if mass is None else mass
    _check_qkv("mass", mass, (g.B, g.H, nqb, nkb), torch.float32, q.device)
    sc = default_scale(g.D) if scale is None else scale
    _check(lib.svg_block_mass(_ptr(q), _ptr(k), _ptr(lse), g, float(sc), _ptr(mass), _stream(q)))
    return mass


def block_select(mass, F, HH, WW, D, coverage, sel=None):
    """Per query block, the fewest key blocks carrying `coverage` of its mass (svg_block_select).
    Returns uint8 [B, H, nqb, nkb]."""
    B, H, nqb, nkb = mass.shape
    g = Geom(B, H, F, HH, WW, D)
    if block_grid(F * HH * WW) != (nqb, nkb):
        raise ValueError("mass does not match the block grid of the token grid")
    _check_qkv("mass", mass, (B, H, nqb, nkb), torch.float32, mass.device)
    sel = torch.empty((B, H, nqb, nkb), dtype=torch.uint8, device=mass.device) if sel is None else sel
    _check_qkv("sel", sel, (B, H, nqb, nkb), torch.uint8, mass.device)
    _check(lib.svg_block_select(_ptr(mass), g, float(coverage), _ptr(sel), _stream(mass)))
    return sel


def block_sparse_attn(q, k, v, sel, F, HH, WW, scale=None, o=None, ws=None):
    """Attention of each query to the keys of its query block's chosen key blocks
    (svg_block_sparse_attn).  Returns o [B, H, S, D] bf16."""
    g = geometry(q, F, HH, WW)
    shp = _shape(g)
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_qkv(n, t, shp, device=q.device)
    nqb, nkb = block_grid(shp[2])
    _check_qkv("sel", sel, (g.B, g.H, nqb, nkb), torch.uint8, q.device)
    o = torch.empty_like(q) if o is None else o
    _check_qkv("o", o, shp, device=q.device)
    ws = _workspace(OP_BLOCK_ATTN, g, 0, q.device, ws)
    sc = default_scale(g.D) if scale is None else scale
    _check(lib.svg_block_sparse_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(sel), g, float(sc), _ptr(o), _ptr(ws),
                                     ws.numel(), _stream(q)))
    return o

