#!/usr/bin/env python3
"""Benchmark of the sparse 3D attention path at the HunyuanVideo-720p token grid on one MI355X.

A step is one layer of the path over one batch of synthetic activations already resident in
HBM: QK-RMSNorm + 3D RoPE -> per-head profiling on 64 sampled queries -> layout
transformation of the temporal heads -> block-sparse attention -> frame-major output.  With
--layout fused (the default) the attention kernel applies the layout transformation as it
loads and stores rows; with --layout explicit the step materialises token-major copies of
Q/K/V (svg_permute) and restores the output (svg_unpermute).  The other layout is timed too
(unless --no-compare) and reported under "compare".  Steps cycle over 4 layers of fresh
seeded inputs (B=1, H=24, F=33 x 45 x 80 tokens = 118800, D=128, bf16, half the heads
planted spatial and half temporal; w_f = 1 frame, w_p = 64 positions).

Prints one JSON line on stdout (progress goes to stderr).  `value` is the effective
attention throughput of the whole step: FLOPs of the attention tiles (4*D per query-key pair
of every 128x64 tile of the exported block mask, clipped at the sequence end) divided by the
step time.  The kernel's 256-row workgroups walk the union of two 128-row blocks' key runs,
about 2% more work at 720p, which this count leaves out.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_hunyuan720p_traffic.json")
CLUSTER_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "cluster_attn_hunyuan720p_svg2_traffic.json")
BLOCK_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "block_attn_hunyuan720p_blocks_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_busy_hunyuan720p.json")
HBM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_kernels_hunyuan720p_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=12)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--layout", choices=("fused", "explicit"), default="fused",
                    help="layout transformation of temporal heads inside the attention kernel, or as separate "
                         "permute / unpermute passes")
    ap.add_argument("--no-compare", action="store_true", help="do not also time the other layout")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU oracle leg (for profiler runs, which only need the GPU kernels)")
    ap.add_argument("--no-isolated", action="store_true",
                    help="skip the isolated timing of the HBM-bound kernels (MALL flushed before every launch)")
    ap.add_argument("--workload", choices=("hunyuan720p_step", "cogvideox", "wan", "hunyuan720p_svg2",
                                           "hunyuan720p_blocks"),
                    default="hunyuan720p_step",
                    help="token grid of the step (default: the HunyuanVideo-720p layer the headline is quoted on; "
                         "cogvideox and wan are the CogVideoX-like D=64 and the Wan-like grids; hunyuan720p_svg2 "
                         "times the semantic clustering path instead, on the 720p grid; hunyuan720p_blocks the head-adaptive "
                         "block-sparse path with an LSE-cached search)")
    ap.add_argument("--denoise", type=int, default=0, metavar="N",
                    help="instead: time the attention layers of an N-step denoising loop through the step driver "
                         "(dense attention for the first quarter of the steps, then profiling + sparse attention), "
                         "eager and with HIP-graph replay, and print that JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (the reference kernel that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "repeats": 3}), flush=True)


def tile_flops(svg, kind, g, w_f, w_p, bm, bn):
    """FLOPs of the 128x64 tiles of the library's exported block mask: each 128-row query block's
    run of key tiles.  The attention kernel's 256-row workgroups walk the union of two such runs,
    slightly more work (about 2% at 720p), which this count leaves out."""
    import torch
    mask = svg.build_block_mask(kind, g.F, g.HH, g.WW, w_f, w_p, bm, bn).to(torch.float64)
    S = g.S
    rows = torch.full((mask.shape[2],), float(bm), dtype=torch.float64, device=mask.device)
    rows[-1] = S - bm * (mask.shape[2] - 1)
    cols = torch.full((mask.shape[3],), float(bn), dtype=torch.float64, device=mask.device)
    cols[-1] = S - bn * (mask.shape[3] - 1)
    pairs = torch.einsum("bhij,i,j->", mask, rows, cols).item()
    return 4.0 * g.D * pairs


def token_flops(kind_np, g, w_f, w_p):
    """4*D per allowed (query, key) pair: the token-level work of the masks."""
    def band(n_groups, group, w):
        return group * group * sum(min(n_groups - 1, i + w) - max(0, i - w) + 1 for i in range(n_groups))
    per = {0: band(g.F, g.P, w_f), 1: band(g.P, g.F, w_p), 2: g.S * g.S}
    return 4.0 * g.D * sum(per[int(k)] for k in kind_np.ravel())


def kernel_sha(group="attn_fwd"):
    """Hash of the kernel code (comments and whitespace ignored) that stored counter figures were
    taken on (see rocprof_report.py, which writes them)."""
    import rocprof_report
    return rocprof_report.source_sha(group)


def _load_json(path):
    try:
        with open(path) as fh:
            return json.load(fh)
    except (OSError, ValueError):
        return None


def measured_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch of an attention kernel from the committed counter runs, if they were
    taken on the current kernel source; else None."""
    t = _load_json(path)
    if t is None or t.get("kernel_sha") != kernel_sha():
        return None
    return t.get("bytes_per_launch")


def measured_hbm_traffic():
    """HBM bytes per launch of the norm/RoPE, profiling and layout-transformation kernels from the
    committed counter runs, if taken on the current source; else {}."""
    t = _load_json(HBM_TRAFFIC_FILE)
    if t is None or t.get("kernel_sha") != kernel_sha("hbm"):
        return {}
    return {k: {"bytes_per_launch": round(v["bytes_per_launch"]), "algorithmic_bytes": v["algorithmic_bytes"]}
            for k, v in t.get("kernels", {}).items()}


def measured_mfma(which):
    """MFMA busy fraction and clock of the attention kernel at 720p from the committed counter runs
    (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE), if taken on the current source; else {}."""
    t = _load_json(MFMA_FILE)
    if t is None or t.get("kernel_sha") != kernel_sha():
        return {}
    k = t.get("kernels", {}).get(which)
    if k is None:
        return {}
    return {"mfma_busy": round(k["mfma_busy"], 3), "clock_ghz": round(k["clock_ghz"], 2)}


def host_cores():
    """CPU counts of this host: all cores, the ones this process may run on, and the BLAS
    threads numpy's matrix products use (the threads the oracle actually runs on)."""
    affinity = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl
        blas = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # threadpoolctl missing: numpy's BLAS defaults to the affinity size
        blas = affinity
    return {"cores": int(blas), "cpu_count": os.cpu_count(), "affinity": affinity, "blas_threads": int(blas)}


def cpu_baseline(q, k, v, kinds, g, w_f, w_p):
    """The fp64 oracle on a bounded sample of the same layer: 8192 query rows of one spatial
    and one temporal head against all S keys; token-level FLOPs / wall time."""
    import numpy as np
    import oracle.svg_oracle as O
    hc = host_cores()
    heads = [int(np.argmax(kinds == 0)), int(np.argmax(kinds == 1))]
    rng = np.random.default_rng(123)
    rows = np.sort(rng.choice(g.S, 8192, replace=False))
    sc = 1.0 / math.sqrt(g.D)
    flops = 0.0
    elapsed = 0.0
    for h in heads:
        f64 = lambda t: t[0, h].detach().cpu().double().numpy()
        qh, kh, vh = f64(q), f64(k), f64(v)
        kind = int(kinds[h])
        t0 = time.perf_counter()
        O.head_attention_rows(qh, kh, vh, rows, kind, g.F, g.P, w_f, w_p, sc)
        elapsed += time.perf_counter() - t0
        m = O.mask_rows(kind, rows, g.S, g.P, w_f, w_p)
        flops += 4.0 * g.D * float(m.sum())
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", **hc, "kind": "oracle",
            "sample": "fp64 numpy oracle, sparse attention of 8192 sampled query rows of one spatial and one "
                      f"temporal head of the layer (S={g.S}, D={g.D}) against all keys; token-level FLOPs",
            "seconds": round(elapsed, 2)}


def denoise(args):
    """Attention layers of an N-step denoising loop through svg.StepDriver (one svg_layer call,
    or one graph replay, per layer).  Inputs are copied into the driver's buffers outside the
    timed region, where a model's QKV projection would write them."""
    import numpy as np
    import torch

    import spatial_temporal_sparse_amd as svg
    from workloads import WORKLOADS, make_qkv, norm_weights, sample_queries

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = WORKLOADS["hunyuan720p_step"]
    g = wl.geom
    n_steps, L = args.denoise, max(1, args.layers)
    log(f"[denoise] {n_steps} steps x {L} layers of {g}")
    layers = []
    for l in range(L):
        q, k, v = make_qkv(wl, device="cuda", layer=l)
        layers.append((q, k, v))
    wq, wk = norm_weights(g.D, wl.seed)
    norm = (torch.from_numpy(wq).to(dev), torch.from_numpy(wk).to(dev), wl.eps, wl.rope_base)
    out = {}
    for graphs in (False, True):
        drv = svg.StepDriver(g.B, g.H, g.F, g.HH, g.WW, g.D, n_steps, wl.w_f, wl.w_p, n_q=wl.n_q, norm=norm,
                             graphs=graphs, device=dev)

        def loop(timed):
            per_step = []
            for s_ in range(n_steps):
                evs = []
                for l in range(L):
                    q, k, v = layers[l]
                    drv.q.copy_(q)
                    drv.k.copy_(k)
                    drv.v.copy_(v)
                    drv.q_idx.copy_(torch.from_numpy(sample_queries(g.S, wl.n_q, wl.idx_seed + s_ * L + l)))
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    drv.layer(s_)
                    e1.record()
                    evs.append((e0, e1))
                torch.cuda.synchronize()
                per_step.append(sum(a.elapsed_time(b) for a, b in evs))
            return per_step

        loop(False)                 # warm-up (and, with graphs, capture)
        per_step = loop(True)
        dense = [drv.is_dense(s_) for s_ in range(n_steps)]
        out[graphs] = (per_step, dense)
        log(f"[denoise] graphs={graphs}: {[round(x, 2) for x in per_step]} ms per step")
    per_step, dense = out[True]
    eager = out[False][0]
    d_ms = float(np.mean([t for t, d in zip(per_step, dense) if d])) if any(dense) else None
    s_ms = float(np.mean([t for t, d in zip(per_step, dense) if not d])) if not all(dense) else None
    mean = float(np.mean(per_step))
    res = {
        "metric": "denoising loop: attention ms per step (dense first quarter, then profiling + sparse), 720p shape",
        "value": round(mean, 3), "unit": "ms", "higher_is_better": False, "n_gpus": 1, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"hunyuan720p_step: {n_steps} denoising steps x {L} attention layers "
                               f"(QK-RMSNorm + 3D RoPE in every layer)", "dense_fraction": 0.25,
                   "dense_steps": int(sum(dense)), "B": g.B, "H": g.H, "F": g.F, "HH": g.HH, "WW": g.WW, "D": g.D,
                   "w_f": wl.w_f, "w_p": wl.w_p, "n_q": wl.n_q},
        "dense_step_ms": None if d_ms is None else round(d_ms, 3),
        "sparse_step_ms": None if s_ms is None else round(s_ms, 3),
        "graph_ms_per_step": round(mean, 3),
        "eager_ms_per_step": round(float(np.mean(eager)), 3),
        "speedup_vs_all_dense": None if d_ms is None else round(d_ms / mean, 3),
    }
    print(json.dumps(res), flush=True)


def cluster_flops(cq, ck, sel, D, tile_rows, tile_keys):
    """(token-level FLOPs, computed-tile FLOPs, mean density) of one clustering-path layer.

    Token level: 4*D per query and key of its selected clusters.  Computed tiles: every query
    cluster runs ceil(n/256) tiles of 256 rows over ceil(L/64) key tiles of 64.
    """
    import torch
    nq = (cq.offsets[..., 1:] - cq.offsets[..., :-1]).double()                # [B, H, Cq]
    nk = (ck.offsets[..., 1:] - ck.offsets[..., :-1]).double()                # [B, H, Ck]
    L = torch.einsum("bhij,bhj->bhi", sel.double(), nk)                      # keys per query cluster
    tok = 4.0 * D * float((nq * L).sum())
    tiles = torch.ceil(nq / tile_rows) * tile_rows * torch.ceil(L / tile_keys) * tile_keys
    S = nq.sum(dim=-1)                                                      # [B, H]
    density = float(((nq * L).sum(dim=-1) / (S * S)).mean())
    return tok, 4.0 * D * float(tiles.sum()), density


def cluster_cpu_baseline(q, k, v, lq, lk, sel, D):
    """The fp64 oracle's attention over the selected clusters for 4096 sampled query rows of one
    head of the layer (given the GPU's clusters and selection); token-level FLOPs / wall time."""
    import numpy as np
    import oracle.svg2_oracle as O2
    hc = host_cores()
    f64 = lambda t: t.detach().cpu().double().numpy()
    S = q.shape[2]
    rows = np.sort(np.random.default_rng(321).choice(S, 4096, replace=False))
    qh, kh, vh = f64(q[0, 0]), f64(k[0, 0]), f64(v[0, 0])
    lqh, lkh = lq[0, 0].cpu().numpy(), lk[0, 0].cpu().numpy()
    s = sel[0, 0].cpu().numpy().astype(bool)
    t0 = time.perf_counter()
    O2.semantic_attention_rows(qh, kh, vh, rows, lqh, lkh, s, 1.0 / math.sqrt(D))
    el = time.perf_counter() - t0
    pairs = float(O2.semantic_mask(lqh[rows], lkh, s).sum())
    return {"value": 4.0 * D * pairs / el / 1e12, "unit": "TFLOP/s", **hc, "kind": "oracle",
            "sample": f"fp64 numpy oracle, attention over the selected clusters of 4096 sampled query rows of one "
                      f"head (S={S}, D={D}) given the GPU's clusters and selection; token-level FLOPs",
            "seconds": round(el, 2)}


def cluster_bench(args):
    """The semantic clustering path at the 720p grid: per layer, k-means of Q and K warm-started
    from the previous step's centroids, centroid top-p selection, attention over the selected
    clusters.  Steps cycle over the layers; each layer keeps its own centroid cache."""
    import numpy as np
    import torch

    import spatial_temporal_sparse_amd as svg
    from workloads import SEMANTIC_WORKLOADS, init_token_indices, make_qkv_semantic

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = SEMANTIC_WORKLOADS[args.workload]
    g = wl.geom
    L = max(1, min(args.layers, 2))
    log(f"[bench] clustering path: {L} layers of {g}, Cq={wl.Cq} Ck={wl.Ck} p={wl.p} iters={wl.iters}")
    layers = []
    for l in range(L):
        q, k, v = make_qkv_semantic(wl, device="cuda", step=l)
        iq = torch.from_numpy(init_token_indices(g.S, wl.Cq, wl.seed + 10 * l)).to(dev)
        ik = torch.from_numpy(init_token_indices(g.S, wl.Ck, wl.seed + 10 * l + 1)).to(dev)
        layer = svg.ClusterLayer(q, g.F, g.HH, g.WW, wl.Cq, wl.Ck, wl.p, wl.iters, iq, ik)
        layers.append((q, k, v, layer))
    F, HH, WW = g.F, g.HH, g.WW

    def step(l, ev=None):
        q, k, v, ly = layers[l]
        if ev is not None:
            ev[0].record()
        svg.kmeans(q, F, HH, WW, wl.Cq, wl.iters, init_idx=None if ly.warm else ly.init_q, out=ly.cq, ws=ly.ws_km)
        if ev is not None:
            ev[1].record()
        svg.kmeans(k, F, HH, WW, wl.Ck, wl.iters, init_idx=None if ly.warm else ly.init_k, out=ly.ck, ws=ly.ws_km)
        if ev is not None:
            ev[2].record()
        svg.centroid_topp(ly.cq, ly.ck, F, HH, WW, wl.p, ly.scale, sel=ly.sel)
        if ev is not None:
            ev[3].record()
        svg.cluster_attn(q, k, v, ly.cq, ly.ck, ly.sel, F, HH, WW, ly.scale, o=ly.o, ws=ly.ws_attn)
        if ev is not None:
            ev[4].record()
        ly.warm = True

    for i in range(max(args.warmup, 2 * L)):      # cold start, then warm steps
        step(i % L)
    torch.cuda.synchronize()
    log(f"[bench] warmup done; timing {args.steps} steps")
    names = ["kmeans_q", "kmeans_k", "centroid_topp", "cluster_attn"]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i % L, evs[i])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    st = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(4)] for i in range(args.steps)])
    stage_ms = {n: float(st[:, j].mean()) for j, n in enumerate(names)}
    fl = [cluster_flops(ly.cq, ly.ck, ly.sel, g.D, 256, 64) for (_, _, _, ly) in layers]
    tok = np.array([fl[i % L][0] for i in range(args.steps)])
    tile = np.array([fl[i % L][1] for i in range(args.steps)])
    density = float(np.mean([f[2] for f in fl]))
    attn_tflops = float(np.mean(tile / (st[:, 3] * 1e-3)) / 1e12)
    tok_tflops = float(np.mean(tok / (st[:, 3] * 1e-3)) / 1e12)
    BH, S, D = g.B * g.H, g.S, g.D
    # k-means: the assignment products (2*D per row and padded centroid) and one read of the rows
    cpad = lambda C: -(-C // 64) * 64
    km_flops = {n: 2.0 * BH * S * cpad(C) * D * wl.iters for n, C in (("kmeans_q", wl.Cq), ("kmeans_k", wl.Ck))}
    # the same attention kernel run dense, for the speedup
    q, k, v, ly = layers[0]
    od = torch.empty_like(q)
    svg.dense_attn(q, k, v, F, HH, WW, o=od)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    svg.dense_attn(q, k, v, F, HH, WW, o=od)
    e1.record()
    torch.cuda.synchronize()
    dense_ms = e0.elapsed_time(e1)
    log(f"[bench] {ms_per_step:.3f} ms/step; stages {json.dumps({k_: round(v_, 4) for k_, v_ in stage_ms.items()})}")
    result = {
        "metric": "cluster-attn ms/layer + effective TFLOP/s (% bf16 MFMA peak), 720p shape, semantic clustering",
        "value": round(float(np.mean(tok)) / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{wl.name}: one layer (k-means of Q and K warm-started from the previous step's "
                               f"centroids, {wl.iters} iterations each; centroid top-p; attention over the selected "
                               f"clusters) over {L} layers of fresh inputs",
                   "B": g.B, "H": g.H, "F": g.F, "HH": g.HH, "WW": g.WW, "S": S, "D": D, "Cq": wl.Cq, "Ck": wl.Ck,
                   "p": wl.p, "iters": wl.iters, "n_classes": wl.n_classes, "layers": L,
                   "parallelism": "single GPU"},
        "density": round(density, 4),
        "token_tflop_per_layer": round(float(tok.mean()) / 1e12, 4),
        "tile_tflop_per_layer": round(float(tile.mean()) / 1e12, 4),
        "cluster_attn_ms": round(stage_ms["cluster_attn"], 4),
        "cluster_attn_tflops_tile": round(attn_tflops, 2),
        "cluster_attn_tflops_token": round(tok_tflops, 2),
        "kmeans_tflops": {n: round(km_flops[n] / (stage_ms[n] * 1e-3) / 1e12, 2) for n in km_flops},
        "dense_attn_ms": round(dense_ms, 3),
        "speedup_vs_dense_kernel": round(dense_ms / stage_ms["cluster_attn"], 3),
        "speedup_vs_dense_step": round(dense_ms / ms_per_step, 3),
        "stage_ms": {k_: round(v_, 4) for k_, v_ in stage_ms.items()},
        "roofline": {"bound": "mfma", "kernel": f"cluster_attn_kernel<{D}>", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(CLUSTER_TRAFFIC_FILE),
                     **measured_mfma("cluster_attn"),
                     "note": "computed-tile FLOPs over the svg_cluster_attn call (key lists + attention kernel)"},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cluster_cpu_baseline(q, k, v, ly.cq.labels, ly.ck.labels, ly.sel, D)
    print(json.dumps(result), flush=True)


def block_cpu_baseline(q, k, v, sel, D):
    """The fp64 oracle's attention over the chosen blocks for 4096 sampled query rows of one head
    (given the GPU's choice); token-level FLOPs / wall time."""
    import numpy as np
    import oracle.adaspa_oracle as A
    hc = host_cores()
    f64 = lambda t: t.detach().cpu().double().numpy()
    S = q.shape[2]
    rows = np.sort(np.random.default_rng(321).choice(S, 4096, replace=False))
    s = sel[0, 0].cpu().numpy().astype(bool)
    qh, kh, vh = f64(q[0, 0]), f64(k[0, 0]), f64(v[0, 0])
    t0 = time.perf_counter()
    A.block_sparse_attention_rows(qh, kh, vh, s, rows, 1.0 / math.sqrt(D))
    el = time.perf_counter() - t0
    pairs = float(A.block_token_mask(s, rows, S).sum())
    return {"value": 4.0 * D * pairs / el / 1e12, "unit": "TFLOP/s", **hc, "kind": "oracle",
            "sample": f"fp64 numpy oracle, attention over the chosen blocks of 4096 sampled query rows of one head "
                      f"(S={S}, D={D}) given the GPU's block choice; token-level FLOPs",
            "seconds": round(el, 2)}


def block_bench(args):
    """The head-adaptive block-sparse path at the 720p grid.  Per layer, a dense step (attention
    with each row's log-sum-exp, cached) precedes the timed sparse step on the next step's
    activations: block search with the cached LSE, block choice, attention over the chosen
    blocks.  Also timed: a sparse step that reuses the previous step's block choice."""
    import numpy as np
    import torch

    import spatial_temporal_sparse_amd as svg
    from workloads import WORKLOADS, make_qkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = WORKLOADS["hunyuan720p"]
    g = wl.geom
    F, HH, WW, D = g.F, g.HH, g.WW, g.D
    S, BH = g.S, g.B * g.H
    cov = 0.9
    L = max(1, min(args.layers, 2))
    nqb, nkb = svg.block_grid(S)
    log(f"[bench] block path: {L} layers of {g}, blocks {svg.BLOCK_Q}x{svg.BLOCK_K}, coverage {cov}")
    layers = []
    for l in range(L):
        q0, k0, v0 = make_qkv(wl, device="cuda", layer=l, step=0)
        _, lse = svg.dense_attn_lse(q0, k0, v0, F, HH, WW)        # the dense step: LSE cached
        del q0, k0, v0
        q, k, v = make_qkv(wl, device="cuda", layer=l, step=1)
        bufs = {"lse": lse, "mass": torch.empty((g.B, g.H, nqb, nkb), dtype=torch.float32, device=dev),
                "sel": torch.empty((g.B, g.H, nqb, nkb), dtype=torch.uint8, device=dev), "o": torch.empty_like(q),
                "ws": torch.empty(max(256, svg.workspace_bytes(svg.OP_BLOCK_ATTN, svg.geometry(q, F, HH, WW))),
                                  dtype=torch.uint8, device=dev)}
        layers.append((q, k, v, bufs))
    torch.cuda.synchronize()

    def step(l, ev=None, search=True):
        q, k, v, b = layers[l]
        if ev is not None:
            ev[0].record()
        if search:
            svg.block_mass(q, k, b["lse"], F, HH, WW, mass=b["mass"])
        if ev is not None:
            ev[1].record()
        if search:
            svg.block_select(b["mass"], F, HH, WW, D, cov, sel=b["sel"])
        if ev is not None:
            ev[2].record()
        svg.block_sparse_attn(q, k, v, b["sel"], F, HH, WW, o=b["o"], ws=b["ws"])
        if ev is not None:
            ev[3].record()

    def timed(search):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i % L, evs[i], search)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / args.steps
        st = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(3)] for i in range(args.steps)])
        return ms, st

    for i in range(max(args.warmup, L)):
        step(i % L)
    torch.cuda.synchronize()
    log(f"[bench] warmup done; timing {args.steps} steps with the search, then {args.steps} reusing the choice")
    ms_search, st = timed(True)
    ms_reuse, st_reuse = timed(False)
    names = ["block_mass", "block_select", "block_sparse_attn"]
    stage_ms = {n: float(st[:, j].mean()) for j, n in enumerate(names)}
    # work of the chosen blocks: each query block runs its rows against its chosen keys
    fl_tok, fl_tile, dens = [], [], []
    for (q, k, v, b) in layers:
        sel = b["sel"].double()
        kb = torch.full((nkb,), float(svg.BLOCK_K), dtype=torch.float64, device=dev)
        kb[-1] = S - svg.BLOCK_K * (nkb - 1)
        qrows = torch.full((nqb,), float(svg.BLOCK_Q), dtype=torch.float64, device=dev)
        qrows[-1] = S - svg.BLOCK_Q * (nqb - 1)
        keys = torch.einsum("bhij,j->bhi", sel, kb)                      # keys per query block
        fl_tok.append(4.0 * D * float(torch.einsum("bhi,i->", keys, qrows)))
        fl_tile.append(4.0 * D * float((torch.ceil(keys / 64) * 64).sum()) * svg.BLOCK_Q)
        dens.append(float(torch.einsum("bhi,i->bh", keys, qrows).mean()) / S ** 2)
    tok = np.array([fl_tok[i % L] for i in range(args.steps)])
    tile = np.array([fl_tile[i % L] for i in range(args.steps)])
    attn_tflops = float(np.mean(tile / (st[:, 2] * 1e-3)) / 1e12)
    q, k, v, b = layers[0]
    od = torch.empty_like(q)
    svg.dense_attn(q, k, v, F, HH, WW, o=od)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    svg.dense_attn(q, k, v, F, HH, WW, o=od)
    e1.record()
    torch.cuda.synchronize()
    dense_ms = e0.elapsed_time(e1)
    e0.record()
    svg.dense_attn_lse(q, k, v, F, HH, WW, o=od, lse=torch.empty_like(b["lse"]))
    e1.record()
    torch.cuda.synchronize()
    dense_lse_ms = e0.elapsed_time(e1)
    mass_flops = 2.0 * D * S * S * BH
    log(f"[bench] {ms_search:.3f} ms/step with search, {ms_reuse:.3f} reusing; stages "
        f"{json.dumps({k_: round(v_, 4) for k_, v_ in stage_ms.items()})}")
    result = {
        "metric": "block-sparse attn ms/layer + effective TFLOP/s (% bf16 MFMA peak), 720p shape, LSE-cached block "
                  "search",
        "value": round(float(np.mean(tok)) / (ms_search * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_search, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"hunyuan720p (planted spatial/temporal heads): per layer, the block search of step 1 "
                               f"with the LSE cached by a dense step 0, block choice at coverage {cov}, attention "
                               f"over the chosen blocks, over {L} layers",
                   "B": g.B, "H": g.H, "F": F, "HH": HH, "WW": WW, "S": S, "D": D, "block": [svg.BLOCK_Q, svg.BLOCK_K],
                   "coverage": cov, "layers": L, "parallelism": "single GPU"},
        "density": round(float(np.mean(dens)), 4),
        "token_tflop_per_layer": round(float(tok.mean()) / 1e12, 4),
        "tile_tflop_per_layer": round(float(tile.mean()) / 1e12, 4),
        "block_sparse_attn_ms": round(stage_ms["block_sparse_attn"], 4),
        "block_sparse_attn_tflops_tile": round(attn_tflops, 2),
        "block_mass_ms": round(stage_ms["block_mass"], 4),
        "block_mass_tflops": round(mass_flops / (stage_ms["block_mass"] * 1e-3) / 1e12, 2),
        "block_select_ms": round(stage_ms["block_select"], 4),
        "ms_per_step_reusing_choice": round(ms_reuse, 4),
        "dense_attn_ms": round(dense_ms, 3),
        "dense_attn_lse_ms": round(dense_lse_ms, 3),
        "speedup_vs_dense_step": round(dense_ms / ms_search, 3),
        "speedup_vs_dense_step_reusing_choice": round(dense_ms / ms_reuse, 3),
        "stage_ms": {k_: round(v_, 4) for k_, v_ in stage_ms.items()},
        "roofline": {"bound": "mfma", "kernel": f"block_attn_kernel<{D}>", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(BLOCK_TRAFFIC_FILE),
                     **measured_mfma("block_attn"),
                     "note": "computed-tile FLOPs over the svg_block_sparse_attn call (block lists + attention kernel)"},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = block_cpu_baseline(q, k, v, b["sel"], D)
    print(json.dumps(result), flush=True)


def isolated_hbm(svg, layer, bufs, norm, g, wl, reps=20):
    """The HBM-bound kernels one at a time on one layer's inputs, each launch preceded by a
    512 MiB read that evicts the 256 MB Infinity Cache (MALL), so that no launch finds its
    inputs cached by the one before: median and min over `reps` launches, and the algorithmic
    bytes per launch.  The eviction reads rather than writes, so that the timed launch does
    not also pay for writing back the eviction's own dirty lines."""
    import numpy as np
    import torch
    q, k, v, idx = layer
    F, HH, WW, w_f, w_p = g.F, g.HH, g.WW, wl.w_f, wl.w_p
    svg.qknorm_rope(q, k, norm[0], norm[1], F, HH, WW, wl.eps, wl.rope_base, q_out=bufs.qn, k_out=bufs.kn)
    svg.profile_heads(bufs.qn, bufs.kn, v, idx, F, HH, WW, w_f, w_p, mse=bufs.mse, kind=bufs.kind, ws=bufs.ws_profile)
    n_tmp = int((bufs.kind == 1).sum().item())
    row = g.S * g.D * 2
    BH = g.B * g.H

    def permute_qkv():
        for src, dst in ((bufs.qn, bufs.qt), (bufs.kn, bufs.kt), (v, bufs.vt)):
            svg.permute(src, F, HH, WW, bufs.kind, svg.TEMPORAL, out=dst)

    ops = {
        "qknorm_rope": (lambda: svg.qknorm_rope(q, k, norm[0], norm[1], F, HH, WW, wl.eps, wl.rope_base,
                                                q_out=bufs.qn, k_out=bufs.kn), 4 * BH * row),
        "profile_heads": (lambda: svg.profile_heads(bufs.qn, bufs.kn, v, idx, F, HH, WW, w_f, w_p, mse=bufs.mse,
                                                    kind=bufs.kind, ws=bufs.ws_profile), 2 * BH * row),
        "permute_qkv": (permute_qkv, 6 * n_tmp * row),
        "unpermute": (lambda: svg.unpermute(bufs.ot, F, HH, WW, bufs.kind, svg.TEMPORAL, out=bufs.o), 2 * n_tmp * row),
    }
    flush = torch.ones(128 << 20, dtype=torch.int32, device=q.device)   # 512 MiB
    out = {}
    for name, (fn, nbytes) in ops.items():
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            flush.sum()
            ev[i][0].record()
            fn()
            ev[i][1].record()
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in ev])
        med = float(np.median(ms))
        out[name] = {"ms_median": round(med, 4), "ms_min": round(float(ms.min()), 4), "bytes": int(nbytes),
                     "gbs_median": round(nbytes / (med * 1e-3) / 1e9, 1),
                     "frac_of_peak_median": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)}
    del flush
    return out


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.denoise > 0:
        if args.gpus != 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        denoise(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards over heads with no "
              f"exchange, so per-GPU throughput is the one-GPU figure.", file=sys.stderr)
        sys.exit(2)
    if args.workload == "hunyuan720p_svg2":
        cluster_bench(args)
        return
    if args.workload == "hunyuan720p_blocks":
        block_bench(args)
        return
    import numpy as np
    import torch

    import spatial_temporal_sparse_amd as svg
    from workloads import WORKLOADS, make_qkv, norm_weights, sample_queries

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = WORKLOADS[args.workload]
    headline = args.workload == "hunyuan720p_step"
    g = wl.geom
    L = max(1, args.layers)
    log(f"[bench] generating {L} layers of {g} on {torch.cuda.get_device_name(dev)}")
    layers = []
    for l in range(L):
        q, k, v = make_qkv(wl, device="cuda", layer=l)
        idx = torch.from_numpy(sample_queries(g.S, wl.n_q, wl.idx_seed + l)).to(dev)
        layers.append((q, k, v, idx))
    wq, wk = norm_weights(g.D, wl.seed)
    norm = (torch.from_numpy(wq).to(dev), torch.from_numpy(wk).to(dev), wl.eps, wl.rope_base)
    bufs = svg.LayerBuffers(layers[0][0], wl.n_q, g.F, g.HH, g.WW)
    bm, bn = svg.tile_shape()
    F, HH, WW, w_f, w_p = g.F, g.HH, g.WW, wl.w_f, wl.w_p

    def step(l, ev=None, layout=args.layout):
        q, k, v, idx = layers[l]
        if ev is not None:
            ev[0].record()
        qn, kn = svg.qknorm_rope(q, k, norm[0], norm[1], F, HH, WW, wl.eps, wl.rope_base, q_out=bufs.qn, k_out=bufs.kn)
        if ev is not None:
            ev[1].record()
        svg.profile_heads(qn, kn, v, idx, F, HH, WW, w_f, w_p, mse=bufs.mse, kind=bufs.kind, ws=bufs.ws_profile)
        if ev is not None:
            ev[2].record()
        if layout == "explicit":
            svg.permute(qn, F, HH, WW, bufs.kind, svg.TEMPORAL, out=bufs.qt)
            svg.permute(kn, F, HH, WW, bufs.kind, svg.TEMPORAL, out=bufs.kt)
            svg.permute(v, F, HH, WW, bufs.kind, svg.TEMPORAL, out=bufs.vt)
        if ev is not None:
            ev[3].record()
        if layout == "explicit":
            svg.sparse_attn(qn, kn, v, bufs.qt, bufs.kt, bufs.vt, bufs.kind, F, HH, WW, w_f, w_p, o=bufs.o,
                            ot=bufs.ot, ws=bufs.ws_attn)
        else:
            svg.sparse_attn(qn, kn, v, None, None, None, bufs.kind, F, HH, WW, w_f, w_p, o=bufs.o, ws=bufs.ws_attn)
        if ev is not None:
            ev[4].record()
        if layout == "explicit":
            svg.unpermute(bufs.ot, F, HH, WW, bufs.kind, svg.TEMPORAL, out=bufs.o)
        if ev is not None:
            ev[5].record()

    # one untimed pass per layer: the kinds each layer chooses fix its tile work
    kinds, flops_tile, flops_tok = [], [], []
    for l in range(L):
        step(l)
        kd = bufs.kind.clone()
        kinds.append(kd.cpu().numpy()[0])
        flops_tile.append(tile_flops(svg, kd, g, w_f, w_p, bm, bn))
        flops_tok.append(token_flops(kd.cpu().numpy(), g, w_f, w_p))
    torch.cuda.synchronize()
    log(f"[bench] kinds per layer: {[k.tolist() for k in kinds]}")

    for i in range(args.warmup):
        step(i % L)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps")

    names = ["qknorm_rope", "profile_heads", "permute_qkv", "sparse_attn", "unpermute"]

    def timed(layout):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i % L, evs[i], layout)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        st = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(5)] for i in range(args.steps)])
        return (t1 - t0) * 1e3 / args.steps, st

    ms_per_step, stage = timed(args.layout)
    stage_ms = {n: float(stage[:, j].mean()) for j, n in enumerate(names)}
    stage_med = {n: round(float(np.median(stage[:, j])), 4) for j, n in enumerate(names)}
    stage_min = {n: round(float(stage[:, j].min()), 4) for j, n in enumerate(names)}
    other = "explicit" if args.layout == "fused" else "fused"
    compare = None
    if not args.no_compare:
        for i in range(args.warmup):
            step(i % L, None, other)
        o_ms, o_stage = timed(other)
        compare = {"layout": other, "ms_per_step": round(o_ms, 4),
                   "stage_ms": {n: round(float(o_stage[:, j].mean()), 4) for j, n in enumerate(names)}}
        log(f"[bench] {other} layout: {o_ms:.3f} ms/step")
    ex_stage = stage if args.layout == "explicit" else (o_stage if compare else None)
    step_tile = np.array([flops_tile[i % L] for i in range(args.steps)])
    step_tok = np.array([flops_tok[i % L] for i in range(args.steps)])
    attn_ms = stage[:, 3]
    attn_tflops = float(np.mean(step_tile / (attn_ms * 1e-3)) / 1e12)
    log(f"[bench] {ms_per_step:.3f} ms/step; stages {json.dumps({k: round(v, 4) for k, v in stage_ms.items()})}")

    # HBM-bound stages: algorithmic bytes over time
    BH, S, D = g.B * g.H, g.S, g.D
    n_tmp = np.array([int((kinds[i % L] == 1).sum()) for i in range(args.steps)])
    row = S * D * 2
    hbm = {
        "qknorm_rope": float(np.mean(4 * BH * row / (stage[:, 0] * 1e-3)) / 1e9),
        "profile_heads": float(np.mean(2 * BH * row / (stage[:, 1] * 1e-3)) / 1e9),
    }
    if ex_stage is not None:   # the separate layout passes, from the explicit-layout steps
        hbm["permute_qkv"] = float(np.mean(6 * n_tmp * row / (ex_stage[:, 2] * 1e-3)) / 1e9)
        hbm["unpermute"] = float(np.mean(2 * n_tmp * row / (ex_stage[:, 4] * 1e-3)) / 1e9)

    # the same kernel run dense, on layer 0
    q, k, v, _ = layers[0]
    svg.dense_attn(q, k, v, F, HH, WW, o=bufs.o)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    svg.dense_attn(q, k, v, F, HH, WW, o=bufs.o)
    e1.record()
    torch.cuda.synchronize()
    dense_ms = e0.elapsed_time(e1)
    dense_flops = 4.0 * S * S * D * BH

    traffic = measured_traffic() if headline else None    # the counters were taken on the 720p layer
    tile_per_launch = float(step_tile.mean())
    result = {
        "metric": "sparse-attn ms/layer + effective TFLOP/s (% bf16 MFMA peak), "
                  + ("720p shape" if headline else f"{wl.name} shape"),
        "value": round(float(np.mean(step_tile)) / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: one layer (qknorm+rope, profile {wl.n_q} queries, layout "
                               f"transformation of temporal heads, block-sparse attention) over {L} layers of "
                               "fresh inputs",
                   "layout": args.layout,
                   "B": g.B, "H": g.H, "F": g.F, "HH": g.HH, "WW": g.WW, "S": S, "D": D, "w_f": w_f, "w_p": w_p,
                   "n_q": wl.n_q, "layers": L, "tile": [bm, bn], "parallelism": "single GPU"},
        "sparse_attn_ms": round(float(attn_ms.mean()), 4),
        "sparse_attn_ms_median": round(float(np.median(attn_ms)), 4),
        "sparse_attn_ms_min": round(float(attn_ms.min()), 4),
        "sparse_attn_tflops": round(attn_tflops, 2),
        "sparse_attn_frac_of_bf16_peak": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
        "tile_tflop_per_layer": round(tile_per_launch / 1e12, 4),
        "token_tflop_per_layer": round(float(step_tok.mean()) / 1e12, 4),
        "dense_attn_ms": round(dense_ms, 3),
        "dense_attn_tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 2),
        "speedup_vs_dense_kernel": round(dense_ms / float(attn_ms.mean()), 3),
        "speedup_vs_dense_step": round((stage_ms["qknorm_rope"] + dense_ms) / ms_per_step, 3),
        "profile_over_attn": round(stage_ms["profile_heads"] / stage_ms["sparse_attn"], 4),
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "stage_ms_median": stage_med,
        "stage_ms_min": stage_min,
        "compare": compare,
        "hbm_gbs": {k: round(v, 1) for k, v in hbm.items()},
        "hbm_frac_of_peak": {k: round(v / PEAK_HBM_GBS, 3) for k, v in hbm.items()},
        "roofline": {"bound": "mfma", "kernel": f"attn_fwd_kernel<{D}>", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     **(measured_mfma("attn_fwd sparse") if headline else {})},
    }
    hbm_traffic = measured_hbm_traffic() if headline else {}
    if hbm_traffic:
        result["hbm_traffic"] = hbm_traffic
    if not args.no_isolated:
        log("[bench] HBM-bound kernels one at a time, the MALL flushed before every launch")
        result["hbm_isolated"] = isolated_hbm(svg, layers[0], bufs, norm, g, wl)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        # the last timed layer's normalised Q/K (recomputed: the isolated leg overwrote them)
        last = (args.steps - 1) % L
        q, k, v, _ = layers[last]
        svg.qknorm_rope(q, k, norm[0], norm[1], F, HH, WW, wl.eps, wl.rope_base, q_out=bufs.qn, k_out=bufs.kn)
        result["cpu_baseline"] = cpu_baseline(bufs.qn, bufs.kn, v, kinds[last], g, w_f, w_p)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
