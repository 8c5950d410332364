"""GPU parity of online profiling (per-head MSE and choice) and of QK-RMSNorm + 3D RoPE."""
import numpy as np
import pytest
import torch

import oracle.svg_oracle as O
from tests.gpu_util import bf16_ulp, host64, note
from workloads import WORKLOADS, Geometry, Workload, expected_planted_kinds, make_qkv, norm_weights, sample_queries

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# Error budget of a profiled MSE.  The kernel forms each sampled output from bf16 inputs with
# fp32 accumulation and bf16-rounded softmax weights, so every output element carries an
# absolute error e of at most a few 1e-3 (bf16 has 8 significant bits; weights <= 1).  An MSE
# of (O_x - O_dense)^2 then moves by at most 2*sqrt(mse)*(2e) + (2e)^2.
E_OUT = 4e-3


def _mse_tol(mse):
    return 2.0 * np.sqrt(mse) * (2 * E_OUT) + (2 * E_OUT) ** 2


def _check_profile(gpu, q, k, v, idx, g, w_f, w_p, expect=None, what=""):
    mse_g, kind_g = gpu.profile_heads(q, k, v, torch.from_numpy(idx).to(DEV), g.F, g.HH, g.WW, w_f, w_p)
    torch.cuda.synchronize()
    mse_g, kind_g = mse_g.cpu().numpy(), kind_g.cpu().numpy()
    # the choice is the argmin of the stored fp32 errors, ties to spatial
    assert np.array_equal(kind_g, np.where(mse_g[..., 0] <= mse_g[..., 1], O.SPATIAL, O.TEMPORAL))
    mse_o = np.zeros((g.B, g.H, 2))
    kind_o = np.zeros((g.B, g.H), dtype=np.uint8)
    sc = O.default_scale(g.D)
    for b in range(g.B):
        for h in range(g.H):
            a, c, kd = O.profile_head(host64(q[b, h]), host64(k[b, h]), host64(v[b, h]), idx, g.F, g.P, w_f, w_p, sc)
            mse_o[b, h] = (a, c)
            kind_o[b, h] = kd
    assert (np.abs(mse_g - mse_o) <= _mse_tol(mse_o)).all(), f"{what}: mse {mse_g} vs {mse_o}"
    assert O.choices_agree(kind_g, kind_o, mse_o, 1e-6).all(), f"{what}: kinds {kind_g} vs {kind_o} ({mse_o})"
    if expect is not None:
        assert np.array_equal(kind_g[0], expect), f"{what}: planted {expect}, got {kind_g[0]}"
    return mse_g, kind_g


def test_profile_tiny(gpu):
    wl = WORKLOADS["tiny"]
    g = wl.geom
    note("profile tiny")
    q, k, v = make_qkv(wl, device="cpu")
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    idx = sample_queries(g.S, wl.n_q, wl.idx_seed)
    _check_profile(gpu, q, k, v, idx, g, wl.w_f, wl.w_p, what="tiny")


@pytest.mark.parametrize("n_q", [1, 17, 64, 100])
def test_profile_query_counts(gpu, n_q):
    g = Geometry(1, 4, 6, 7, 9, 64)
    wl = Workload("nq", g, 1, 3, n_q, 31, 131, planted=True)
    note(f"profile n_q={n_q}")
    q, k, v = make_qkv(wl, device=DEV)
    idx = sample_queries(g.S, n_q, wl.idx_seed)
    _check_profile(gpu, q, k, v, idx, g, 1, 3, what=f"n_q={n_q}")


def test_profile_planted_cogvideox_shape(gpu):
    wl = WORKLOADS["cogvideox"]
    g = wl.geom
    note("profile CogVideoX-like, 48 heads, S=17550")
    q, k, v = make_qkv(wl, device=DEV)
    idx = sample_queries(g.S, wl.n_q, wl.idx_seed)
    _check_profile(gpu, q, k, v, idx, g, wl.w_f, wl.w_p, expect=expected_planted_kinds(wl), what="cogvideox")


# In-frame positions per key (frames of < 64 tokens, or a band leaving < 52 positions of a frame
# out) instead of one band interval per tile.  64 heads, so that each key split holds several
# tiles of 64 keys (the two tile buffers alternate); the last split is ragged.
PER_KEY_CASES = [  # name, F, HH, WW, D, w_p
    ("P24_D64", 60, 4, 6, 64, 5),
    ("P24_D128", 60, 4, 6, 128, 5),
    ("P80_wide_band", 60, 8, 10, 128, 20),
    ("P1_one_location", 200, 1, 1, 128, 3),
]


@pytest.mark.parametrize("case", PER_KEY_CASES, ids=[c[0] for c in PER_KEY_CASES])
def test_profile_per_key_positions(gpu, case):
    _, F, HH, WW, D, w_p = case
    g = Geometry(1, 64, F, HH, WW, D)
    note(f"profile per-key positions {case[0]}")
    q, k, v = make_qkv(Workload("perkey", g, 1, w_p, 64, 33, 133, planted=True), device=DEV)
    idx = sample_queries(g.S, 64, 133)
    _check_profile(gpu, q, k, v, idx, g, 1, w_p, what=case[0])


def test_profile_full_cover_choice(gpu):
    g = Geometry(1, 2, 4, 6, 6, 128)
    note("profile with a spatial window covering every frame")
    q, k, v = make_qkv(Workload("cov", g, 3, 1, 32, 32, 132, planted=False), device=DEV)
    idx = sample_queries(g.S, 32, 132)
    mse, kind = _check_profile(gpu, q, k, v, idx, g, g.F - 1, 1, what="cover")
    assert (mse[..., 0] < 1e-10).all() and (kind == O.SPATIAL).all()


NORM_CASES = [
    ("tiny64", Geometry(1, 2, 4, 8, 8, 64), None),
    ("odd_dims64", Geometry(2, 2, 3, 5, 7, 64), (16, 24, 24)),
    ("wan", WORKLOADS["wan"].geom, None),
    ("t_only128", Geometry(1, 2, 5, 3, 4, 128), (128, 0, 0)),
]


@pytest.mark.parametrize("case", NORM_CASES, ids=[c[0] for c in NORM_CASES])
def test_qknorm_rope_vs_oracle(gpu, case):
    name, g, dims = case
    note(f"qknorm+rope {name} {g}")
    wl = Workload(name, g, 1, 1, 64, 41, 141, planted=True)
    q, k, _ = make_qkv(wl, device=DEV)
    wq, wk = norm_weights(g.D, 41)
    tq, tk = torch.from_numpy(wq).to(DEV), torch.from_numpy(wk).to(DEV)
    qo, ko = gpu.qknorm_rope(q, k, tq, tk, g.F, g.HH, g.WW, 1e-6, 10000.0, dims)
    torch.cuda.synchronize()
    for src, w, out in ((q, wq, qo), (k, wk, ko)):
        for b in range(g.B):
            for h in range(g.H):
                want = O.rope_3d(O.rms_norm(host64(src[b, h]), w.astype(np.float64), 1e-6), g.F, g.HH, g.WW,
                                 10000.0, dims)
                got = host64(out[b, h])
                err = np.abs(got - want)
                # one bf16 step of the exact value, plus the fp32 evaluation error of the
                # rotation, which scales with the length of the rotated pair
                pair = np.repeat(np.hypot(want[:, 0::2], want[:, 1::2]), 2, axis=1)
                tol = bf16_ulp(want) + 1e-6 + 2.0 ** -20 * pair
                assert (err <= tol).all(), f"{name}: max err {err.max()}, worst excess {(err - tol).max()}"
    # in place gives the same bits
    q2, k2 = q.clone(), k.clone()
    gpu.qknorm_rope(q2, k2, tq, tk, g.F, g.HH, g.WW, 1e-6, 10000.0, dims, q_out=q2, k_out=k2)
    assert torch.equal(q2, qo) and torch.equal(k2, ko)


# Sharp rows: a sampled query meets one planted key of huge score outside both of its masks,
# so that its masked scores lie far more than 126 (log2 units) below its unmasked maximum.
# The shared-reference fast path loses such a state's exponentials to underflow; the kernel
# must then merge by each state's own mass and recompute the marked states exactly.
SHARP_CASES = [  # name, F, HH, WW, D, w_p
    ("P64_interval_D128", 8, 8, 8, 128, 3),
    ("P48_per_key_D64", 10, 6, 8, 64, 3),
]


@pytest.mark.parametrize("case", SHARP_CASES, ids=[c[0] for c in SHARP_CASES])
def test_profile_sharp_rows(gpu, case):
    name, F, HH, WW, D, w_p = case
    g = Geometry(1, 2, F, HH, WW, D)
    note(f"profile sharp rows {name}")
    q, k, v = make_qkv(Workload("sharp", g, 1, w_p, 64, 41, 141, planted=False), device="cpu")
    idx = sample_queries(g.S, 64, 141)
    P = g.P
    c = O.default_scale(D) * np.log2(np.e)
    qf, kf = q.float(), k.float()
    planted = []
    for h in range(g.H):
        for j in (0, 7, 30):
            tq = int(idx[j])
            fq, pq = divmod(tq, P)
            # a key outside both masks: at least two frames away and w_p + 2 positions away
            ff = (fq + F // 2) % F
            pf = (pq + P // 2) % P
            assert abs(ff - fq) > 1 and abs(pf - pq) > w_p
            t_far = ff * P + pf
            qv = qf[0, h, tq]
            kf[0, h, t_far] = qv * (170.0 / (c * float(qv.norm()) ** 2))   # score of about 170 log2 units
            planted.append((h, tq))
    k = kf.to(torch.bfloat16)
    # the planted rows are in the regime: every masked score far below the unmasked maximum
    q64, k64 = q.double().numpy(), k.double().numpy()
    for h, tq in planted:
        sc = (q64[0, h, tq] @ k64[0, h].T) * c
        t = np.arange(g.S)
        sp = np.abs(t // P - tq // P) <= 1
        tp = np.abs(t % P - tq % P) <= w_p
        assert sc.max() - sc[sp].max() > 140 and sc.max() - sc[tp].max() > 140
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    _check_profile(gpu, q, k, v, idx, g, 1, w_p, what=name)
