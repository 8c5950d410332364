"""GPU parity, bit-exact: the layout transformation and the tile mask against the oracle."""
import numpy as np
import pytest
import torch

import oracle.svg_oracle as O
from tests.gpu_util import note

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

GEOMS = [  # B, H, F, HH, WW, D
    (1, 2, 4, 8, 8, 64),
    (2, 3, 3, 5, 7, 128),      # ragged: S = 105
    (1, 4, 13, 30, 45, 64),    # CogVideoX-like grid
    (1, 2, 33, 45, 80, 128),   # 720p grid, two heads
    (1, 3, 1, 6, 6, 64),       # a single frame
    (1, 3, 9, 1, 1, 128),      # one location per frame
]


def _kinds(B, H, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 3, size=(B, H)).astype(np.uint8)


@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: "x".join(map(str, g)))
def test_permute_index_rows_bit_exact(gpu, geom):
    B, H, F, HH, WW, D = geom
    P, S = HH * WW, F * HH * WW
    note(f"permute index rows {geom}")
    # every row holds its own (head, token) number, exact in fp32
    ids = torch.arange(B * H * S, dtype=torch.float32).view(B, H, S, 1).expand(B, H, S, D).contiguous()
    x = ids.to(DEV)
    y = gpu.permute(x, F, HH, WW)
    want = O.permute(ids.numpy(), F, P)
    assert np.array_equal(y.cpu().numpy(), want)
    assert torch.equal(gpu.unpermute(y, F, HH, WW), x)
    # selection by kind: only heads of the selected kind are written
    kinds = _kinds(B, H, 3)
    for sel in (O.SPATIAL, O.TEMPORAL, O.DENSE):
        out = torch.full_like(x, -1.0)
        gpu.permute(x, F, HH, WW, torch.from_numpy(kinds).to(DEV), sel, out=out)
        got = out.cpu().numpy()
        for b in range(B):
            for h in range(H):
                if kinds[b, h] == sel:
                    assert np.array_equal(got[b, h], want[b, h])
                else:
                    assert (got[b, h] == -1.0).all()
        back = torch.full_like(x, -2.0)
        gpu.unpermute(out, F, HH, WW, torch.from_numpy(kinds).to(DEV), sel, out=back)
        bk = back.cpu().numpy()
        for b in range(B):
            for h in range(H):
                if kinds[b, h] == sel:
                    assert np.array_equal(bk[b, h], ids.numpy()[b, h])
                else:
                    assert (bk[b, h] == -2.0).all()


@pytest.mark.parametrize("geom", GEOMS[:3], ids=lambda g: "x".join(map(str, g)))
def test_permute_bf16_round_trip(gpu, geom):
    B, H, F, HH, WW, D = geom
    note(f"permute bf16 {geom}")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    x = torch.randn((B, H, F * HH * WW, D), generator=gen, device=DEV).to(torch.bfloat16)
    y = gpu.permute(x, F, HH, WW)
    pi = torch.from_numpy(O.perm_indices(F, HH * WW)).to(DEV)
    assert torch.equal(y, x[:, :, pi, :])
    assert torch.equal(gpu.unpermute(y, F, HH, WW), x)


MASK_CASES = [  # geometry, windows, tiles
    ((1, 3, 4, 8, 8), (1, 2), [(128, 64), (64, 64), (7, 5), (100, 30), (256, 256)]),
    ((2, 3, 3, 5, 7), (1, 3), [(128, 64), (5, 7), (1, 1), (105, 105)]),
    ((1, 3, 6, 9, 11), (2, 5), [(128, 64), (33, 17)]),
    ((1, 3, 13, 30, 45), (1, 8), [(128, 128), (128, 64)]),
]


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: "x".join(map(str, c[0])))
def test_block_mask_bit_exact(gpu, case):
    (B, H, F, HH, WW), (w_f, w_p), tiles = case
    P, S = HH * WW, F * HH * WW
    kinds = np.array([[(h + b) % 3 for h in range(H)] for b in range(B)], dtype=np.uint8)   # S, T, D mixed
    kd = torch.from_numpy(kinds).to(DEV)
    for bm, bn in tiles:
        note(f"block mask {case[0]} w=({w_f},{w_p}) tile {bm}x{bn}")
        got = gpu.build_block_mask(kd, F, HH, WW, w_f, w_p, bm, bn).cpu().numpy()
        for b in range(B):
            for h in range(H):
                want = O.block_mask(int(kinds[b, h]), F, P, w_f, w_p, bm, bn)
                assert np.array_equal(got[b, h], want), (b, h, bm, bn)
