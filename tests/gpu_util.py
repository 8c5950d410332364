"""Helpers shared by the GPU parity tests (comparison and host copies only)."""
import sys

import numpy as np
import torch

# Contract for bf16 attention outputs against the fp64 oracle.
MAX_ABS = 2e-2
REL_L2 = 5e-3


def note(msg: str) -> None:
    """Name the case on stdout before GPU work, so a failing run says where it was."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def assert_close_attn(got: np.ndarray, want: np.ndarray, what: str) -> None:
    err = np.abs(got - want)
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert err.max() <= MAX_ABS and rel <= REL_L2, f"{what}: max-abs {err.max():.3e}, rel-L2 {rel:.3e}"


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)
