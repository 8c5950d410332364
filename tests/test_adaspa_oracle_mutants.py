"""Plant plausible mistakes in the AdaSpa-style oracle (on the CPU) and check that the pins of
test_adaspa_oracle_pins.py catch each one."""
import numpy as np
import pytest

import oracle.adaspa_oracle as A
from tests import test_adaspa_oracle_pins as pins

ORIG = {n: getattr(A, n) for n in ("row_lse", "block_mass", "select_blocks", "block_token_mask")}


def _mut_lse_no_scale(q, k, scale):
    return ORIG["row_lse"](q, k, 1.0)


def _mut_lse_max_only(q, k, scale):
    return (scale * (np.asarray(q) @ np.asarray(k).T)).max(axis=1)               # forgets the sum


def _mut_lse_log2(q, k, scale):
    return ORIG["row_lse"](q, k, scale) / np.log(2.0)                             # base-2 normaliser


def _mut_mass_no_lse(q, k, lse, scale, bq=A.BQ, bk=A.BK, q_blocks=None):
    return ORIG["block_mass"](q, k, np.zeros(len(q)), scale, bq, bk, q_blocks)     # unnormalised


def _mut_mass_swapped_blocks(q, k, lse, scale, bq=A.BQ, bk=A.BK, q_blocks=None):
    return ORIG["block_mass"](q, k, lse, scale, bk, bq, None)                      # block sizes swapped


def _mut_mass_mean(q, k, lse, scale, bq=A.BQ, bk=A.BK, q_blocks=None):
    M = ORIG["block_mass"](q, k, lse, scale, bq, bk, q_blocks)
    return M / bk                                                                  # a mean, not a sum


def _mut_select_vs_max(M, coverage):
    M = np.asarray(M, dtype=np.float64)
    sel = np.zeros(M.shape, dtype=bool)
    for i in range(M.shape[0]):
        sel[i] = M[i] >= (1.0 - coverage) * M[i].max()                            # threshold, not coverage
        sel[i] &= M[i] > 0
    return sel


def _mut_select_ascending(M, coverage):
    M = np.asarray(M, dtype=np.float64)
    return ORIG["select_blocks"](np.where(M > 0, M.max() + 1.0 - M, 0.0), coverage)


def _mut_select_strict(M, coverage):
    M = np.asarray(M, dtype=np.float64)
    sel = np.zeros(M.shape, dtype=bool)
    for i in range(M.shape[0]):
        target, acc = coverage * M[i].sum(), 0.0
        for j in sorted(range(M.shape[1]), key=lambda j: (-M[i, j], j)):
            if M[i, j] <= 0.0:
                break
            sel[i, j] = True
            acc += M[i, j]
            if acc > target:                                                       # one block too many
                break
    return sel


def _mut_mask_wrong_block(sel, rows, S, bq=A.BQ, bk=A.BK):
    return ORIG["block_token_mask"](sel, rows, S, bq, bq)                          # key blocks of the query size


MUTANTS = [
    ("row_lse", _mut_lse_no_scale), ("row_lse", _mut_lse_max_only), ("row_lse", _mut_lse_log2),
    ("block_mass", _mut_mass_no_lse), ("block_mass", _mut_mass_swapped_blocks), ("block_mass", _mut_mass_mean),
    ("select_blocks", _mut_select_vs_max), ("select_blocks", _mut_select_ascending),
    ("select_blocks", _mut_select_strict), ("block_token_mask", _mut_mask_wrong_block),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[f"{n}:{m.__name__}" for n, m in MUTANTS])
def test_pins_catch_mutant(monkeypatch, name, mutant):
    monkeypatch.setattr(A, name, mutant)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as exc:
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught mutant {mutant.__name__} of {name}"
