"""Pins of the AdaSpa-style block-sparse oracle (oracle/adaspa_oracle.py) to things other than
itself: scipy's logsumexp, brute force on tiny inputs, closed forms and invariants.  Each
`pin_*` raises AssertionError on disagreement; test_adaspa_oracle_mutants.py plants mistakes in
the oracle and checks that a pin catches each.
"""
import itertools
import math

import numpy as np
import pytest

import oracle.adaspa_oracle as A
import oracle.svg_oracle as O


def _rng(seed):
    return np.random.default_rng(seed)


def pin_lse_matches_scipy():
    from scipy.special import logsumexp
    r = _rng(1)
    q, k = r.standard_normal((37, 8)) * 2.0, r.standard_normal((53, 8))
    got = A.row_lse(q, k, 0.7)
    want = logsumexp(0.7 * (q @ k.T), axis=1)
    assert np.abs(got - want).max() < 1e-12


def pin_lse_closed_forms():
    # one key: LSE = scale * q.k;  n equal logits: log n + logit
    q = np.array([[1.0, 2.0]])
    assert abs(A.row_lse(q, np.array([[3.0, -1.0]]), 0.5)[0] - 0.5) < 1e-15
    k = np.tile([[0.5, 0.25]], (7, 1))
    assert abs(A.row_lse(q, k, 2.0)[0] - (math.log(7) + 2.0)) < 1e-14


def _brute_mass(q, k, lse, scale, bq, bk):
    S, T = len(q), len(k)
    nqb, nkb = -(-S // bq), -(-T // bk)
    M = [[0.0] * nkb for _ in range(nqb)]
    for a in range(S):
        for b in range(T):
            dot = sum(x * y for x, y in zip(q[a], k[b]))
            M[a // bq][b // bk] += math.exp(scale * dot - lse[a])
    return np.array(M)


def pin_block_mass_brute_force():
    r = _rng(2)
    for S, bq, bk in [(10, 4, 3), (17, 5, 4), (8, 8, 8)]:
        q, k = r.standard_normal((2, S, 3))
        lse = A.row_lse(q, k, 0.9)
        got = A.block_mass(q, k, lse, 0.9, bq, bk)
        assert np.abs(got - _brute_mass(q, k, lse, 0.9, bq, bk)).max() < 1e-12


def pin_block_mass_rows_sum_to_block_height():
    """With the exact LSE every row's weights sum to 1: a block row holds its row count."""
    r = _rng(3)
    S, bq, bk = 300, 64, 32
    q, k = r.standard_normal((2, S, 6)) * 1.5
    M = A.block_mass(q, k, A.row_lse(q, k, 0.4), 0.4, bq, bk)
    heights = np.minimum(bq, S - bq * np.arange(M.shape[0]))
    assert np.abs(M.sum(axis=1) - heights).max() < 1e-10
    # a cached LSE that is off by delta scales every mass by exp(-delta)
    M2 = A.block_mass(q, k, A.row_lse(q, k, 0.4) + 0.3, 0.4, bq, bk)
    assert np.abs(M2 - M * math.exp(-0.3)).max() < 1e-12


def pin_select_brute_force():
    r = _rng(4)
    for trial in range(60):
        n = int(r.integers(1, 8))
        M = (r.dirichlet(np.ones(n) * 0.8) * r.uniform(0.5, 50))[None, :]
        cov = float(r.choice([0.5, 0.8, 0.9, 0.95, 1.0]))
        sel = A.select_blocks(M, cov)[0]
        target = cov * M.sum()
        best_k, best_sum = None, None
        for kk in range(1, n + 1):
            sums = [M[0, list(s)].sum() for s in itertools.combinations(range(n), kk)]
            if max(sums) >= target - 1e-12 * M.sum():
                best_k, best_sum = kk, max(sums)
                break
        if best_k is None:
            assert sel.all()
            continue
        assert sel.sum() == best_k
        assert abs(M[0, sel].sum() - best_sum) < 1e-12 * M.sum()


def pin_select_hand_cases():
    M = np.array([[2.0, 4.0, 2.0, 0.0], [0.0, 0.0, 0.0, 5.0]])
    assert A.select_blocks(M, 0.75).tolist() == [[True, True, False, False], [False, False, False, True]]
    assert A.select_blocks(M, 0.76)[0].tolist() == [True, True, True, False]
    assert A.select_blocks(M, 1.0)[0].tolist() == [True, True, True, False]     # zero mass never
    with pytest.raises(ValueError):
        A.select_blocks(M, 0.0)


def pin_attention_all_blocks_is_dense():
    r = _rng(5)
    S, D = 150, 8
    q, k, v = r.standard_normal((3, S, D))
    sel = np.ones((-(-S // 32), -(-S // 16)), dtype=bool)
    got = A.block_sparse_attention(q, k, v, sel, 0.3, 32, 16)
    assert np.abs(got - O.attention(q, k, v, np.ones((S, S), bool), 0.3)).max() < 1e-13


def pin_attention_hand_example():
    # zero queries: every allowed key weighs the same; rows 0-1 form query block 0, rows 2-3
    # block 1; key blocks of 2: block 0 = keys 0-1, block 1 = keys 2-3, block 2 = key 4
    q = np.zeros((4, 2))
    k = np.arange(10.0).reshape(5, 2)
    v = np.array([[1.0, 0], [2, 0], [3, 0], [4, 0], [5, 1]])
    sel = np.array([[True, False, True], [False, True, False]])
    out = A.block_sparse_attention(q, k, v, sel, 1.0, 2, 2)
    assert np.abs(out[0] - [(1 + 2 + 5) / 3, 1 / 3]).max() < 1e-15
    assert np.abs(out[3] - [3.5, 0.0]).max() < 1e-15


def pin_token_mask_brute_force():
    r = _rng(6)
    S, bq, bk = 23, 5, 4
    sel = r.random((-(-S // bq), -(-S // bk))) < 0.5
    m = A.block_token_mask(sel, np.arange(S), S, bq, bk)
    for a in range(S):
        for b in range(S):
            assert m[a, b] == sel[a // bq][b // bk]


ALL_PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_") and callable(v)]


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()
