"""Pins of the oracle's top-k: brute-force sort with the (score desc, index asc) order."""
import numpy as np
import pytest

import oracle


def brute_topk(row, k, nv):
    order = sorted(range(nv), key=lambda j: (-float(row[j]), j))
    sel = sorted(order[:k])
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("seed", range(6))
def test_topk_random_rows_with_planted_ties(seed):
    rng = np.random.default_rng(seed)
    R, N = 8, 300
    s = rng.normal(size=(R, N)).astype(np.float32)
    # plant ties: copy values across positions, including at the k-boundary
    for r in range(R):
        src = rng.integers(0, N, 40)
        dst = rng.integers(0, N, 40)
        s[r, dst] = s[r, src]
    s[0, :] = 1.0  # all equal: the lowest indices win
    s[1, ::2] = 0.0
    s[1, 1::2] = -0.0  # -0 and +0 tie
    nv = rng.integers(0, N + 1, R)
    nv[2] = N
    for k in (1, 7, 64, 299, 300, 301):
        got = oracle.topk(s, k, n_valid=nv)
        for r in range(R):
            assert got[r].tolist() == brute_topk(s[r], k, int(nv[r])), (r, k)


def test_topk_all_equal_takes_lowest_indices():
    s = np.zeros((1, 1000), dtype=np.float32)
    got = oracle.topk(s, 10)
    assert got[0].tolist() == list(range(10))


def test_topk_fewer_valid_than_k_pads():
    s = np.arange(20, dtype=np.float32)[None, :]
    got = oracle.topk(s, 8, n_valid=np.array([5]))
    assert got[0].tolist() == [0, 1, 2, 3, 4, -1, -1, -1]


def test_topk_infinities_order():
    s = np.array([[-np.inf, 3.0, np.inf, -np.inf, 0.0]], dtype=np.float32)
    assert oracle.topk(s, 2)[0].tolist() == [1, 2]
    assert oracle.topk(s, 4)[0].tolist() == [0, 1, 2, 4]
