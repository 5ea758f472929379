"""Pins of the oracle's semi-join (RT-HiSS Sec. II-A: a query set Q distinct
from the dataset D; (q_j, p_i) is a result pair iff dist(p_i, q_j) <= eps).

Each fact comes from outside the oracle's semi-join routine: the self-join
it must reduce to, a closed form on a lattice, the symmetry of the distance,
and a plain python double loop.
"""
import math

import numpy as np
import pytest

import oracle
from workloads import lattice


def pair_set(P):
    return set(map(tuple, np.asarray(P, dtype=np.int64).tolist()))


def test_semijoin_with_q_equal_x_is_the_selfjoin():
    rng = np.random.default_rng(31)
    X = rng.random((500, 6), dtype=np.float32)
    for eps in (0.0, 0.25, 0.6):
        assert np.array_equal(oracle.semijoin_pairs(X, X, eps), oracle.selfjoin_pairs(X, eps))


def test_semijoin_query_rows_are_selfjoin_rows():
    rng = np.random.default_rng(32)
    X = rng.random((400, 4), dtype=np.float32)
    rows = rng.choice(400, 57, replace=False)
    cp_s, c_s = oracle.join_rows(X, 0.3, rows)
    cp_q, c_q = oracle.semijoin_rows(X[rows], X, 0.3)
    assert np.array_equal(cp_s, cp_q) and np.array_equal(c_s, c_q)


@pytest.mark.parametrize("m,d", [(4, 2), (3, 3), (3, 4)])
def test_cell_centres_see_their_corners(m, d):
    """Q = centres of the unit cells of the Z^d box [0, m)^d, X = its lattice
    points.  A centre is at squared distance d/4 from its 2^d corners and at
    least d/4 + 2 from every other lattice point (both exact in binary64), so
    with the smallest eps whose square reaches d/4 every query has exactly 2^d
    neighbours, and with the largest eps whose square stays below, none."""
    X = lattice(m, d)
    Q = (lattice(m - 1, d) + np.float32(0.5)).astype(np.float32)
    t = d / 4.0
    hi = math.sqrt(t)
    while hi * hi < t:
        hi = math.nextafter(hi, math.inf)
    while math.nextafter(hi, 0.0) ** 2 >= t:
        hi = math.nextafter(hi, 0.0)
    lo = math.nextafter(hi, 0.0)
    assert hi * hi >= t > lo * lo
    cp, _ = oracle.semijoin_rows(Q, X, hi)
    assert np.all(np.diff(cp) == 2 ** d)
    cp, _ = oracle.semijoin_rows(Q, X, lo)
    assert cp[-1] == 0


def test_swapping_roles_transposes_the_pairs():
    rng = np.random.default_rng(33)
    X = rng.random((300, 5), dtype=np.float32)
    Q = rng.random((170, 5), dtype=np.float32)
    a = pair_set(oracle.semijoin_pairs(Q, X, 0.35))
    b = pair_set(oracle.semijoin_pairs(X, Q, 0.35))
    assert a == {(j, i) for (i, j) in b}
    assert len(a) > 0


def test_semijoin_brute_force_tiny_python():
    rng = np.random.default_rng(34)
    X = (rng.random((30, 3)) * 4).astype(np.float32)
    Q = (rng.random((25, 3)) * 4).astype(np.float32)
    eps = 1.1
    want = set()
    for j in range(25):
        for i in range(30):
            s = sum((float(Q[j, k]) - float(X[i, k])) ** 2 for k in range(3))
            if s <= eps * eps:
                want.add((j, i))
    assert pair_set(oracle.semijoin_pairs(Q, X, eps)) == want


def test_far_queries_and_limits():
    rng = np.random.default_rng(35)
    X = rng.random((200, 3), dtype=np.float32)
    far = X + np.float32(10.0)
    assert oracle.semijoin_pairs(far, X, 1.0).shape[0] == 0
    assert oracle.semijoin_pairs(far, X, math.inf).shape[0] == 200 * 200
    counts = [oracle.semijoin_pairs(X[:50], X, e).shape[0] for e in (0.1, 0.2, 0.4)]
    assert counts == sorted(counts)


def test_semijoin_rejects_bad_input():
    X = np.zeros((10, 3), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.semijoin_rows(np.zeros((4, 2), dtype=np.float32), X, 1.0)
    Q = np.zeros((4, 3), dtype=np.float32)
    Q[1, 2] = np.nan
    with pytest.raises(ValueError):
        oracle.semijoin_rows(Q, X, 1.0)
