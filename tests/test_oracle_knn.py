"""Pins of the oracle's exact kNN (RT-HiSS Sec. VI: k nearest neighbours as
similarity searches with a growing radius, exact; ranked by the canonical
binary64 squared distance D64, ties by the smaller point id).

Each fact comes from outside the oracle's kNN routine: closed forms on
integer lattices (shells of known radius, ids known from the row-major
enumeration), duplicated points, scipy's kd-tree on continuous data, and the
oracle's semi-join on both sides of the k-th distance.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.spatial import cKDTree

import oracle
from workloads import lattice


def lattice_id(c, m):
    i = 0
    for v in c:
        i = i * m + int(v)
    return i


@pytest.mark.parametrize("m,d", [(5, 2), (4, 3), (4, 4)])
def test_interior_lattice_points_closed_form(m, d):
    """An interior point of the lattice {0..m-1}^d has itself at distance 0,
    its 2d axis neighbours at 1 and its 2d(d-1) diagonal neighbours at 2
    (squared, exact); within a shell ids ascend."""
    X = lattice(m, d)
    k = 1 + 2 * d + 2 * d * (d - 1)
    interior = [c for c in itertools.product(range(1, m - 1), repeat=d)]
    rows = np.array([lattice_id(c, m) for c in interior], dtype=np.int64)
    ids, dist = oracle.knn(X, k, rows)
    for r, c in enumerate(interior):
        axis = sorted(lattice_id([c[a] + (s if a == b else 0) for a in range(d)], m)
                      for b in range(d) for s in (-1, 1))
        diag = sorted(lattice_id([c[a] + (sa if a == b1 else sb if a == b2 else 0) for a in range(d)], m)
                      for b1 in range(d) for b2 in range(b1 + 1, d) for sa in (-1, 1) for sb in (-1, 1))
        want = [lattice_id(c, m)] + axis + diag
        assert ids[r].tolist() == want
        assert dist[r].tolist() == [0.0] + [1.0] * len(axis) + [2.0] * len(diag)


def test_duplicates_rank_by_id():
    """Three copies of each point (ids i, i + n0, i + 2 n0): the first three
    neighbours of any copy are the three copies in id order, at distance 0."""
    rng = np.random.default_rng(41)
    base = rng.random((60, 5), dtype=np.float32)
    X = np.concatenate([base, base, base])
    ids, dist = oracle.knn(X, 3)
    for i in range(X.shape[0]):
        j = i % 60
        assert ids[i].tolist() == [j, j + 60, j + 120]
        assert dist[i].tolist() == [0.0, 0.0, 0.0]


@pytest.mark.parametrize("m,d", [(4, 2), (3, 3)])
def test_cell_centres_get_their_corners(m, d):
    """Q = centres of the unit cells of [0, m-1]^d: the 2^d corners are at
    squared distance d/4 (exact), every other lattice point at >= d/4 + 2."""
    X = lattice(m, d)
    Q = (lattice(m - 1, d) + np.float32(0.5)).astype(np.float32)
    ids, dist = oracle.knn_rows(Q, X, 2 ** d)
    cells = list(itertools.product(range(m - 1), repeat=d))
    for r, c in enumerate(cells):
        corners = sorted(lattice_id([c[a] + o[a] for a in range(d)], m)
                         for o in itertools.product((0, 1), repeat=d))
        assert ids[r].tolist() == corners
        assert np.all(dist[r] == d / 4.0)


@pytest.mark.parametrize("n,d,k", [(2000, 3, 10), (1500, 8, 32), (800, 20, 5)])
def test_agrees_with_a_kd_tree(n, d, k):
    """Continuous random data has no ties: scipy's kd-tree (its own distance
    code) returns the same neighbours in the same order, and the same
    distances to rounding."""
    rng = np.random.default_rng(n + d)
    X = rng.random((n, d), dtype=np.float32)
    Q = rng.random((300, d), dtype=np.float32)
    ids, dist = oracle.knn_rows(Q, X, k)
    td, ti = cKDTree(X.astype(np.float64)).query(Q.astype(np.float64), k=k)
    td = np.asarray(td).reshape(len(Q), k)
    ti = np.asarray(ti).reshape(len(Q), k)
    assert np.allclose(np.sqrt(dist), td, rtol=1e-12, atol=0)
    # neighbours whose distances are clearly apart must come in the same order
    gap = np.diff(np.concatenate([dist, np.full((len(Q), 1), np.inf)], axis=1), axis=1)
    sure = np.concatenate([np.ones((len(Q), 1), bool), gap[:, :-1] > 1e-9], axis=1) & (gap > 1e-9)
    assert np.array_equal(ids[sure], ti[sure].astype(np.uint32))
    assert sure.mean() > 0.99


def test_between_the_semijoins_at_the_kth_distance():
    """With r = D64 of the k-th neighbour: the semi-join at the largest eps
    with fl(eps^2) < r finds only kNN members (all strictly closer), and at
    the smallest eps with fl(eps^2) >= r it finds all of them."""
    rng = np.random.default_rng(44)
    X = rng.random((700, 6), dtype=np.float32)
    Q = rng.random((40, 6), dtype=np.float32)
    k = 12
    ids, dist = oracle.knn_rows(Q, X, k)
    for r in range(len(Q)):
        t = dist[r, -1]
        hi = math.sqrt(t)
        while hi * hi < t:
            hi = math.nextafter(hi, math.inf)
        while math.nextafter(hi, 0.0) ** 2 >= t:
            hi = math.nextafter(hi, 0.0)
        lo = math.nextafter(hi, 0.0)
        _, inner = oracle.semijoin_rows(Q[r:r + 1], X, lo)
        _, outer = oracle.semijoin_rows(Q[r:r + 1], X, hi)
        assert set(inner.tolist()) <= set(ids[r].tolist())
        assert set(ids[r].tolist()) <= set(outer.tolist())
        assert len(inner) < k <= len(outer)


def test_invariants_and_rows():
    rng = np.random.default_rng(45)
    X = rng.random((300, 4), dtype=np.float32)
    ids, dist = oracle.knn(X, X.shape[0])
    for r in range(X.shape[0]):
        assert sorted(ids[r].tolist()) == list(range(X.shape[0]))
        assert np.all(np.diff(dist[r]) >= 0)
        assert ids[r, 0] == r and dist[r, 0] == 0.0
    rows = np.array([5, 17, 299, 0])
    ids_r, dist_r = oracle.knn(X, 7, rows)
    ids_a, dist_a = oracle.knn(X, 7)
    assert np.array_equal(ids_r, ids_a[rows]) and np.array_equal(dist_r, dist_a[rows])


def test_bad_input():
    X = np.zeros((5, 2), dtype=np.float32)
    for k in (0, 6):
        with pytest.raises(ValueError):
            oracle.knn(X, k)
    Y = X.copy()
    Y[1, 1] = np.nan
    with pytest.raises(ValueError):
        oracle.knn(Y, 2)
