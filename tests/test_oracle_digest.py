"""Pins of the oracle's neighbour-list fingerprints and its threshold-band count.

The result these summarise is the self-join of "RT-HiSS: Ray Tracing
Accelerated High Dimensional Vector Similarity Searches", Sec. II-A (pairs
at Euclidean distance at most eps, self pairs included).  The pins come
from outside the oracle: the published output sequence of the splitmix64
generator, integer-lattice neighbourhoods enumerated by index arithmetic,
closed-form pair counts at a given lattice distance, and exact rational
arithmetic on inputs whose binary64 squared distance is exact.  The band is
the set of pairs whose squared distance lies within rel * eps^2 of eps^2,
the pairs a reduced-precision classifier cannot decide without the exact
test.
"""
import itertools
import math
import os
import sys
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import lattice, make_config

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import make_digests  # noqa: E402

GOLDEN_RATIO_64 = 0x9e3779b97f4a7c15
M64 = (1 << 64) - 1


def test_mix64_is_splitmix64_output():
    # splitmix64 started from state 0 outputs these three words first
    # (the state advances by the golden-ratio constant before each output)
    want = [0xe220a8397b1dcdaf, 0x6e789e6aa1b965f4, 0x06c45d188009454f]
    for k, w in enumerate(want):
        assert oracle.mix64((k * GOLDEN_RATIO_64) & M64) == w
    v = np.array([(k * GOLDEN_RATIO_64) & M64 for k in range(3)], dtype=np.uint64)
    with np.errstate(over="ignore"):
        assert make_digests.mix64_np(v).tolist() == want


def lattice_ids(m, d):
    """Row id of lattice point p in ``lattice(m, d)`` (row-major enumeration)."""
    return lambda p: sum(c * m ** (d - 1 - k) for k, c in enumerate(p))


@pytest.mark.parametrize("m,d", [(4, 3), (3, 4), (7, 2)])
def test_digests_on_lattice_by_index_arithmetic(m, d):
    X = lattice(m, d)
    rid = lattice_ids(m, d)
    want_c, want_h, want_b = [], [], []
    for p in itertools.product(range(m), repeat=d):
        nb = [p]
        for k in range(d):
            for s in (-1, 1):
                q = list(p)
                q[k] += s
                if 0 <= q[k] < m:
                    nb.append(tuple(q))
        want_c.append(len(nb))
        want_h.append(sum(oracle.mix64(rid(q)) for q in nb) & M64)
        want_b.append(len(nb) - 1)  # exactly at distance 1; the self pair is 1 away from eps^2
    for fn in (lambda: oracle.digest_all(X, 1.0), lambda: oracle.digest_rows(X, 1.0)):
        c, h, b = fn()
        assert c.tolist() == want_c
        assert [int(v) for v in h] == want_h
        assert b.tolist() == want_b


@pytest.mark.parametrize("m,d", [(4, 3), (5, 2), (3, 4)])
def test_band_count_lattice_closed_forms(m, d):
    X = lattice(m, d)
    # pairs at squared distance exactly 1 (one coordinate differs by one)
    n1 = 2 * d * (m - 1) * m ** (d - 1)
    assert oracle.band_count(X, 1.0) == n1
    # eps = sqrt(2): fl(eps^2) is 2 + 2^-51, within 1e-6 of 2 but not of 1
    n2 = math.comb(d, 2) * 4 * (m - 1) ** 2 * m ** (d - 2)
    e = math.sqrt(2.0)
    assert oracle.band_count(X, e) == n2
    assert int(oracle.digest_all(X, e)[2].sum()) == n2
    # rel = 0 keeps only pairs exactly at fl(eps^2)
    assert oracle.band_count(X, 1.0, rel=0.0) == n1
    assert oracle.band_count(X, e, rel=0.0) == 0


def test_band_edges_exact_rational():
    # One dimension: every coordinate is a float32 near 0 or near 1, so each
    # difference and its square are exact in binary64 and D64 is the exact
    # squared distance; membership |D64 - 1| <= fl(1e-6) is then decided in
    # exact rational arithmetic.
    pts = [0.0]
    for t in np.linspace(-3e-6, 3e-6, 61):
        pts.append(float(np.float32(math.sqrt(1.0 + t))))
    for t in (-1e-6, 1e-6):  # the float32 roots nearest the band edges and their neighbours
        r = np.float32(math.sqrt(1.0 + t))
        pts += [float(np.nextafter(r, np.float32(0))), float(r), float(np.nextafter(r, np.float32(2)))]
    X = np.array(pts, dtype=np.float32).reshape(-1, 1)
    w = Fraction(1e-6)  # fl(1e-6 * fl(1 * 1))
    want = 0
    for a in X[:, 0]:
        for b in X[:, 0]:
            s = (Fraction(float(a)) - Fraction(float(b))) ** 2
            want += abs(s - 1) <= w
    assert 0 < want < X.shape[0] ** 2 // 4
    assert oracle.band_count(X, 1.0) == want
    assert int(oracle.digest_rows(X, 1.0)[2].sum()) == want
    assert int(oracle.digest_all(X, 1.0)[2].sum()) == want


def test_digests_match_neighbour_lists():
    X = make_config("c2", 3000)
    eps = 0.11
    colptr, cols = oracle.join_rows(X, eps)
    cnt = np.diff(colptr).astype(np.uint32)
    with np.errstate(over="ignore"):
        mixed = make_digests.mix64_np(cols.astype(np.uint64))
    h = np.array([int(mixed[colptr[i]:colptr[i + 1]].sum(dtype=np.uint64)) for i in range(X.shape[0])],
                 dtype=np.uint64)
    for c, d, b in (oracle.digest_all(X, eps), oracle.digest_rows(X, eps)):
        assert np.array_equal(c, cnt)
        assert np.array_equal(d, h)
    rows = np.array([5, 17, 2999, 0], dtype=np.int64)
    c, d, b = oracle.digest_rows(X, eps, rows)
    assert np.array_equal(c, cnt[rows]) and np.array_equal(d, h[rows])
    assert int(b.sum()) == oracle.band_count(X, eps, rows=rows)


def test_block_fold_sees_swapped_rows():
    rng = np.random.default_rng(3)
    cnt = rng.integers(1, 50, 200).astype(np.uint32)
    dig = rng.integers(0, 2 ** 63, 200, dtype=np.uint64)
    band = np.zeros(200, dtype=np.uint32)
    bc, fp, bb = make_digests.block_fold(cnt, dig, band)
    assert bc.size == 4 and int(bc.sum()) == int(cnt.sum())
    c2, d2 = cnt.copy(), dig.copy()
    c2[[3, 4]] = c2[[4, 3]]
    d2[[3, 4]] = d2[[4, 3]]
    _, fp2, _ = make_digests.block_fold(c2, d2, band)
    assert fp2[0] != fp[0] and np.array_equal(fp2[1:], fp[1:])
