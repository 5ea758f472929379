"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what it pins.  Together they are chosen so that a plausible
slip anywhere in the oracle (strict instead of inclusive comparison, a
dropped dimension or term, a wrong row or column index, a different
summation order, a missing self pair, a mirrored pair lost) fails at least
one of them.  The worked examples come from "RT-HiSS: Ray Tracing
Accelerated High Dimensional Vector Similarity Searches" (Fig. 3, Fig. 5)
and are stored under tests/golden/ with their citations.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import fig3_points, fig5_points, lattice

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U64 = 2.0 ** -53


def gamma(n, u=U64):
    return n * u / (1 - n * u)


def pair_set(P):
    return set(map(tuple, np.asarray(P, dtype=np.int64).tolist()))


# ---- inclusive comparison and the squared test (Sec. II-A: dist <= eps) ----

def test_345_boundary_inclusive():
    X = np.array([[0, 0], [3, 4]], dtype=np.float32)
    assert oracle.d64(X[0], X[1]) == 25.0
    assert pair_set(oracle.selfjoin_pairs(X, 5.0)) == {(0, 0), (0, 1), (1, 0), (1, 1)}
    below = math.nextafter(5.0, 0.0)
    assert pair_set(oracle.selfjoin_pairs(X, below)) == {(0, 0), (1, 1)}


# ---- the canonical binary64 squared distance ----

def test_d64_integer_inputs_exact():
    rng = np.random.default_rng(11)
    for d in (1, 3, 16, 57, 384):
        a = rng.integers(-1000, 1000, d).astype(np.float32)
        b = rng.integers(-1000, 1000, d).astype(np.float32)
        exact = sum((int(x) - int(y)) ** 2 for x, y in zip(a, b))
        assert oracle.d64(a, b) == float(exact)


@pytest.mark.parametrize("scale", [1e-30, 1e-3, 1.0, 1e4, 1e30])
def test_d64_within_error_bound_of_exact(scale):
    rng = np.random.default_rng(12)
    for d in (2, 18, 64, 384):
        a = (rng.standard_normal(d) * scale).astype(np.float32)
        b = (rng.standard_normal(d) * scale).astype(np.float32)
        exact = sum((Fraction(float(x)) - Fraction(float(y))) ** 2 for x, y in zip(a, b))
        got = Fraction(oracle.d64(a, b))
        assert abs(got - exact) <= Fraction(gamma(d + 2)) * exact


def test_d64_sequential_in_input_dimension_order():
    # four terms of 2^-54 then a 1: summed first to last they reach 1 + 2^-52
    # exactly; summed last to first each small term is lost to rounding.
    t = np.float32(2.0 ** -27)
    a = np.array([t, t, t, t, 1.0], dtype=np.float32)
    z = np.zeros(5, dtype=np.float32)
    assert oracle.d64(a, z) == 1.0 + 2.0 ** -52
    assert oracle.d64(a[::-1].copy(), z) == 1.0


def test_e64_is_rounded_square():
    for eps in (0.1, 1.0 / 3.0, 0.8931347294895747, 5.0):
        assert oracle.e64(eps) == eps * eps
    assert Fraction(oracle.e64(0.1)) != Fraction(0.1) ** 2


# ---- closed forms on integer lattices ----

def lattice_count(m, d, e2):
    """Ordered pairs of {0..m-1}^d at squared distance <= e2 (e2 < 3)."""
    per_axis_pairs = 2 * (m - 1)          # ordered (a, b) with |a-b| = 1
    c = m ** d
    if e2 >= 1:
        c += d * per_axis_pairs * m ** (d - 1)
    if e2 >= 2:
        c += math.comb(d, 2) * per_axis_pairs ** 2 * m ** (d - 2)
    return c


@pytest.mark.parametrize("m,d", [(3, 1), (7, 2), (5, 3), (3, 5)])
def test_lattice_closed_forms(m, d):
    X = lattice(m, d)
    assert X.shape == (m ** d, d)
    assert oracle.selfjoin_pairs(X, 1.0).shape[0] == lattice_count(m, d, 1.0)
    assert oracle.selfjoin_pairs(X, math.nextafter(1.0, 0)).shape[0] == m ** d
    e = math.sqrt(2.0)
    assert e * e >= 2.0
    assert oracle.selfjoin_pairs(X, e).shape[0] == lattice_count(m, d, 2.0)


def test_lattice_1d_m3_is_seven():
    assert oracle.selfjoin_pairs(lattice(3, 1), 1.0).shape[0] == 7


def test_lattice_per_row_counts():
    m, d = 4, 3
    X = lattice(m, d)
    colptr, _ = oracle.join_rows(X, 1.0)
    counts = np.diff(colptr)
    idx = np.stack(np.meshgrid(*[np.arange(m)] * d, indexing="ij"), -1).reshape(-1, d)
    expect = 1 + ((idx > 0).astype(int) + (idx < m - 1).astype(int)).sum(1)
    assert np.array_equal(counts, expect)


# ---- limits and invariants ----

def test_eps_inf_and_diameter_give_all_pairs():
    rng = np.random.default_rng(13)
    X = rng.random((150, 7), dtype=np.float32)
    n = X.shape[0]
    assert oracle.selfjoin_pairs(X, math.inf).shape[0] == n * n
    assert oracle.selfjoin_pairs(X, math.sqrt(7) + 1e-6).shape[0] == n * n


def test_eps_zero_counts_duplicate_groups():
    rng = np.random.default_rng(14)
    base = rng.random((20, 5), dtype=np.float32)
    sizes = rng.integers(1, 6, 20)
    X = np.repeat(base, sizes, axis=0)
    X = X[rng.permutation(X.shape[0])]
    P = oracle.selfjoin_pairs(X, 0.0)
    assert P.shape[0] == int((sizes ** 2).sum())
    assert np.all(np.all(X[P[:, 0]] == X[P[:, 1]], axis=1))


def test_symmetry_selfinclusion_monotonicity():
    rng = np.random.default_rng(15)
    X = rng.random((400, 6), dtype=np.float32)
    prev = None
    for eps in (0.0, 0.1, 0.2, 0.35, 0.5):
        S = pair_set(oracle.selfjoin_pairs(X, eps))
        assert all((j, i) in S for (i, j) in S)
        assert all((i, i) in S for i in range(X.shape[0]))
        if prev is not None:
            assert prev <= S
        prev = S


def test_row_permutation_permutes_pairs():
    rng = np.random.default_rng(16)
    X = rng.random((300, 9), dtype=np.float32)
    perm = rng.permutation(300)
    A = pair_set(oracle.selfjoin_pairs(X, 0.45))
    B = pair_set(oracle.selfjoin_pairs(X[perm], 0.45))
    assert {(int(perm[i]), int(perm[j])) for i, j in B} == A


def test_selected_rows_match_full_join():
    rng = np.random.default_rng(17)
    X = rng.random((500, 4), dtype=np.float32)
    cp_all, c_all = oracle.join_rows(X, 0.2)
    rows = np.array([499, 0, 17, 17, 250])
    cp, c = oracle.join_rows(X, 0.2, rows)
    for r, i in enumerate(rows):
        assert np.array_equal(c[cp[r]:cp[r + 1]], c_all[cp_all[i]:cp_all[i + 1]])


def test_brute_force_tiny_python():
    """Plain double loop over python floats, compared on a tiny input."""
    rng = np.random.default_rng(18)
    X = (rng.random((40, 3)) * 4).astype(np.float32)
    eps = 1.3
    want = set()
    for i in range(40):
        for j in range(40):
            s = sum((float(X[i, k]) - float(X[j, k])) ** 2 for k in range(3))
            if s <= eps * eps:
                want.add((i, j))
    assert pair_set(oracle.selfjoin_pairs(X, eps)) == want


def test_agrees_with_scipy_ckdtree_outside_band():
    from scipy.spatial import cKDTree
    rng = np.random.default_rng(19)
    X = rng.random((3000, 5), dtype=np.float32)
    eps = 0.12
    S = pair_set(oracle.selfjoin_pairs(X, eps))
    kd = cKDTree(X.astype(np.float64))
    T = {(i, j) for i, j in kd.query_pairs(eps, output_type="ndarray").tolist()}
    T |= {(j, i) for (i, j) in T} | {(i, i) for i in range(X.shape[0])}
    e2 = eps * eps
    for (i, j) in S ^ T:
        assert abs(oracle.d64(X[i], X[j]) - e2) <= 1e-12 * e2, (i, j)


# ---- worked examples on the pages ----

def test_fig3_neighbour_structure():
    with open(os.path.join(GOLDEN, "fig3_pairs.json")) as f:
        g = json.load(f)
    want = {tuple(p) for p in g["pairs"]} | {(i, i) for i in range(7)}
    want |= {(j, i) for (i, j) in want}
    assert pair_set(oracle.selfjoin_pairs(fig3_points(), g["eps"])) == want


def test_fig5_row_positions():
    with open(os.path.join(GOLDEN, "fig5_compaction.json")) as f:
        g = json.load(f)
    mask = g["mask"]
    assert [i for i, b in enumerate(mask) if b] == g["compressed"]
    colptr, cols = oracle.join_rows(fig5_points(), 1.0, [g["query"]])
    assert cols.tolist() == g["compressed"]


# ---- epsilon calibration ----

def test_calibration_selects_kth_smallest():
    rng = np.random.default_rng(20)
    X = rng.random((300, 4), dtype=np.float32)
    nq, k = 30, 5
    vals = sorted(oracle.d64(X[q], X[j]) for q in range(nq) for j in range(300) if j != q)
    a, b = oracle.calibrate_bounds(X, nq, k)
    assert (a, b) == (vals[nq * k - 1], vals[nq * k])
    eps, _, _ = oracle.calibrate_eps(X, nq, k)
    colptr, _ = oracle.join_rows(X, eps, np.arange(nq))
    assert int(colptr[-1]) - nq == nq * k


def test_calibration_heap_retry_path():
    """A clustered query has far more than 4k neighbours below b: the first
    heap size is too small and the routine must grow it."""
    rng = np.random.default_rng(21)
    X = np.concatenate([np.zeros((400, 3)), rng.random((2000, 3)) * 10]).astype(np.float32)
    X[:400] += rng.random((400, 3)).astype(np.float32) * 1e-3
    a, b = oracle.calibrate_bounds(X, 10, 2)
    vals = sorted(oracle.d64(X[q], X[j]) for q in range(10) for j in range(X.shape[0]) if j != q)
    assert (a, b) == (vals[19], vals[20])


def test_rejects_bad_input():
    X = np.ones((4, 3), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.join_rows(X, -1.0)
    with pytest.raises(ValueError):
        oracle.join_rows(X, float("nan"))
    X[2, 1] = np.inf
    with pytest.raises(ValueError):
        oracle.join_rows(X, 1.0)


def test_oracle_d64_is_unfused():
    """For pairs where a fused multiply-add accumulation rounds differently,
    the oracle returns the canonical (separately rounded) value and decides
    the pair at fl(eps^2) accordingly."""
    from fused_pairs import canonical_d64, discriminating_pairs
    for a, b, eps, inside in discriminating_pairs(40, 7, 5):
        assert oracle.d64(a, b) == canonical_d64(a, b)
        X = np.stack([a, b])
        got = {tuple(p) for p in oracle.selfjoin_pairs(X, eps).tolist()}
        assert ((0, 1) in got) == inside and ((1, 0) in got) == inside
