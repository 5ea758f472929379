"""Tighter pruning keeps the oracle's pair set exactly.

The finer grid (grid_reach = 2: cells of width eps/2, 5x5x5 stencil) with
both refinement kernels, never with more candidates than the default grid;
and the block box test of both kernels (on by default, compared here with
it switched off): it must skip work on clustered data and change nothing.
Cases: random data with ragged sizes, clustered workload shapes, lattices
with pairs exactly at eps (cell walls at multiples of eps/2, box gaps of
exactly eps), eps = 0, and the semi-join."""
import math

import numpy as np
import pytest
import torch

import exact_range_similarity_amd as ersj
import oracle
from workloads import lattice, make_config, make_queries

from gpu_util import KERNELS, check_against_oracle, keys_of, say

pytestmark = pytest.mark.gpu
FINE = ersj.default_options(grid_reach=2)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ersj.lib()


def candidates(X, eps, reach):
    h = ersj.build_index(torch.from_numpy(X).cuda(), eps, ersj.default_options(grid_reach=reach))
    total = ersj.count_pass(h)
    st = ersj.get_stats(h)
    h.free()
    return total, st["cells"]


@pytest.mark.parametrize("n,d", [(1, 3), (257, 5), (2000, 2), (3001, 9), (1500, 40)])
def test_random(n, d):
    rng = np.random.default_rng(n + 100 * d)
    X = rng.random((n, d), dtype=np.float32)
    for eps in (0.05 * math.sqrt(d), 0.3 * math.sqrt(d)):
        check_against_oracle(X, eps, f"reach 2 random n={n} d={d}", options=FINE)


@pytest.mark.parametrize("name,n", [("c2", 20000), ("c4", 30011), ("c3", 8000)])
def test_workload_shapes_and_fewer_candidates(name, n):
    X = make_config(name, n)
    eps, _, _ = oracle.calibrate_eps(X, min(1000, n), 32)
    check_against_oracle(X, eps, f"reach 2 {name} n={n}", options=FINE)
    c1, m1 = candidates(X, eps, 1)
    c2, m2 = candidates(X, eps, 2)
    say(f"[gpu] {name} n={n}: candidates {c1} -> {c2}, cells {m1} -> {m2}")
    assert c2 <= c1 and m2 >= m1


@pytest.mark.parametrize("m,d", [(9, 2), (6, 3)])
def test_lattice_pairs_at_eps(m, d):
    X = lattice(m, d)
    for eps in (1.0, math.nextafter(1.0, 0.0), 2.0, math.sqrt(2.0), 0.5):
        check_against_oracle(X, eps, f"reach 2 lattice m={m} d={d}", options=FINE)


def test_eps_zero_and_infinite():
    rng = np.random.default_rng(61)
    base = rng.random((40, 4), dtype=np.float32)
    X = np.repeat(base, 3, axis=0)
    check_against_oracle(X, 0.0, "reach 2 eps = 0", options=FINE)
    for k in KERNELS:
        got = ersj.pairs_to_numpy(ersj.self_join(torch.from_numpy(base).cuda(), math.inf,
                                                 options=ersj.default_options(grid_reach=2,
                                                                              refine_kernel=k)))
        assert got.shape[0] == 40 * 40


def test_semi_join_with_the_finer_grid():
    X = make_config("c2", 15000)
    Q = make_queries("c2", 4000, 7, 15000)
    eps = 0.11
    want = np.sort(keys_of(oracle.semijoin_pairs(Q, X, eps)))
    for k in KERNELS:
        opts = ersj.default_options(grid_reach=2, refine_kernel=k)
        parts = ersj.semi_join(torch.from_numpy(Q).cuda(), torch.from_numpy(X).cuda(), eps, 0, opts)
        got = np.sort(keys_of(ersj.pairs_to_numpy(parts)))
        assert np.array_equal(got, want)


def _join(X, eps, kernel=ersj.REFINE_MFMA, **opt):
    h = ersj.build_index(torch.from_numpy(X).cuda(), eps,
                         ersj.default_options(refine_kernel=kernel, timing=1, **opt))
    ersj.count_pass(h)
    nb = ersj.plan_batches(h, 0)
    parts = list(ersj.iter_batches(h, nb))
    st = ersj.get_stats(h)
    h.free()
    return np.sort(keys_of(ersj.pairs_to_numpy(parts))), st


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("name,n,reach", [("c2", 40000, 1), ("c2", 40000, 2), ("c4", 30011, 1),
                                          ("c3", 9000, 1)])
def test_block_prune_skips_work_and_changes_nothing(name, n, reach, kernel):
    X = make_config(name, n)
    eps, _, _ = oracle.calibrate_eps(X, min(1000, n), 32)
    want = np.sort(keys_of(oracle.selfjoin_pairs(X, eps)))
    on, st_on = _join(X, eps, kernel, grid_reach=reach)
    off, st_off = _join(X, eps, kernel, grid_reach=reach, block_prune=-1)
    say(f"[gpu] {name} n={n} reach={reach} kernel={kernel}: skipped "
        f"{st_on['skipped_candidates']} of {st_on['refined_candidates']} comparisons")
    assert np.array_equal(on, want) and np.array_equal(off, want)
    assert st_off["skipped_candidates"] == 0
    assert st_on["skipped_candidates"] < st_on["refined_candidates"]
    # at this size c2's cells hold one or two clusters' worth of rows and no
    # block of them is ε away from another; the clustered workloads prune
    if name != "c2":
        assert st_on["skipped_candidates"] > 0
    assert st_on["last_skipped"] == st_on["skipped_candidates"]  # one batch


@pytest.mark.parametrize("m,d", [(9, 2), (6, 3), (5, 4)])
def test_block_prune_lattice_at_eps(m, d):
    # integer lattices: many box gaps equal eps exactly; eps just below an
    # integer distance puts the threshold between lattice distances
    X = lattice(m, d)
    for eps in (1.0, math.nextafter(1.0, 0.0), 2.0, math.nextafter(2.0, 3.0), 3.0):
        want = np.sort(keys_of(oracle.selfjoin_pairs(X, eps)))
        for k in KERNELS:
            got, st = _join(X, eps, k)
            assert np.array_equal(got, want), (m, d, eps, k)


def test_norm_test_on_clusters_apart_off_the_grid_axes():
    # Two point families share the grid cells but sit in opposite corners of
    # them (so their query blocks are pure and the box test keeps them
    # paired) and 3 apart on a fourth axis: the refinement's norm test
    # decides their cross products.  Partners of the first family one unit up
    # on that axis are exactly eps = 1 away; every coordinate is a multiple of
    # 1/16, so all distances are exact.
    rng = np.random.default_rng(71)
    n = 1500
    cell = rng.integers(0, 8, size=(n, 3)).astype(np.float32)
    fine = rng.integers(0, 2, size=(n, 3)).astype(np.float32) / 16
    A = np.zeros((n, 8), np.float32)
    A[:, :3] = cell + fine
    B = A.copy()
    B[:, :3] += np.float32(14 / 16)
    B[:, 3] = 3.0
    C = A[: n // 3].copy()
    C[:, 3] = 1.0
    X = np.concatenate([A, B, C])
    X = X[rng.permutation(len(X))]
    check_against_oracle(X, 1.0, "families apart on a fourth axis")
    check_against_oracle(X, math.nextafter(1.0, 0.0), "families apart, eps just below 1")


@pytest.mark.parametrize("name,n", [("c2", 20000), ("c3", 12000), ("c4", 30011), ("c1", 5000)])
def test_cell_order_keeps_pairs_and_prunes_more(name, n):
    # rows of a cell in Morton order over the cell's box in the first 8
    # dimensions (cell_order 2, the default for the MFMA kernels) against
    # 8 x 8 x 8 sub-cells on the grid axes (1): the same pairs and the same
    # candidates (the pruning each order gets at full size is measured by
    # the benchmark)
    X = make_config(name, n)
    eps, _, _ = oracle.calibrate_eps(X, min(1000, n), 32)
    want = np.sort(keys_of(oracle.selfjoin_pairs(X, eps)))
    st = {}
    for order in (2, 1):
        got, st[order] = _join(X, eps, ersj.REFINE_MFMA16, cell_order=order)
        say(f"[gpu] {name} n={n} cell_order={order}: candidates {st[order]['refined_candidates']}, "
            f"box-settled {st[order]['skipped_candidates']}")
        assert np.array_equal(got, want), f"{name} cell_order={order}"
    assert st[2]["refined_candidates"] == st[1]["refined_candidates"]


@pytest.mark.parametrize("case", ["c5", "rand100", "dups80", "tiny", "one_cell_large"])
def test_tree_order_keeps_pairs(case):
    # rows of each cell as the leaves of a balanced tree (cell_order 3, the
    # default above 64 dimensions) against the 8-dimension kd order (2): the
    # same pairs; the tree's 32-row blocks of clustered data are purer, so
    # at least as many comparisons are settled by the partial test
    rng = np.random.default_rng(len(case))
    if case == "c5":
        X = make_config("c5", 6000)
        eps, _, _ = oracle.calibrate_eps(X, 1000, 50)
    elif case == "rand100":
        X = rng.random((3001, 100), dtype=np.float32)
        eps = 0.33 * math.sqrt(100 / 6.0)
    elif case == "dups80":
        # many equal rows and equal values in every dimension: zero sampled
        # variance in most nodes, ties everywhere in the sort
        base = rng.integers(0, 3, size=(60, 80)).astype(np.float32)
        X = base[rng.integers(0, 60, 2500)]
        eps = 1.5
    elif case == "tiny":
        X = rng.random((45, 70), dtype=np.float32)
        eps = 1.2
    else:
        # one cell far larger than the 2^k leaf sizes, ragged at its end
        X = rng.normal(0.0, 1.0, (5003, 66)).astype(np.float32)
        eps = 9.0
    want = np.sort(keys_of(oracle.selfjoin_pairs(X, eps)))
    st = {}
    for order in (3, 2):
        got, st[order] = _join(X, eps, ersj.REFINE_MFMA16, cell_order=order)
        say(f"[gpu] tree order {case} n={X.shape[0]} d={X.shape[1]} cell_order={order}: {got.size} pairs, "
            f"settled from 64 dimensions {st[order]['last_partial']}")
        assert np.array_equal(got, want), f"{case} cell_order={order}"
    auto, st0 = _join(X, eps, ersj.REFINE_MFMA16)
    assert np.array_equal(auto, want)
    assert st0["last_partial"] == st[3]["last_partial"]  # the default above 64 dimensions
    if case == "c5":
        assert st[3]["last_partial"] >= st[2]["last_partial"]


def test_tree_order_semi_join():
    X = make_config("c5", 6000)
    Q = make_queries("c5", 2500, 11, 6000)
    eps, _, _ = oracle.calibrate_eps(X, 1000, 50)
    want = np.sort(keys_of(oracle.semijoin_pairs(Q, X, eps)))
    for order in (3, 1):
        opts = ersj.default_options(cell_order=order)
        parts = ersj.semi_join(torch.from_numpy(Q).cuda(), torch.from_numpy(X).cuda(), eps, 0, opts)
        got = np.sort(keys_of(ersj.pairs_to_numpy(parts)))
        assert np.array_equal(got, want), order
