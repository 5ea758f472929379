"""Semi-join on the GPU (RT-HiSS Sec. II-A: query set Q distinct from the
dataset D) against the CPU oracle: identical (query id, point id) pair sets,
no duplicates, both refinement kernels.  Sizes span several row tiles and
candidate segments with ragged tails; the edge cases are queries outside the
points' bounding box (one cell out, far out), queries on duplicate points,
nq = 1, fewer than three grid dimensions, and the handle's state rules."""
import math

import numpy as np
import pytest
import torch

import exact_range_similarity_amd as ersj
import oracle
from workloads import lattice, make_config

from gpu_util import KERNELS, keys_of, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ersj.lib()


def gpu_semi(Q, X, eps, kernel, budget=0):
    opts = ersj.default_options(refine_kernel=kernel)
    q = torch.from_numpy(np.ascontiguousarray(Q, dtype=np.float32)).cuda()
    x = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).cuda()
    parts = ersj.semi_join(q, x, eps, budget, opts)
    torch.cuda.synchronize()
    return ersj.pairs_to_numpy(parts)


def check(Q, X, eps, label, kernels=KERNELS, budget=0):
    want = np.sort(keys_of(oracle.semijoin_pairs(Q, X, eps)))
    for k in kernels:
        say(f"[gpu] semi-join {label}: nq={Q.shape[0]} n={X.shape[0]} d={X.shape[1]} eps={eps!r} kernel={k}")
        got = np.sort(keys_of(gpu_semi(Q, X, eps, k, budget)))
        assert np.unique(got).size == got.size, f"{label} kernel={k}: duplicate pairs"
        if not np.array_equal(got, want):
            extra = np.setdiff1d(got, want)[:5]
            missing = np.setdiff1d(want, got)[:5]
            raise AssertionError(f"{label} kernel={k}: |gpu|={got.size} |oracle|={want.size} "
                                 f"extra={extra.tolist()} missing={missing.tolist()}")
    return want.size


@pytest.mark.parametrize("nq,n,d", [(1, 500, 4), (700, 3000, 8), (4000, 2500, 16), (2100, 6000, 33),
                                    (300, 300, 2), (513, 777, 1), (900, 1200, 3), (1500, 2000, 48),
                                    (600, 900, 100), (257, 300, 200)])
def test_random_queries(nq, n, d):
    rng = np.random.default_rng(nq * 7 + n + d)
    X = rng.random((n, d), dtype=np.float32)
    Q = rng.random((nq, d), dtype=np.float32)
    for eps in (0.08 * math.sqrt(d), 0.25 * math.sqrt(d)):
        check(Q, X, eps, f"random nq={nq} n={n} d={d}")


def test_queries_equal_to_points_give_the_self_join():
    X = make_config("c2", 12000)
    eps = 0.11
    want = np.sort(keys_of(oracle.selfjoin_pairs(X, eps)))
    for k in KERNELS:
        got = np.sort(keys_of(gpu_semi(X, X, eps, k)))
        assert np.array_equal(got, want)


def test_queries_outside_the_box():
    rng = np.random.default_rng(41)
    X = rng.random((3000, 5), dtype=np.float32)
    eps = 0.2
    near = rng.random((500, 5), dtype=np.float32)
    near[:, 0] = -0.15 - 0.1 * rng.random(500, dtype=np.float32)   # up to ~1-2 cells below
    near[250:, 1] = 1.1 + 0.1 * rng.random(250, dtype=np.float32)  # above on another axis
    far = rng.random((200, 5), dtype=np.float32) + np.float32(7.0)
    Q = np.concatenate([near, far, X[:100] + np.float32(0.05)])
    n_pairs = check(Q, X, eps, "queries around and far outside the box")
    assert n_pairs > 0
    assert gpu_semi(far, X, eps, ersj.REFINE_AUTO).shape[0] == 0


def test_duplicate_points_and_queries_on_them():
    rng = np.random.default_rng(42)
    base = rng.random((60, 6), dtype=np.float32)
    X = np.repeat(base, rng.integers(1, 6, 60), axis=0)
    Q = np.concatenate([base[::3], base[::3]])
    check(Q, X, 0.0, "eps = 0 on duplicates")
    check(Q, X, 0.3, "duplicates")


def test_cell_centres_see_their_corners():
    X = lattice(5, 4)
    Q = (lattice(4, 4) + np.float32(0.5)).astype(np.float32)
    n = check(Q, X, 1.0, "cell centres, eps = 1")
    assert n == Q.shape[0] * 16
    check(Q, X, math.nextafter(1.0, 0.0), "cell centres, one ulp below")


def test_multi_batch_semi_join():
    X = make_config("c2", 15000)
    rng = np.random.default_rng(43)
    Q = (X[rng.choice(15000, 6000, replace=False)] + rng.normal(0, 0.01, (6000, 32))).astype(np.float32)
    eps = 0.11
    x = torch.from_numpy(X).cuda()
    q = torch.from_numpy(Q).cuda()
    h = ersj.build_index(x, eps)
    ersj.set_queries(h, q)
    ersj.count_pass(h)
    words = ersj.get_stats(h)["total_mask_words"]
    nb = ersj.plan_batches(h, words * 8 // 5)
    assert nb >= 4
    parts = list(ersj.iter_batches(h, nb))
    st = ersj.get_stats(h)
    assert st["n_queries"] == 6000 and st["n"] == 15000
    h.free()
    got = np.sort(keys_of(ersj.pairs_to_numpy(parts)))
    want = np.sort(keys_of(oracle.semijoin_pairs(Q, X, eps)))
    assert np.array_equal(got, want)


def test_state_rules_and_replacing_queries():
    rng = np.random.default_rng(44)
    X = rng.random((2000, 7), dtype=np.float32)
    Q1 = rng.random((300, 7), dtype=np.float32)
    Q2 = rng.random((450, 7), dtype=np.float32)
    x = torch.from_numpy(X).cuda()
    h = ersj.build_index(x, 0.3)
    ersj.set_queries(h, torch.from_numpy(Q1).cuda())
    ersj.count_pass(h)
    ersj.plan_batches(h, 0)
    # new queries discard the plan
    ersj.set_queries(h, torch.from_numpy(Q2).cuda())
    with pytest.raises(ersj.ErsjError) as e:
        ersj.fill_pass(h, 0)
    assert e.value.code == ersj.ERR_STATE
    ersj.count_pass(h)
    nb = ersj.plan_batches(h, 0)
    got = np.sort(keys_of(ersj.pairs_to_numpy(list(ersj.iter_batches(h, nb)))))
    assert np.array_equal(got, np.sort(keys_of(oracle.semijoin_pairs(Q2, X, 0.3))))
    # a rejected query set leaves the self-join
    bad = Q1.copy()
    bad[5, 3] = np.inf
    with pytest.raises(ersj.ErsjError) as e:
        ersj.set_queries(h, torch.from_numpy(bad).cuda())
    assert e.value.code == ersj.ERR_INVALID_ARG
    assert ersj.get_stats(h)["n_queries"] == 2000
    ersj.count_pass(h)
    nb = ersj.plan_batches(h, 0)
    got = np.sort(keys_of(ersj.pairs_to_numpy(list(ersj.iter_batches(h, nb)))))
    assert np.array_equal(got, np.sort(keys_of(oracle.selfjoin_pairs(X, 0.3))))
    with pytest.raises(ValueError):
        ersj.set_queries(h, torch.zeros((4, 6), dtype=torch.float32, device="cuda"))
    h.free()


def test_large_query_coordinates_choose_the_direct_kernel():
    rng = np.random.default_rng(45)
    X = rng.random((800, 6), dtype=np.float32)
    Q = rng.random((100, 6), dtype=np.float32)
    Q[7] = np.float32(1e19)
    x = torch.from_numpy(X).cuda()
    h = ersj.build_index(x, 0.4)
    assert ersj.get_stats(h)["refine_kernel"] == ersj.REFINE_MFMA16
    ersj.set_queries(h, torch.from_numpy(Q).cuda())
    assert ersj.get_stats(h)["refine_kernel"] == ersj.REFINE_DIRECT
    ersj.count_pass(h)
    nb = ersj.plan_batches(h, 0)
    got = np.sort(keys_of(ersj.pairs_to_numpy(list(ersj.iter_batches(h, nb)))))
    h.free()
    assert np.array_equal(got, np.sort(keys_of(oracle.semijoin_pairs(Q, X, 0.4))))
