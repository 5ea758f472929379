"""Exact kNN on the GPU (ersj_knn; RT-HiSS Sec. VI: growing similarity
searches) against the oracle's kNN, element by element: the same point ids in
the same order and the same binary64 D64 values.

Cases: random and clustered data over several rounds (adaptive and fixed
growth), ties (integer lattices, duplicated points), query sets distinct from
the points (cell centres, queries far outside the data), rows with more than
1024 neighbours (the radix-select path), rows cut to the bucket prefix
holding their k smallest keys, the largest k, k = n, an infinite
first radius, and both refinement kernels.
"""
import math

import numpy as np
import pytest
import torch

import exact_range_similarity_amd as ersj
import oracle
from workloads import lattice, make_config, make_queries

from gpu_util import KERNELS, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ersj.lib()


def gpu_knn(X, k, eps0, Q=None, growth=0.0, kernel=ersj.REFINE_AUTO, with_dist=True):
    xt = torch.from_numpy(np.ascontiguousarray(X)).cuda()
    qt = torch.from_numpy(np.ascontiguousarray(Q)).cuda() if Q is not None else None
    ids, dist, info = ersj.knn(xt, k, eps0, qt, growth, ersj.default_options(refine_kernel=kernel),
                               with_dist=with_dist)
    torch.cuda.synchronize()
    ids = ids.cpu().numpy().view(np.uint32)
    return ids, (dist.cpu().numpy() if dist is not None else None), info


def check(X, k, eps0, Q=None, rows=None, label="", **kw):
    for kern in kw.pop("kernels", KERNELS):
        say(f"[gpu] knn {label}: n={X.shape[0]} d={X.shape[1]} k={k} eps0={eps0!r} kernel={kern}")
        ids, dist, info = gpu_knn(X, k, eps0, Q, kernel=kern, **kw)
        say(f"[gpu]   rounds={info['rounds']} queries={info['queries']} eps={info['eps']}")
        sel = np.arange(ids.shape[0]) if rows is None else np.asarray(rows)
        if Q is None:
            want_ids, want_d = oracle.knn(X, k, sel)
        else:
            want_ids, want_d = oracle.knn_rows(Q, X, k, sel)
        bad = np.nonzero(~np.all(ids[sel] == want_ids, axis=1))[0]
        assert bad.size == 0, f"{label} kernel={kern}: rows {sel[bad[:5]]} differ: " \
                              f"{ids[sel[bad[0]]][:8]} vs {want_ids[bad[0]][:8]}"
        if dist is not None:
            assert np.array_equal(dist[sel], want_d), f"{label} kernel={kern}: D64 differs"
        assert info["queries"][0] == ids.shape[0]
        assert all(a >= b for a, b in zip(info["queries"], info["queries"][1:]))
    return info


@pytest.mark.parametrize("n,d,k", [(3001, 5, 1), (3001, 5, 7), (2500, 12, 64), (700, 40, 33), (900, 100, 20)])
def test_random_adaptive(n, d, k):
    rng = np.random.default_rng(n + d + k)
    X = rng.random((n, d), dtype=np.float32)
    info = check(X, k, 0.01, label="random")
    if k > 1:
        assert info["rounds"] >= 2  # a small first radius needs growth


@pytest.mark.parametrize("name,n,k", [("c2", 20000, 64), ("c4", 30011, 16), ("c3", 8000, 32)])
def test_clustered_workloads(name, n, k):
    X = make_config(name, n)
    eps = None
    for kc in (k, k + 1, k + 3):  # a tie at the calibration point: try the next count
        try:
            eps, _, _ = oracle.calibrate_eps(X, min(1000, n), kc)
            break
        except RuntimeError:
            continue
    assert eps is not None
    rows = np.random.default_rng(7).choice(n, 400, replace=False)
    check(X, k, eps, rows=rows, label=f"{name}")
    check(X, k, eps * 0.5, rows=rows, label=f"{name} fixed growth", growth=1.3,
          kernels=(ersj.REFINE_MFMA,))


@pytest.mark.parametrize("m,d,k", [(7, 2, 9), (6, 3, 27), (5, 4, 40)])
def test_lattice_ties(m, d, k):
    X = lattice(m, d)
    for eps0 in (1.0, 0.3, 2.5):
        check(X, k, eps0, label=f"lattice m={m} d={d}")


def test_duplicates():
    rng = np.random.default_rng(71)
    base = rng.random((500, 4), dtype=np.float32)
    X = np.concatenate([base, base, base])
    check(X, 5, 0.05, label="duplicates")


def test_query_sets():
    X = lattice(5, 3)
    Q = (lattice(4, 3) + np.float32(0.5)).astype(np.float32)
    check(X, 8, 0.9, Q=Q, label="cell centres")
    rng = np.random.default_rng(72)
    P = rng.random((2000, 6), dtype=np.float32)
    far = (rng.random((300, 6), dtype=np.float32) * 40 - 20).astype(np.float32)
    info = check(P, 10, 0.02, Q=far, label="far queries")
    assert info["rounds"] >= 3
    Xc = make_config("c2", 15000)
    Qc = make_queries("c2", 3000, 9, 15000)
    check(Xc, 20, 0.1, Q=Qc, rows=np.arange(0, 3000, 7), label="c2 queries")


def test_more_than_1024_neighbours_and_limits():
    rng = np.random.default_rng(73)
    X = rng.random((5000, 3), dtype=np.float32)
    # a first radius holding thousands of neighbours per query: radix path
    check(X, 10, 0.5, rows=np.arange(0, 5000, 11), label="radix path")
    check(X, 1024, 0.05, rows=np.arange(0, 5000, 97), label="k = 1024")
    Y = rng.random((200, 7), dtype=np.float32)
    check(Y, 200, 0.1, label="k = n")
    info = check(Y, 17, math.inf, label="infinite radius")
    assert info["rounds"] == 1
    ids, dist, _ = gpu_knn(Y, 17, 0.2, with_dist=False)
    assert dist is None and np.array_equal(ids, oracle.knn(Y, 17)[0])


def test_large_rows_through_each_narrowing_level():
    # 1-D uniform points: about 40,000 neighbours per query, a sixteenth of
    # them in the first value bucket, so the bucket is split once more
    rng = np.random.default_rng(74)
    X = rng.random((200000, 1), dtype=np.float32)
    check(X, 10, 0.1, rows=np.arange(0, 200000, 4001), label="sub-buckets",
          kernels=(ersj.REFINE_MFMA,))
    # 3,000 copies of one point: every bucket holds them all (D64 = 0), so the
    # exact radix select over (D64, id) decides, ranking the copies by id
    Y = np.concatenate([rng.random((500, 3), dtype=np.float32),
                        np.repeat(np.float32([[0.5, 0.5, 0.5]]), 3000, axis=0)])
    check(Y, 700, 0.2, rows=np.arange(0, 3500, 53), label="tied bucket")


def test_rows_cut_to_their_bucket_prefix_before_the_sort():
    # uniform 3-D points: a first radius giving each row a few hundred
    # neighbours, more than 2k of them but at most the 1024 keys a wave
    # holds, so the keys are cut to the value-bucket prefix holding the k
    # smallest before the sort (58%, 86% and 67% of the sampled rows)
    rng = np.random.default_rng(75)
    X = rng.random((20000, 3), dtype=np.float32)
    check(X, 100, 0.14, rows=np.arange(0, 20000, 37), label="cut, k = 100")
    check(X, 150, 0.19, rows=np.arange(0, 20000, 41), label="cut, k = 150")
    check(X, 128, 0.16, rows=np.arange(0, 20000, 43), label="cut, k = 128")


def test_bad_arguments_raise():
    x = torch.zeros((10, 3), dtype=torch.float32, device="cuda")
    for k, eps0, growth in ((0, 1.0, 0.0), (11, 1.0, 0.0), (3, 0.0, 0.0), (3, float("nan"), 0.0),
                            (3, 1.0, 1.0), (3, 1.0, float("inf"))):
        with pytest.raises(ersj.ErsjError):
            ersj.knn(x, k, eps0, growth=growth)
    bad = x.clone()
    bad[2, 1] = float("nan")
    with pytest.raises(ersj.ErsjError):
        ersj.knn(bad, 2, 1.0)
