"""Parity of the HIP path with the CPU oracle: identical pair sets.

Sizes here let the oracle finish in seconds while still spanning many row
tiles (32 rows), candidate chunks (256) and segments, with ragged tails.
The bar is bit-exact: the set of (query id, point id) pairs must equal the
oracle's, with no duplicates.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import exact_range_similarity_amd as ersj
import oracle
from workloads import CONFIGS, fig3_points, fig5_points, lattice, make_config

from gpu_util import KERNELS, assert_same_pairs, check_against_oracle, gpu_pairs, keys_of, say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ersj.lib()


def eps_table():
    with open(os.path.join(GOLDEN, "eps_configs.json")) as f:
        return json.load(f)


def test_c1_full_config():
    rec = eps_table()["c1"]
    X = make_config("c1")
    check_against_oracle(X, float.fromhex(rec["eps"]), "c1 full")


@pytest.mark.parametrize("name,n", [("c2", 24000), ("c3", 12000), ("c4", 30011), ("c5", 6000)])
def test_reduced_config_shapes(name, n):
    X = make_config(name, n)
    eps, _, _ = oracle.calibrate_eps(X, min(1000, n), CONFIGS[name].k)
    check_against_oracle(X, eps, f"{name} n={n}")


@pytest.mark.parametrize("n,d", [(1, 1), (1, 7), (2, 2), (33, 3), (257, 5), (1000, 1), (777, 2),
                                 (513, 17), (300, 384)])
def test_small_and_ragged(n, d):
    rng = np.random.default_rng(n * 1000 + d)
    X = rng.random((n, d), dtype=np.float32)
    for eps in (0.05, 0.3, 1.1):
        check_against_oracle(X, eps, f"random n={n} d={d}")


def test_345():
    X = np.array([[0, 0], [3, 4]], dtype=np.float32)
    check_against_oracle(X, 5.0, "3-4-5 at eps")
    check_against_oracle(X, math.nextafter(5.0, 0.0), "3-4-5 below eps")


@pytest.mark.parametrize("m,d", [(12, 2), (6, 3), (4, 5), (40, 1)])
def test_lattice_exact_boundaries(m, d):
    X = lattice(m, d)
    for eps in (1.0, math.nextafter(1.0, 0.0), math.sqrt(2.0), math.sqrt(3.0), 2.0):
        check_against_oracle(X, eps, f"lattice m={m} d={d}")


def test_scaled_lattice_inexact_squares():
    X = lattice(7, 3, spacing=0.1)
    for eps in (0.1, math.nextafter(0.1, 1), math.nextafter(0.1, 0), 0.1 * math.sqrt(2)):
        check_against_oracle(X, eps, "lattice spacing 0.1")


def test_eps_zero_duplicates_and_identical_points():
    rng = np.random.default_rng(5)
    base = rng.random((50, 6), dtype=np.float32)
    X = np.repeat(base, rng.integers(1, 8, 50), axis=0)
    X = X[rng.permutation(X.shape[0])]
    check_against_oracle(X, 0.0, "eps=0 duplicates")
    same = np.full((300, 4), 0.25, dtype=np.float32)
    check_against_oracle(same, 0.0, "identical points eps=0")
    check_against_oracle(same, 1e-3, "identical points")


def test_eps_infinite_and_huge():
    rng = np.random.default_rng(6)
    X = rng.random((700, 9), dtype=np.float32)
    for k in KERNELS:
        got = gpu_pairs(X, math.inf, options=ersj.default_options(refine_kernel=k))
        assert got.shape[0] == 700 * 700
    check_against_oracle(X, 1e30, "eps huge")
    check_against_oracle(X, 1e-30, "eps tiny")


def test_wide_value_ranges():
    rng = np.random.default_rng(7)
    for scale in (1e-20, 1e15):
        X = (rng.standard_normal((900, 10)) * scale).astype(np.float32)
        eps = 0.6 * scale * math.sqrt(10)
        check_against_oracle(X, eps, f"scale {scale}")


def test_strided_rows():
    rng = np.random.default_rng(8)
    X = rng.random((1500, 13), dtype=np.float32)
    check_against_oracle(X, 0.45, "ld=16", ld=16)


def test_fig3_structure():
    with open(os.path.join(GOLDEN, "fig3_pairs.json")) as f:
        g = json.load(f)
    got = gpu_pairs(fig3_points(), g["eps"])
    want = {tuple(p) for p in g["pairs"]} | {(i, i) for i in range(7)}
    want |= {(j, i) for (i, j) in want}
    assert set(map(tuple, got.astype(np.int64).tolist())) == want


def test_fig5_compaction():
    with open(os.path.join(GOLDEN, "fig5_compaction.json")) as f:
        g = json.load(f)
    got = gpu_pairs(fig5_points(), 1.0)
    row = sorted(int(j) for i, j in got.tolist() if i == g["query"])
    assert row == g["compressed"]


def test_large_d_and_offset_data():
    rng = np.random.default_rng(12)
    X = (rng.random((700, 700)) + 5.0).astype(np.float32)
    check_against_oracle(X, 10.5, "d=700 offset")
    # at d = 2000 the fp32 MFMA form's query tile exceeds the LDS; the split
    # form runs on operands prepared per point and is the automatic choice
    Z = (rng.random((300, 2000)) + 5.0).astype(np.float32)
    check_against_oracle(Z, 17.0, "d=2000 offset", kernels=(ersj.REFINE_DIRECT, ersj.REFINE_MFMA16))
    h = ersj.build_index(torch.from_numpy(Z).cuda(), 17.0)
    assert ersj.get_stats(h)["refine_kernel"] == ersj.REFINE_MFMA16
    h.free()
    with pytest.raises(ersj.ErsjError) as e:
        ersj.build_index(torch.from_numpy(Z).cuda(), 17.0, ersj.default_options(refine_kernel=ersj.REFINE_MFMA))
    assert e.value.code == ersj.ERR_INVALID_ARG
    Y = (rng.standard_normal((2000, 40)) * 0.01 + 100.0).astype(np.float32)
    check_against_oracle(Y, 0.085, "offset cluster")


def test_multi_batch_equals_single_batch():
    X = make_config("c2", 20000)
    eps, _, _ = oracle.calibrate_eps(X, 1000, 64)
    xt = torch.from_numpy(X).cuda()
    h = ersj.build_index(xt, eps)
    ersj.count_pass(h)
    st = ersj.get_stats(h)
    words = st["total_mask_words"]
    parts_by_budget = {}
    for budget in (0, words * 8 // 5, words * 8 // 17):
        nb = ersj.plan_batches(h, budget)
        say(f"[gpu] multi-batch budget={budget} batches={nb}")
        if budget:
            assert nb >= 4
        rows = []
        for b in range(nb):
            r0, nr, mw = ersj.batch_info(h, b)
            rows.append((r0, nr))
            if budget:
                assert mw * 8 <= budget
        assert rows[0][0] == 0 and sum(r[1] for r in rows) == X.shape[0]
        assert all(rows[i][0] + rows[i][1] == rows[i + 1][0] for i in range(nb - 1))
        parts = list(ersj.iter_batches(h, nb))
        parts_by_budget[budget] = np.sort(keys_of(ersj.pairs_to_numpy(parts)))
    h.free()
    ref = parts_by_budget[0]
    for b, k in parts_by_budget.items():
        assert np.array_equal(k, ref), b
    want = oracle.selfjoin_pairs(X, eps)
    assert np.array_equal(ref, np.sort(keys_of(want)))


def test_pairs_buffer_aligned_to_four_bytes_only():
    # the output starts one int32 into its allocation: pairs are stored as
    # two 4-byte words instead of one 8-byte word; the word before the
    # output and the one after it stay untouched
    X = make_config("c2", 6000)
    eps, _, _ = oracle.calibrate_eps(X, 600, 64)
    xt = torch.from_numpy(X).cuda()
    h = ersj.build_index(xt, eps)
    try:
        ersj.count_pass(h)
        nb = ersj.plan_batches(h, 0)
        assert nb == 1
        try:
            m = ersj.fill_pass(h, 0, None, 0)
        except ersj.ErsjError as e:
            m = e.required
        buf = torch.full((2 * m + 2,), -7, dtype=torch.int32, device="cuda")
        view = buf[1:2 * m + 1]
        assert view.data_ptr() % 8 == 4
        assert ersj.fill_pass(h, 0, view, m) == m
        torch.cuda.synchronize()
        out = buf.cpu().numpy()
    finally:
        h.free()
    assert out[0] == -7 and out[-1] == -7
    got = out[1:-1].view(np.uint32).reshape(m, 2)
    say(f"[gpu] 4-byte aligned output: {m} pairs")
    assert_same_pairs(X, eps, got, oracle.selfjoin_pairs(X, eps), "4-byte aligned output")


def test_capacity_and_budget_errors():
    rng = np.random.default_rng(9)
    X = rng.random((4000, 8), dtype=np.float32)
    xt = torch.from_numpy(X).cuda()
    h = ersj.build_index(xt, 0.4)
    ersj.count_pass(h)
    with pytest.raises(ersj.ErsjError) as e:
        ersj.plan_batches(h, 64)
    assert e.value.code == ersj.ERR_BUDGET
    with pytest.raises(ersj.ErsjError) as e:
        ersj.fill_pass(h, 0)
    assert e.value.code == ersj.ERR_STATE
    nb = ersj.plan_batches(h, 0)
    assert nb == 1
    with pytest.raises(ersj.ErsjError) as e:
        ersj.fill_pass(h, 0, None, 0)
    assert e.value.code == ersj.ERR_CAPACITY
    need = e.value.required
    small = torch.empty((need - 1, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(ersj.ErsjError) as e:
        ersj.fill_pass(h, 0, small)
    assert e.value.code == ersj.ERR_CAPACITY and e.value.required == need
    out = torch.empty((need, 2), dtype=torch.int32, device="cuda")
    assert ersj.fill_pass(h, 0, out) == need
    with pytest.raises(ersj.ErsjError) as e:
        ersj.fill_pass(h, 1, out)
    assert e.value.code == ersj.ERR_INVALID_ARG
    got = ersj.pairs_to_numpy([out])
    h.free()
    assert_same_pairs(X, 0.4, got, oracle.selfjoin_pairs(X, 0.4), "capacity retry")


def test_non_finite_input_rejected():
    X = np.random.default_rng(10).random((500, 4), dtype=np.float32)
    X[123, 2] = np.nan
    with pytest.raises(ersj.ErsjError) as e:
        ersj.build_index(torch.from_numpy(X).cuda(), 0.1)
    assert e.value.code == ersj.ERR_INVALID_ARG
    X[123, 2] = np.inf
    with pytest.raises(ersj.ErsjError) as e:
        ersj.build_index(torch.from_numpy(X).cuda(), 0.1)
    assert e.value.code == ersj.ERR_INVALID_ARG


@pytest.mark.parametrize("kernel", KERNELS)
def test_boundary_list_overflow_regrows(kernel):
    X = lattice(9, 3)
    opts = ersj.default_options(boundary_capacity=16, refine_kernel=kernel)
    say(f"[gpu] lattice with a 16-entry boundary list, kernel={kernel}")
    got = gpu_pairs(X, 1.0, options=opts)
    assert_same_pairs(X, 1.0, got, oracle.selfjoin_pairs(X, 1.0), "blist regrow")


def test_kernel_choice():
    rng = np.random.default_rng(11)
    X = rng.random((500, 6), dtype=np.float32)
    xt = torch.from_numpy(X).cuda()
    for k in (ersj.REFINE_AUTO,) + KERNELS:
        h = ersj.build_index(xt, 0.3, ersj.default_options(refine_kernel=k))
        used = ersj.get_stats(h)["refine_kernel"]
        h.free()
        assert used == (ersj.REFINE_MFMA16 if k == ersj.REFINE_AUTO else k)
    big = (X * 1e18).astype(np.float32)
    for k in (ersj.REFINE_MFMA, ersj.REFINE_MFMA16):
        with pytest.raises(ersj.ErsjError) as e:
            ersj.build_index(torch.from_numpy(big).cuda(), 1e18, ersj.default_options(refine_kernel=k))
        assert e.value.code == ersj.ERR_INVALID_ARG
    h = ersj.build_index(torch.from_numpy(big).cuda(), 1e18)
    assert ersj.get_stats(h)["refine_kernel"] == ersj.REFINE_DIRECT
    h.free()


def test_deterministic_output_order():
    X = make_config("c4", 20000)
    a = gpu_pairs(X, 0.05)
    b = gpu_pairs(X, 0.05)
    assert np.array_equal(a, b)


def test_stats_are_consistent():
    X = make_config("c2", 10000)
    xt = torch.from_numpy(X).cuda()
    opts = ersj.default_options(timing=1)
    parts, h = ersj.self_join(xt, 0.11, options=opts, return_index=True)
    st = ersj.get_stats(h)
    h.free()
    total = sum(p.shape[0] for p in parts)
    assert st["n"] == 10000 and st["d"] == 32
    assert st["n_batches"] == 1 and st["last_batch_pairs"] == total
    assert st["last_batch_candidates"] == st["total_candidates"]
    assert st["total_candidates"] >= total
    assert st["refine_launches"] >= 1 and st["refine_ms"] > 0
    assert sorted(st["index_dims"]) == sorted(set(st["index_dims"]))
    # counters summed over their per-workgroup slots
    assert 0 <= st["last_recheck_in"] <= st["last_boundary_pairs"]
    assert 0 <= st["last_skipped"] <= st["last_batch_candidates"]
    assert st["skipped_candidates"] == st["last_skipped"]  # one batch
