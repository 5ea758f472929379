"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (default options; the d=64 workload with a budget that forces at
least four memory-limited batches).

The oracle cannot join these in seconds, so parity is checked on sampled
rows (each row's neighbour list equal to the oracle's, computed row by
row) and on properties that hold at any size: rows 0..999 carry exactly
the neighbour count epsilon was calibrated for, every point pairs with
itself, no pair is duplicated, and the pair multiset is symmetric.
"""
import json
import os

import numpy as np
import pytest
import torch

import exact_range_similarity_amd as ersj
import oracle
from workloads import CONFIGS, make_config, x_digest

from gpu_util import say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CHUNK = 1 << 27


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ersj.lib()


def u32(t):
    return t.to(torch.int64) & 0xffffffff


def chunks(parts):
    for p in parts:
        for s in range(0, p.shape[0], CHUNK):
            blk = p[s:s + CHUNK]
            yield u32(blk[:, 0]), u32(blk[:, 1])


def sym_hash(parts):
    """Two asymmetric pair hashes summed over the set and over its transpose."""
    C = [(0x5bd1e995, 0x1b873593, 0x2545f491), (0x27d4eb2f, 0x165667b1, 0x61c88647)]
    fwd = [0, 0]
    rev = [0, 0]
    for q, x in chunks(parts):
        for k, (a, b, c) in enumerate(C):
            m = (1 << 30) - 1
            fwd[k] += int((((q * a) ^ (x * b + c)) & m).sum())
            rev[k] += int((((x * a) ^ (q * b + c)) & m).sum())
    return fwd, rev


def rows_of(parts, rows):
    R = torch.as_tensor(np.asarray(rows, dtype=np.int64), device="cuda")
    got = {int(r): [] for r in rows}
    for q, x in chunks(parts):
        sel = torch.isin(q, R)
        if sel.any():
            for a, b in zip(q[sel].tolist(), x[sel].tolist()):
                got[a].append(b)
    return {r: sorted(v) for r, v in got.items()}


def run_full(name, budget_div=0.0):
    with open(os.path.join(GOLDEN, "eps_configs.json")) as f:
        rec = json.load(f)[name]
    spec = CONFIGS[name]
    X = make_config(name)
    assert x_digest(X) == rec["x_sha256"]
    eps = float.fromhex(rec["eps"])
    say(f"[gpu-full] {name}: n={X.shape[0]} d={X.shape[1]} eps={eps!r} budget_div={budget_div}")
    xt = torch.from_numpy(X).cuda()
    h = ersj.build_index(xt, eps)
    ersj.count_pass(h)
    st0 = ersj.get_stats(h)
    budget = int(st0["total_mask_words"] * 8 / budget_div) if budget_div else 0
    nb = ersj.plan_batches(h, budget)
    parts = list(ersj.iter_batches(h, nb))
    torch.cuda.synchronize()
    st = ersj.get_stats(h)
    h.free()
    del xt
    total = sum(p.shape[0] for p in parts)
    say(f"[gpu-full] {name}: batches={nb} cells={st['cells']} candidates={st['total_candidates']} "
        f"pairs={total}")
    return X, eps, rec, spec, parts, nb, total


def check_common(name, X, eps, rec, spec, parts, total, n_sample=48, symmetric=True):
    n = X.shape[0]
    # calibration identity over rows 0..nq-1
    nq = rec["nq"]
    cnt = 0
    self_pairs = 0
    for q, x in chunks(parts):
        cnt += int((q < nq).sum())
        self_pairs += int((q == x).sum())
    assert cnt == nq * (spec.k + 1), (cnt, nq * (spec.k + 1))
    assert self_pairs == n
    # sampled rows against the oracle, row by row
    rng = np.random.default_rng(1234)
    rows = np.unique(np.concatenate([np.arange(16), rng.integers(0, n, n_sample)]))
    got = rows_of(parts, rows)
    colptr, cols = oracle.join_rows(X, eps, rows)
    for r_i, r in enumerate(rows):
        want = cols[colptr[r_i]:colptr[r_i + 1]].tolist()
        assert got[int(r)] == want, f"{name}: row {r} differs ({len(got[int(r)])} vs {len(want)})"
    if symmetric:
        fwd, rev = sym_hash(parts)
        assert fwd == rev, f"{name}: pair set is not symmetric"


def check_unique(parts):
    keys = torch.cat([(q << 32) | x for q, x in chunks(parts)])
    s = torch.sort(keys).values
    assert bool((s[1:] != s[:-1]).all())


def test_full_c2():
    X, eps, rec, spec, parts, nb, total = run_full("c2")
    check_common("c2", X, eps, rec, spec, parts, total)
    check_unique(parts)


def test_full_c3_four_plus_batches():
    X, eps, rec, spec, parts, nb, total = run_full("c3", budget_div=4.5)
    assert nb >= 4
    check_common("c3", X, eps, rec, spec, parts, total, n_sample=32)
    check_unique(parts)


def test_full_c4():
    X, eps, rec, spec, parts, nb, total = run_full("c4")
    check_common("c4", X, eps, rec, spec, parts, total, n_sample=32)


def test_full_c5():
    X, eps, rec, spec, parts, nb, total = run_full("c5")
    check_common("c5", X, eps, rec, spec, parts, total, n_sample=24)
    check_unique(parts)
