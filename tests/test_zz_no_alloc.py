"""ersj_fill_pass_noalloc (the fill pass whose working memory is the
library's fixed device scratch) against ersj_fill_pass, through the C ABI.

Two joins in a row, the second on a smaller input, each cut into several
batches: every batch's pairs from the allocation-free call must equal, as a
set, those of the ordinary call (and the union the oracle's self-join, which
is the result defined by "RT-HiSS: Ray Tracing Accelerated High Dimensional
Vector Similarity Searches", Sec. II-A).  The scratch keeps the previous
call's contents, so the second, smaller join also checks that nothing stale
leaks into a result.  A batch too large for the scratch is refused before
any device work.
"""
import ctypes
import json
import os

import numpy as np
import pytest
import torch

import exact_range_similarity_amd as ersj
import oracle
from workloads import make_config

from gpu_util import keys_of, say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ersj.lib()


def c_fill(fn, h, b, out, cap):
    n = ctypes.c_uint64()
    ptr = ctypes.c_void_p(out.data_ptr()) if out is not None else None
    rc = fn(h.handle, b, ptr, cap, ctypes.byref(n), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc, n.value


def join_both(X, eps, budget, kernel):
    L = ersj.lib()
    xt = torch.from_numpy(X).cuda()
    h = ersj.build_index(xt, eps, ersj.default_options(refine_kernel=kernel))
    try:
        ersj.count_pass(h)
        nb = ersj.plan_batches(h, budget)
        say(f"[noalloc] n={X.shape[0]} kernel={kernel} budget={budget} batches={nb}")
        got_all = []
        for b in range(nb):
            rc, m = c_fill(L.ersj_fill_pass, h, b, None, 0)
            assert rc in (ersj.OK, ersj.ERR_CAPACITY)
            want = torch.empty((max(m, 1), 2), dtype=torch.int32, device="cuda")
            rc, m1 = c_fill(L.ersj_fill_pass, h, b, want, m)
            assert rc == ersj.OK and m1 == m
            # the allocation-free call: first without room (CAPACITY, count),
            # then into an output with room to spare
            rc, m2 = c_fill(L.ersj_fill_pass_noalloc, h, b, None, 0)
            assert rc == (ersj.ERR_CAPACITY if m else ersj.OK) and m2 == m
            got = torch.full((m + 7, 2), -1, dtype=torch.int32, device="cuda")
            rc, m3 = c_fill(L.ersj_fill_pass_noalloc, h, b, got, m + 7)
            assert rc == ersj.OK, L.ersj_last_error()
            assert m3 == m
            torch.cuda.synchronize()
            g = got[:m].cpu().numpy().view(np.uint32)
            w = want[:m].cpu().numpy().view(np.uint32)
            assert np.array_equal(np.sort(keys_of(g)), np.sort(keys_of(w))), f"batch {b} differs"
            assert (got[m:].cpu().numpy() == -1).all(), "wrote past the pair count"
            got_all.append(g)
        return nb, np.concatenate(got_all)
    finally:
        h.free()


def c1_eps():
    with open(os.path.join(GOLDEN, "eps_configs.json")) as f:
        return float.fromhex(json.load(f)["c1"]["eps"])


@pytest.mark.parametrize("kernel", [ersj.REFINE_AUTO, ersj.REFINE_DIRECT])
def test_noalloc_matches_fill_pass_twice(kernel):
    eps = c1_eps()
    for n, budget in ((12000, 6 << 20), (4000, 1 << 20)):
        X = make_config("c1", n)
        nb, got = join_both(X, eps, budget, kernel)
        assert nb >= 2
        want = oracle.selfjoin_pairs(X, eps)
        assert np.array_equal(np.sort(keys_of(got)), np.sort(keys_of(want)))


def test_noalloc_refuses_a_batch_larger_than_the_scratch():
    X = make_config("c1", 30000)
    xt = torch.from_numpy(X).cuda()
    h = ersj.build_index(xt, float("inf"))
    try:
        ersj.count_pass(h)
        assert ersj.plan_batches(h, 0) == 1  # 30000^2 bits: 112 MB of mask
        say("[noalloc] oversized batch")
        rc, _ = c_fill(ersj.lib().ersj_fill_pass_noalloc, h, 0, None, 0)
        assert rc == ersj.ERR_SCRATCH
        assert b"fixed scratch" in ersj.lib().ersj_last_error()
    finally:
        h.free()
