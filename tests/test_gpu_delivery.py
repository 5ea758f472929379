"""Host delivery (ersj_fill_pass_host / ersj_host_sync): the pairs that land
in host memory are exactly the oracle's, over one and several batches, into
pinned and into pageable memory, with CAPACITY reported as by fill_pass."""
import numpy as np
import pytest
import torch

import exact_range_similarity_amd as ersj
import oracle
from workloads import make_config

from gpu_util import keys_of, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ersj.lib()


def host_keys(t):
    return np.sort(keys_of(t.numpy().view(np.uint32)))


@pytest.mark.parametrize("div", [0, 3, 11])
def test_delivered_pairs_equal_the_oracle(div):
    X = make_config("c2", 20000)
    eps = 0.11
    want = np.sort(keys_of(oracle.selfjoin_pairs(X, eps)))
    h = ersj.build_index(torch.from_numpy(X).cuda(), eps)
    ersj.count_pass(h)
    words = ersj.get_stats(h)["total_mask_words"]
    nb = ersj.plan_batches(h, words * 8 // div if div else 0)
    say(f"[gpu] delivery, {nb} batches")
    if div:
        assert nb >= div - 1
    got = ersj.join_to_host(h, nb)
    assert not got.is_cuda
    assert np.array_equal(host_keys(got), want)
    # one preallocated pinned buffer, batches back to back
    out = torch.empty((want.size + 10, 2), dtype=torch.int32, pin_memory=True)
    got2 = ersj.join_to_host(h, nb, out)
    assert got2.shape[0] == want.size
    assert np.array_equal(host_keys(got2), want)
    h.free()


def test_pageable_memory_and_capacity():
    rng = np.random.default_rng(51)
    X = rng.random((5000, 9), dtype=np.float32)
    eps = 0.45
    want = np.sort(keys_of(oracle.selfjoin_pairs(X, eps)))
    h = ersj.build_index(torch.from_numpy(X).cuda(), eps)
    ersj.count_pass(h)
    assert ersj.plan_batches(h, 0) == 1
    with pytest.raises(ersj.ErsjError) as e:
        ersj.fill_pass_host(h, 0, torch.empty((want.size - 1, 2), dtype=torch.int32))
    assert e.value.code == ersj.ERR_CAPACITY and e.value.required == want.size
    out = torch.empty((want.size, 2), dtype=torch.int32)  # pageable
    assert ersj.fill_pass_host(h, 0, out) == want.size
    ersj.host_sync(h)
    assert np.array_equal(host_keys(out), want)
    with pytest.raises(TypeError):
        ersj.fill_pass_host(h, 0, out.cuda())
    h.free()


def test_semi_join_delivery():
    rng = np.random.default_rng(52)
    X = rng.random((6000, 12), dtype=np.float32)
    Q = rng.random((3000, 12), dtype=np.float32)
    eps = 0.55
    want = np.sort(keys_of(oracle.semijoin_pairs(Q, X, eps)))
    h = ersj.build_index(torch.from_numpy(X).cuda(), eps)
    ersj.set_queries(h, torch.from_numpy(Q).cuda())
    ersj.count_pass(h)
    words = ersj.get_stats(h)["total_mask_words"]
    nb = ersj.plan_batches(h, words * 8 // 4)
    got = ersj.join_to_host(h, nb)
    h.free()
    assert np.array_equal(host_keys(got), want)
