"""Device memory limits and the library's reuse pool.

* max_device_bytes: a cap below what a step needs fails with ERSJ_ERR_OOM
  at the allocation that crosses it (ERSJ_ERR_BUDGET from the planner when
  no mask word fits), any cap that suffices gives the oracle's pair set
  within the cap, and a cap that the index and count pass fit under makes
  the planner split the join into batches that fit the rest.
* ersj_release_cached: blocks the library keeps after ersj_free go back to
  the HIP runtime, where torch's allocator sees them.

The result is the self-join of "RT-HiSS: Ray Tracing Accelerated High
Dimensional Vector Similarity Searches", Sec. II-A."""
import numpy as np
import pytest
import torch

import exact_range_similarity_amd as ersj
import oracle

from gpu_util import assert_same_pairs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ersj.lib()


def data(n=20000, d=24, seed=5):
    rng = np.random.default_rng(seed)
    X = rng.random((n, d), dtype=np.float32)
    eps, _, _ = oracle.calibrate_eps(X, 500, 48)
    return X, eps


def held_after(stage, X, eps):
    """Device bytes the handle holds after build (stage 0) or the count pass (1)."""
    h = ersj.build_index(torch.from_numpy(X).cuda(), eps)
    if stage == 1:
        ersj.count_pass(h)
    b = ersj.get_stats(h)["device_bytes"]
    h.free()
    return b


def test_cap_below_the_index_fails_with_oom_at_build():
    X, eps = data()
    say(f"[gpu] max_device_bytes at build: n={X.shape[0]} d={X.shape[1]}")
    need = held_after(0, X, eps)
    for cap in (1, 4096, need // 2):
        with pytest.raises(ersj.ErsjError) as e:
            ersj.build_index(torch.from_numpy(X).cuda(), eps, ersj.default_options(max_device_bytes=cap))
        assert e.value.code == ersj.ERR_OOM
        assert "max_device_bytes" in str(e.value)


def capped_join(X, eps, cap):
    """(stage reached, error code or None, pairs, batches, device bytes held)."""
    stage, parts, nb, held = "build", None, 0, 0
    h = None
    try:
        h = ersj.build_index(torch.from_numpy(X).cuda(), eps, ersj.default_options(max_device_bytes=cap))
        stage = "count"
        ersj.count_pass(h)
        stage = "plan"
        nb = ersj.plan_batches(h)
        stage = "fill"
        parts = list(ersj.iter_batches(h, nb))
        torch.cuda.synchronize()
        held = ersj.get_stats(h)["device_bytes"]
        return "done", None, parts, nb, held
    except ersj.ErsjError as e:
        return stage, e.code, None, nb, held
    finally:
        if h is not None:
            h.free()


def test_cap_sweep_fails_cleanly_or_joins_exactly():
    # every cap from far too small to ample: the join either completes with
    # the oracle's pairs inside the cap, or stops with OOM (BUDGET when the
    # planner finds no room for a mask word) at the step that needed more
    X, eps = data()
    want = oracle.selfjoin_pairs(X, eps)
    full = held_after(1, X, eps)
    seen = set()
    for cap in [1 << 16] + [int(full * f) for f in (0.5, 0.9, 1.0, 1.05, 1.2, 1.5, 2.0, 3.0, 5.0, 9.0, 17.0)]:
        stage, code, parts, nb, held = capped_join(X, eps, cap)
        say(f"[gpu] cap {cap}: {stage} {code} batches={nb} held={held}")
        seen.add(stage)
        if stage != "done":
            assert code in (ersj.ERR_OOM, ersj.ERR_BUDGET), (cap, stage, code)
            assert code == ersj.ERR_OOM or stage == "plan"
            # a plan made under the cap fits it (the band list of this data
            # never has to grow)
            assert stage != "fill", (cap, stage, code)
            continue
        assert held <= cap
        assert_same_pairs(X, eps, ersj.pairs_to_numpy(parts), want, f"cap {cap}")
    assert "build" in seen and "done" in seen, seen


def test_cap_splits_the_join_into_batches_with_the_same_pairs():
    X, eps = data()
    b1 = held_after(1, X, eps)
    h = ersj.build_index(torch.from_numpy(X).cuda(), eps)
    ersj.count_pass(h)
    mask_bytes = ersj.get_stats(h)["total_mask_words"] * 8
    h.free()
    # beside the index: the per-batch reserve (row arrays, counters, a band
    # list of at most 2^20 16-byte entries, pool rounding) and a third of the
    # mask
    reserve = X.shape[0] * 24 + (1 << 20) * 16 + (10 << 20)
    cap = b1 + reserve + mask_bytes // 3
    opts = ersj.default_options(max_device_bytes=cap)
    h = ersj.build_index(torch.from_numpy(X).cuda(), eps, opts)
    try:
        ersj.count_pass(h)
        nb = ersj.plan_batches(h)
        say(f"[gpu] cap {cap} bytes (mask {mask_bytes}): {nb} batches")
        assert nb >= 2
        parts = list(ersj.iter_batches(h, nb))
        torch.cuda.synchronize()
        assert ersj.get_stats(h)["device_bytes"] <= cap
    finally:
        h.free()
    assert_same_pairs(X, eps, ersj.pairs_to_numpy(parts), oracle.selfjoin_pairs(X, eps), "capped join")


def test_release_cached_returns_pool_blocks_to_the_runtime():
    ersj.release_cached()
    for n, d in ((30000, 16), (12000, 40)):
        X, eps = data(n, d, seed=n)
        parts = ersj.self_join(torch.from_numpy(X).cuda(), eps)
        torch.cuda.synchronize()
        del parts
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free0 = torch.cuda.mem_get_info()[0]
    got = ersj.release_cached()
    free1 = torch.cuda.mem_get_info()[0]
    say(f"[gpu] release_cached: {got} bytes, runtime free {free0} -> {free1}")
    assert got > 0
    assert free1 - free0 >= got // 2
    assert ersj.release_cached() == 0
    assert ersj.release_cached(torch.cuda.current_device()) == 0
