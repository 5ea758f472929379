"""The GPU tests' torch fingerprint code (tests/digest_util.py), run on CPU
tensors, against the numpy code that writes the oracle's digest files and
the oracle's own mix64: the device-side comparison of full-size results
rests on these agreeing bit for bit."""
import os
import sys

import numpy as np
import torch

import oracle
from digest_util import block_fold, mix64, row_digests

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import make_digests  # noqa: E402


def test_mix64_torch_matches_numpy_and_oracle():
    rng = np.random.default_rng(7)
    v = rng.integers(0, 2 ** 63, 4096, dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, 4096, dtype=np.uint64)
    with np.errstate(over="ignore"):
        want = make_digests.mix64_np(v)
    got = mix64(torch.from_numpy(v.view(np.int64))).numpy().view(np.uint64)
    assert np.array_equal(got, want)
    for j in (0, 1, 2 ** 32 - 1, int(v[5])):
        assert oracle.mix64(j) == int(make_digests.mix64_np(np.array([j], dtype=np.uint64))[0])


def test_row_digests_and_fold_match_the_digest_files_code():
    rng = np.random.default_rng(8)
    n = 1000
    q = rng.integers(0, n, 20000).astype(np.uint32)
    x = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    P = np.stack([q, x], axis=1).view(np.int32)
    parts = [torch.from_numpy(P[:7000].copy()), torch.from_numpy(P[7000:].copy())]
    cnt, dig = row_digests(parts, n, chunk=3000)
    want_c = np.bincount(q, minlength=n)
    with np.errstate(over="ignore"):
        mx = make_digests.mix64_np(x.astype(np.uint64))
        want_h = np.zeros(n, dtype=np.uint64)
        np.add.at(want_h, q, mx)
    assert np.array_equal(cnt.numpy(), want_c)
    assert np.array_equal(dig.numpy().view(np.uint64), want_h)
    bc, fp = block_fold(cnt, dig, 64)
    wbc, wfp, _ = make_digests.block_fold(want_c.astype(np.uint32), want_h, np.zeros(n, dtype=np.uint32))
    assert np.array_equal(bc.numpy().astype(np.uint64), wbc)
    assert np.array_equal(fp.numpy().view(np.uint64), wfp)
    rows = torch.tensor([5, 999, 0, 17], dtype=torch.int64)
    c2, d2 = row_digests(parts, n, rows=rows)
    assert np.array_equal(c2.numpy(), want_c[[5, 999, 0, 17]])
    assert np.array_equal(d2.numpy().view(np.uint64), want_h[[5, 999, 0, 17]])
