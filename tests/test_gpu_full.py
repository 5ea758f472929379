"""Full-size workloads on the GPU, in the launch configuration the benchmark
times (default options; the d=64 workload with a budget that forces at
least four memory-limited batches), compared with the oracle's stored
neighbour fingerprints (tests/golden/make_digests.py, oracle only).

The result is the self-join of "RT-HiSS: Ray Tracing Accelerated High
Dimensional Vector Similarity Searches", Sec. II-A.  Per query row the GPU
pairs give a count and a fingerprint (sum of mix64 of the neighbour ids,
tests/digest_util.py), equal to the oracle's exactly when the row's
neighbour list is (up to a 2^-64 chance):

* d=16 and d=32 workloads: every one of their 20,000 and 10^6 rows,
  compared through per-block folds of 64 rows (a differing block is diffed
  row by row against the oracle, so a failure names the rows and pairs);
* the others: the stored sample (rows 0..999, 10,000 seeded rows, every row
  of the largest cluster, and for the background mixture 2,000 background
  rows), row by row.

Properties that hold at any size are checked as well: rows 0..999 carry
exactly the neighbour count epsilon was calibrated for, every point pairs
with itself, no pair is duplicated, and the pair multiset is symmetric.
"""
import json
import os

import numpy as np
import pytest
import torch

import exact_range_similarity_amd as ersj
import oracle
from workloads import CONFIGS, make_config, x_digest

from digest_util import block_fold, row_digests, u32
from gpu_util import say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
CHUNK = 1 << 27


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ersj.lib()


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
        f"pairs={total} band pairs re-checked (last batch)={st['last_boundary_pairs']}")
    return X, eps, rec, spec, parts, nb, total


def diff_rows(X, eps, parts, rows, label):
    """Message naming the rows whose GPU list differs from the oracle's."""
    rows = [int(r) for r in rows][:8]
    got = rows_of(parts, rows)
    colptr, cols = oracle.join_rows(X, eps, np.array(rows))
    e2 = oracle.e64(eps)
    lines = []
    for k, r in enumerate(rows):
        want = cols[colptr[k]:colptr[k + 1]].tolist()
        if got[r] == want:
            continue
        extra = sorted(set(got[r]) - set(want))[:4]
        missing = sorted(set(want) - set(got[r]))[:4]
        dup = len(got[r]) - len(set(got[r]))
        dd = [f"{j}: D64={oracle.d64(X[r], X[j])!r}" for j in extra + missing]
        lines.append(f"row {r}: gpu {len(got[r])} oracle {len(want)} dup {dup} extra {extra} missing {missing} "
                     f"E64={e2!r} {dd}")
    return f"{label}: rows differ\n" + "\n".join(lines)


def check_digests(name, X, eps, rec, parts):
    with open(os.path.join(GOLDEN, "digests.json")) as f:
        meta = json.load(f)[name]
    z = np.load(os.path.join(GOLDEN, f"digests_{name}.npz"))
    assert meta["eps"] == rec["eps"] and meta["x_sha256"] == rec["x_sha256"]
    assert meta["oracle_version"] == oracle.version()
    n = X.shape[0]
    if meta["mode"] == "full":
        cnt, dig = row_digests(parts, n)
        bc, fp = block_fold(cnt, dig, meta["block"])
        want_c = torch.from_numpy(z["block_count"].view(np.int64)).cuda()
        want_f = torch.from_numpy(z["block_digest"].view(np.int64)).cuda()
        bad = torch.nonzero((bc != want_c) | (fp != want_f)).flatten().cpu().numpy()
        if bad.size:
            blk = int(bad[0])
            rows = np.arange(blk * meta["block"], min(n, (blk + 1) * meta["block"]))
            oc, od, _ = oracle.digest_rows(X, eps, rows)
            c = cnt[blk * meta["block"]:(blk + 1) * meta["block"]].cpu().numpy()
            d = dig[blk * meta["block"]:(blk + 1) * meta["block"]].cpu().numpy().view(np.uint64)
            diff = rows[(c != oc) | (d != od)]
            raise AssertionError(f"{len(bad)} blocks differ; " + diff_rows(X, eps, parts, diff, name))
        assert int(cnt.sum()) == meta["pairs"]
        verified = n
    else:
        rows = torch.from_numpy(z["rows"].astype(np.int64)).cuda()
        cnt, dig = row_digests(parts, n, rows)
        want_c = torch.from_numpy(z["count"].astype(np.int64)).cuda()
        want_d = torch.from_numpy(z["digest"].view(np.int64)).cuda()
        bad = torch.nonzero((cnt != want_c) | (dig != want_d)).flatten().cpu().numpy()
        if bad.size:
            raise AssertionError(f"{len(bad)} rows differ; "
                                 + diff_rows(X, eps, parts, z["rows"][bad], name))
        verified = rows.numel()
    say(f"[gpu-full] {name}: {verified} rows equal to the oracle ({meta['mode']}); oracle band pairs "
        f"(|D64 - E64| <= {meta['band_rel']} E64) among them: {meta['band_pairs']}")
    return verified


def check_common(name, X, rec, spec, parts, symmetric=True):
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
    if symmetric:
        fwd, rev = sym_hash(parts)
        assert fwd == rev, f"{name}: pair set is not symmetric"


def check_unique(parts, n, rows_per_pass=None):
    """No pair twice: keys sorted per range of query rows (one range when
    rows_per_pass is None), so the largest results need not sort at once."""
    step = n if rows_per_pass is None else rows_per_pass
    for a in range(0, n, step):
        keys = []
        for q, x in chunks(parts):
            sel = (q >= a) & (q < a + step)
            if bool(sel.any()):
                keys.append((q[sel] << 32) | x[sel])
        if not keys:
            continue
        s = torch.sort(torch.cat(keys)).values
        del keys
        assert bool((s[1:] != s[:-1]).all()), f"duplicate pair among query rows {a}..{a + step - 1}"


def test_full_c1():
    X, eps, rec, spec, parts, nb, total = run_full("c1")
    check_common("c1", X, rec, spec, parts)
    check_unique(parts, X.shape[0])
    assert check_digests("c1", X, eps, rec, parts) == X.shape[0]


def test_full_c2():
    X, eps, rec, spec, parts, nb, total = run_full("c2")
    check_common("c2", X, rec, spec, parts)
    check_unique(parts, X.shape[0])
    assert check_digests("c2", X, eps, rec, parts) == X.shape[0]


def test_full_c3_four_plus_batches():
    X, eps, rec, spec, parts, nb, total = run_full("c3", budget_div=4.5)
    assert nb >= 4
    check_common("c3", X, rec, spec, parts)
    check_unique(parts, X.shape[0])
    assert check_digests("c3", X, eps, rec, parts) >= 11000


def test_full_c4():
    X, eps, rec, spec, parts, nb, total = run_full("c4")
    check_common("c4", X, rec, spec, parts)
    check_unique(parts, X.shape[0], rows_per_pass=1_000_000)
    assert check_digests("c4", X, eps, rec, parts) >= 11000


def test_full_c5():
    X, eps, rec, spec, parts, nb, total = run_full("c5")
    check_common("c5", X, rec, spec, parts)
    check_unique(parts, X.shape[0])
    assert check_digests("c5", X, eps, rec, parts) >= 11000
