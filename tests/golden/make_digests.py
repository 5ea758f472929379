"""Write the CPU oracle's neighbour-list fingerprints of the full-size workloads.

Calls only ``oracle/`` (the binary64 brute force) and ``workloads/`` (the
seeded point generators); nothing here touches the GPU library.  The result
set being fingerprinted is the self-join of "RT-HiSS: Ray Tracing
Accelerated High Dimensional Vector Similarity Searches", Sec. II-A: the
ordered pairs (i, j) with D64(x_i, x_j) <= fl(eps * eps), self pairs
included.

Per row i the oracle gives c_i = |N(i)|, h_i = sum of mix64(j) over N(i)
(mod 2^64) and b_i = the points j with |D64 - E64| <= 1e-6 E64 (the pairs
near the threshold).  Stored, in ``digests_<config>.npz``:

* ``full`` mode (every row; the j >= i half of the pairs is evaluated and
  mirrored): per block of BLOCK consecutive rows, the sum of c_i, the sum of
  b_i, and sum over the block of mix64(h_i + mix64(c_i + i * 2^32)) mod 2^64,
  which changes when any row's list changes, including two rows trading
  lists.
* ``rows`` mode (a fixed sample): the rows themselves and their c_i, h_i and
  b_i.  The sample is rows 0..999 (the rows epsilon was calibrated on),
  10,000 other rows drawn with numpy's default_rng(10000 + seed), every row
  of the largest cluster, and for the mixture with a uniform background
  2,000 background rows drawn with default_rng(20000 + seed).

``digests.json`` records, per config: seed, n, d, eps (hex), the SHA-256 of
the points, the oracle version, the mode, the totals and the oracle time.

    python tests/golden/make_digests.py c2 c3 c4 c5
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import CONFIGS, make_config_labels, x_digest  # noqa: E402

BLOCK = 64
BAND_REL = 1e-6
MODES = {"c1": "full", "c2": "full", "c3": "rows", "c4": "rows", "c5": "rows"}
M64 = (1 << 64) - 1


def mix64_np(v):
    """splitmix64 output function on a uint64 array (wrapping arithmetic)."""
    z = v.astype(np.uint64) + np.uint64(0x9e3779b97f4a7c15)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xbf58476d1ce4e5b9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94d049bb133111eb)
    return z ^ (z >> np.uint64(31))


def block_fold(cnt, dig, band):
    """Per-block sums of the counts and band counts and the block fingerprint."""
    n = cnt.size
    i = np.arange(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        t = mix64_np(dig.astype(np.uint64) + mix64_np(cnt.astype(np.uint64) + (i << np.uint64(32))))
    nblk = (n + BLOCK - 1) // BLOCK
    pad = nblk * BLOCK - n
    tp = np.concatenate([t, np.zeros(pad, dtype=np.uint64)]).reshape(nblk, BLOCK)
    fp = np.zeros(nblk, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for k in range(BLOCK):  # wrapping sum
            fp += tp[:, k]
    bc = np.add.reduceat(cnt.astype(np.uint64), np.arange(0, n, BLOCK))
    bb = np.add.reduceat(band.astype(np.uint64), np.arange(0, n, BLOCK))
    return bc, fp, bb


def sample_rows(name, labels):
    spec = CONFIGS[name]
    n = labels.size
    rows = [np.arange(min(1000, n), dtype=np.int64)]
    rng = np.random.default_rng(10000 + spec.seed)
    rows.append(rng.choice(np.arange(1000, n, dtype=np.int64), size=min(10000, n - 1000), replace=False))
    lab = labels[labels >= 0]
    if lab.size:
        big = int(np.argmax(np.bincount(lab)))
        rows.append(np.flatnonzero(labels == big).astype(np.int64))
    bg = np.flatnonzero(labels < 0)
    if bg.size and lab.size:
        rng2 = np.random.default_rng(20000 + spec.seed)
        rows.append(rng2.choice(bg, size=min(2000, bg.size), replace=False).astype(np.int64))
    return np.unique(np.concatenate(rows))


def make(name, meta):
    spec = CONFIGS[name]
    with open(os.path.join(HERE, "eps_configs.json")) as f:
        rec = json.load(f)[name]
    X, labels = make_config_labels(name)
    sha = x_digest(X)
    if sha != rec["x_sha256"]:
        raise SystemExit(f"{name}: generated points differ from the calibrated ones")
    eps = float.fromhex(rec["eps"])
    mode = MODES[name]
    t = time.time()
    print(f"[digests] {name}: mode {mode}, n={X.shape[0]} d={X.shape[1]}, {oracle.threads()} threads",
          flush=True)
    if mode == "full":
        cnt, dig, band = oracle.digest_all(X, eps, BAND_REL)
        dt = time.time() - t
        bc, fp, bb = block_fold(cnt, dig, band)
        np.savez_compressed(os.path.join(HERE, f"digests_{name}.npz"), block_count=bc, block_digest=fp,
                            block_band=bb)
        total, tband, nrows = int(cnt.sum(dtype=np.uint64)), int(band.sum(dtype=np.uint64)), X.shape[0]
    else:
        rows = sample_rows(name, labels)
        cnt, dig, band = oracle.digest_rows(X, eps, rows, BAND_REL)
        dt = time.time() - t
        np.savez_compressed(os.path.join(HERE, f"digests_{name}.npz"), rows=rows.astype(np.uint32),
                            count=cnt, digest=dig, band=band)
        total, tband, nrows = int(cnt.sum(dtype=np.uint64)), int(band.sum(dtype=np.uint64)), rows.size
    meta[name] = {
        "seed": spec.seed, "n": int(X.shape[0]), "d": int(X.shape[1]), "eps": rec["eps"],
        "x_sha256": sha, "oracle_version": oracle.version(), "mode": mode, "block": BLOCK,
        "band_rel": BAND_REL, "rows": int(nrows), "pairs": total, "band_pairs": tband,
        "oracle_s": round(dt, 1), "threads": oracle.threads(),
    }
    print(f"[digests] {name}: {nrows} rows, {total} pairs, {tband} band pairs, {dt:.0f}s", flush=True)


def main(names):
    path = os.path.join(HERE, "digests.json")
    meta = {}
    if os.path.exists(path):
        with open(path) as f:
            meta = json.load(f)
    for name in names:
        make(name, meta)
        with open(path, "w") as f:
            json.dump(meta, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["c2", "c3", "c4", "c5"])
