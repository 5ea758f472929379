"""Compute epsilon for each synthetic workload with the CPU oracle and store it.

Writes ``tests/golden/eps_configs.json``.  Each workload's epsilon is the
value that gives a mean of k neighbours per point (self excluded, the
selectivity of "RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
Similarity Searches", Sec. V-B) over the first 1,000 points, each counted
against all points of the set.  Only ``workloads`` (to draw the points) and
``oracle`` (for the distances) are used.

    python -m oracle.calibrate [c1 c2 ...]
"""
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import CONFIGS, make_config, x_digest  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "eps_configs.json")
NQ = 1000


def calibrate(name: str, n: int = None):
    spec = CONFIGS[name]
    t0 = time.time()
    X = make_config(name, n)
    t1 = time.time()
    nq = min(NQ, X.shape[0])
    eps, a, b = oracle.calibrate_eps(X, nq, spec.k)
    t2 = time.time()
    return {
        "name": name, "n": int(X.shape[0]), "d": int(X.shape[1]), "k": spec.k, "nq": nq,
        "seed": spec.seed, "eps": eps.hex(), "eps_float": eps, "a": a.hex(), "b": b.hex(),
        "x_sha256": x_digest(X), "oracle_version": oracle.version(),
        "gen_s": round(t1 - t0, 2), "calib_s": round(t2 - t1, 2), "threads": oracle.threads(),
        "desc": spec.desc,
    }


def main(argv):
    names = argv or list(CONFIGS)
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    for nm in names:
        rec = calibrate(nm)
        data[nm] = rec
        print(json.dumps(rec), flush=True)
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:])
