"""Seeded workload generators and the stored epsilon values."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import CONFIGS, make_config, x_digest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def eps_table():
    with open(os.path.join(GOLDEN, "eps_configs.json")) as f:
        return json.load(f)


def test_deterministic_and_shaped():
    for name in CONFIGS:
        a = make_config(name, 3000)
        b = make_config(name, 3000)
        assert a.dtype == np.float32 and a.flags.c_contiguous
        assert a.shape == (3000, CONFIGS[name].d)
        assert np.array_equal(a, b)
        assert np.isfinite(a).all()


def test_value_distributions():
    x1 = make_config("c1", 20000)
    assert x1.min() >= 0.0 and x1.max() < 1.0
    x5 = make_config("c5", 4000)
    nrm = np.linalg.norm(x5.astype(np.float64), axis=1)
    assert np.allclose(nrm, 1.0, atol=1e-6)
    x4 = make_config("c4", 20000)
    # 30% uniform background: roughly 30% of rows sit far from every cluster
    assert 0.0 <= x4.min() and x4.max() < 1.2


def test_stored_eps_match_regenerated_inputs():
    tab = eps_table()
    for name in ("c1", "c2"):
        rec = tab[name]
        X = make_config(name)
        assert X.shape == (rec["n"], rec["d"])
        assert x_digest(X) == rec["x_sha256"]
        eps = float.fromhex(rec["eps"])
        a, b = float.fromhex(rec["a"]), float.fromhex(rec["b"])
        assert a <= oracle.e64(eps) < b


def test_calibration_identity_c1():
    """With the stored eps, rows 0..999 of c1 hold exactly 1000*k non-self neighbours."""
    rec = eps_table()["c1"]
    X = make_config("c1")
    colptr, _ = oracle.join_rows(X, float.fromhex(rec["eps"]), np.arange(rec["nq"]))
    assert int(colptr[-1]) - rec["nq"] == rec["nq"] * rec["k"]


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_eps_table_complete(name):
    rec = eps_table()[name]
    assert rec["n"] == CONFIGS[name].n and rec["d"] == CONFIGS[name].d
    eps = float.fromhex(rec["eps"])
    assert math.isfinite(eps) and eps > 0


def test_query_sets_share_the_structure_of_the_points():
    from workloads import make_queries
    for name in CONFIGS:
        Q1 = make_queries(name, 3000, 11, 20000)
        Q2 = make_queries(name, 3000, 11, 20000)
        assert Q1.dtype == np.float32 and Q1.shape == (3000, CONFIGS[name].d) and Q1.flags.c_contiguous
        assert np.array_equal(Q1, Q2)
        assert not np.array_equal(Q1, make_queries(name, 3000, 12, 20000))
    # same cluster centres as the points: every clustered query lies near some point
    X = make_config("c2", 20000)
    Q = make_queries("c2", 200, 11, 20000)
    d2 = ((Q[:, None, :].astype(np.float64) - X[None, :, :]) ** 2).sum(-1).min(axis=1)
    assert np.all(d2 < 0.05)


def test_smoke_input_calibrates():
    """The smoke case's epsilon gives queries 0..499 a whole number of
    neighbours per query (target 32, or a neighbouring target where 32 falls
    on a tie), and more than one pair per query."""
    import __graft_entry__ as entry
    X, eps = entry.smoke_input()
    colptr, _ = oracle.join_rows(X, eps, np.arange(500))
    total = int(colptr[-1]) - 500
    assert total % 500 == 0 and 30 <= total // 500 <= 34
