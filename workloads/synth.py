"""Seeded synthetic point sets.

The five workload families stand in for the real datasets the method was
measured on ("RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
Similarity Searches", Sec. V-B, Table I: d from 18 to 128, 0.3M to 11.6M
points), which are not available here.  Each family fixes a size, a
dimensionality, a value distribution and a target selectivity k (mean
neighbours per point, self excluded, as in Sec. V-B).  Epsilon is not drawn
here: it is computed from the drawn points by the CPU oracle's calibration.

All draws use ``numpy.random.default_rng(seed)`` in a fixed order, in fixed
row chunks, so an array depends only on (family, n, seed).  ``n`` below the
family's full size shrinks the number of clusters in proportion, keeping the
points-per-cluster density of the full workload.
"""
import dataclasses
import hashlib
import math

import numpy as np

_CHUNK = 1 << 18


@dataclasses.dataclass(frozen=True)
class ConfigSpec:
    name: str
    n: int
    d: int
    k: int                 # target mean neighbours per point, self excluded
    kind: str
    clusters: int = 0
    sigma: float = 0.0
    sig_lo: float = 0.0
    sig_hi: float = 0.0
    frac: float = 0.0      # fraction of clustered rows (mixture with background)
    noise: float = 0.0
    seed: int = 0
    desc: str = ""


CONFIGS = {
    "c1": ConfigSpec("c1", 20_000, 16, 32, "uniform", seed=1,
                     desc="N=20,000, d=16, i.i.d. uniform [0,1)"),
    "c2": ConfigSpec("c2", 1_000_000, 32, 64, "gauss_iso", clusters=100, sigma=0.02, seed=2,
                     desc="N=1,000,000, d=32, 100 isotropic Gaussians (sigma=0.02)"),
    "c3": ConfigSpec("c3", 2_000_000, 64, 128, "gauss_aniso", clusters=1000,
                     sig_lo=0.005, sig_hi=0.05, seed=3,
                     desc="N=2,000,000, d=64, 1,000 anisotropic Gaussians "
                          "(per-dim sigma log-uniform in [0.005,0.05])"),
    "c4": ConfigSpec("c4", 10_000_000, 18, 256, "mix_bg", clusters=500, sigma=0.01, frac=0.7,
                     seed=4, desc="N=10,000,000, d=18, 70% in 500 Gaussians (sigma=0.01) "
                                  "+ 30% uniform background"),
    "c5": ConfigSpec("c5", 1_000_000, 384, 50, "embed", clusters=2000, noise=0.3, seed=5,
                     desc="N=1,000,000, d=384, unit-norm normalize(center + 0.3*noise), "
                          "2,000 centers"),
}


def config_spec(name: str) -> ConfigSpec:
    return CONFIGS[name]


def _scaled_clusters(spec: ConfigSpec, n: int) -> int:
    if n >= spec.n:
        return spec.clusters
    return max(1, int(round(spec.clusters * n / spec.n)))


def _normal_rows(rng, n, d):
    out = np.empty((n, d), dtype=np.float64)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = rng.standard_normal((e - s, d))
    return out


def make_config(name: str, n: int = None, seed: int = None) -> np.ndarray:
    """Points of workload ``name`` as a C-contiguous float32 [n, d] array."""
    return _generate(name, n, seed)[0]


def make_config_labels(name: str, n: int = None, seed: int = None):
    """(points, labels): the array of ``make_config`` and, per row, the index
    of the cluster it was drawn from (int32; -1 for uniform rows and for the
    background of the mixture)."""
    return _generate(name, n, seed)


def _generate(name: str, n: int = None, seed: int = None):
    spec = CONFIGS[name]
    n = spec.n if n is None else int(n)
    seed = spec.seed if seed is None else int(seed)
    if n < 1:
        raise ValueError("n must be positive")
    rng = np.random.default_rng(seed)
    d = spec.d
    if spec.kind == "uniform":
        return rng.random((n, d), dtype=np.float32), np.full(n, -1, dtype=np.int32)
    nc = _scaled_clusters(spec, n)
    if spec.kind == "gauss_iso":
        C = rng.random((nc, d))
        L = rng.integers(0, nc, n)
        X = np.empty((n, d), dtype=np.float32)
        for s in range(0, n, _CHUNK):
            e = min(n, s + _CHUNK)
            X[s:e] = C[L[s:e]] + spec.sigma * rng.standard_normal((e - s, d))
        return X, L.astype(np.int32)
    if spec.kind == "gauss_aniso":
        C = rng.random((nc, d))
        S = np.exp(rng.uniform(math.log(spec.sig_lo), math.log(spec.sig_hi), (nc, d)))
        L = rng.integers(0, nc, n)
        X = np.empty((n, d), dtype=np.float32)
        for s in range(0, n, _CHUNK):
            e = min(n, s + _CHUNK)
            X[s:e] = C[L[s:e]] + S[L[s:e]] * rng.standard_normal((e - s, d))
        return X, L.astype(np.int32)
    if spec.kind == "mix_bg":
        ncl = int(round(spec.frac * n))
        C = rng.random((nc, d))
        L = rng.integers(0, nc, ncl)
        X = np.empty((n, d), dtype=np.float32)
        for s in range(0, ncl, _CHUNK):
            e = min(ncl, s + _CHUNK)
            X[s:e] = C[L[s:e]] + spec.sigma * rng.standard_normal((e - s, d))
        for s in range(ncl, n, _CHUNK):
            e = min(n, s + _CHUNK)
            X[s:e] = rng.random((e - s, d))
        perm = rng.permutation(n)
        lab = np.full(n, -1, dtype=np.int32)
        lab[:ncl] = L
        return np.ascontiguousarray(X[perm]), lab[perm]
    if spec.kind == "embed":
        C = rng.standard_normal((nc, d))
        C /= np.linalg.norm(C, axis=1, keepdims=True)
        L = rng.integers(0, nc, n)
        X = np.empty((n, d), dtype=np.float32)
        scale = spec.noise / math.sqrt(d)
        for s in range(0, n, _CHUNK):
            e = min(n, s + _CHUNK)
            Y = C[L[s:e]] + scale * rng.standard_normal((e - s, d))
            Y /= np.linalg.norm(Y, axis=1, keepdims=True)
            X[s:e] = Y
        return X, L.astype(np.int32)
    raise ValueError(f"unknown workload kind {spec.kind}")


def make_queries(name: str, nq: int, seed: int, n_points: int = None) -> np.ndarray:
    """A query set for a semi-join against ``make_config(name, n_points)``: the
    same structure (cluster centres, per-cluster scales: the generator's first
    draws from the workload's seed) with rows, labels and noise drawn from
    ``seed``.  float32 [nq, d], C-contiguous."""
    spec = CONFIGS[name]
    n_points = spec.n if n_points is None else int(n_points)
    nq = int(nq)
    if nq < 1:
        raise ValueError("nq must be positive")
    d = spec.d
    rs = np.random.default_rng(spec.seed)  # structure, drawn as make_config draws it
    rng = np.random.default_rng(seed)
    if spec.kind == "uniform":
        return rng.random((nq, d), dtype=np.float32)
    nc = _scaled_clusters(spec, n_points)
    Q = np.empty((nq, d), dtype=np.float32)
    if spec.kind in ("gauss_iso", "gauss_aniso", "mix_bg"):
        C = rs.random((nc, d))
        S = None
        if spec.kind == "gauss_aniso":
            S = np.exp(rs.uniform(math.log(spec.sig_lo), math.log(spec.sig_hi), (nc, d)))
        ncl = int(round(spec.frac * nq)) if spec.kind == "mix_bg" else nq
        L = rng.integers(0, nc, ncl)
        for s0 in range(0, ncl, _CHUNK):
            e = min(ncl, s0 + _CHUNK)
            sc = S[L[s0:e]] if S is not None else spec.sigma
            Q[s0:e] = C[L[s0:e]] + sc * rng.standard_normal((e - s0, d))
        for s0 in range(ncl, nq, _CHUNK):
            e = min(nq, s0 + _CHUNK)
            Q[s0:e] = rng.random((e - s0, d))
        if spec.kind == "mix_bg":
            Q = np.ascontiguousarray(Q[rng.permutation(nq)])
        return Q
    if spec.kind == "embed":
        C = rs.standard_normal((nc, d))
        C /= np.linalg.norm(C, axis=1, keepdims=True)
        L = rng.integers(0, nc, nq)
        scale = spec.noise / math.sqrt(d)
        for s0 in range(0, nq, _CHUNK):
            e = min(nq, s0 + _CHUNK)
            Y = C[L[s0:e]] + scale * rng.standard_normal((e - s0, d))
            Y /= np.linalg.norm(Y, axis=1, keepdims=True)
            Q[s0:e] = Y
        return Q
    raise ValueError(f"unknown workload kind {spec.kind}")


def lattice(m: int, d: int, spacing: float = 1.0) -> np.ndarray:
    """All points of the integer box {0..m-1}^d times ``spacing``, row-major enumeration."""
    axes = [np.arange(m, dtype=np.float64)] * d
    g = np.stack(np.meshgrid(*axes, indexing="ij"), axis=-1).reshape(-1, d)
    return np.ascontiguousarray((g * spacing).astype(np.float32))


def fig3_points() -> np.ndarray:
    """Seven 2-D points realising the neighbour structure drawn in Fig. 3 at eps = 1.

    p0-p2, p1-p3 and p5-p6 are neighbours and nothing else (besides self pairs);
    p4, p0, p2 lie close together, p5, p6 near them, p1, p3 far away.
    """
    return np.array([
        [0.0, 0.0],     # p0
        [10.0, 10.0],   # p1
        [0.8, 0.0],     # p2
        [10.5, 10.2],   # p3
        [-1.5, 0.5],    # p4
        [2.5, 0.0],     # p5
        [3.2, 0.3],     # p6
    ], dtype=np.float32)


def fig5_points() -> np.ndarray:
    """Fourteen 2-D points whose point 1 has, at eps = 1, exactly the neighbours
    at positions 1, 5, 8, 9 and 12 of the row drawn in Fig. 5."""
    pts = np.zeros((14, 2), dtype=np.float64)
    near = {1: 0.0, 5: 0.9, 8: 0.5, 9: 0.75, 12: 0.99}
    for i in range(14):
        ang = 0.45 * i
        r = near.get(i, 2.0 + 0.25 * i)
        pts[i] = (r * math.cos(ang), r * math.sin(ang))
    return pts.astype(np.float32)


def x_digest(X: np.ndarray) -> str:
    X = np.ascontiguousarray(X)
    h = hashlib.sha256()
    h.update(str(X.shape).encode())
    h.update(memoryview(X).cast("B"))
    return h.hexdigest()
