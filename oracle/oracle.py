"""ctypes front end of the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY.  Every function here follows the problem statement
of "RT-HiSS: Ray Tracing Accelerated High Dimensional Vector Similarity
Searches", Sec. II-A: Euclidean distance, neighbours iff the distance is at
most epsilon, self-join with Q = D, results as (query id, point id) pairs
(Sec. II-A1), self pairs included (the selectivity of Sec. V-B excludes them
from the per-query mean, so the result set holds them).  The arithmetic is
the canonical binary64 squared distance compared with fl(eps*eps); see the
header of ``oracle.c``.
"""
import ctypes
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = ctypes.POINTER(ctypes.c_float)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_dblp = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_version.restype = ctypes.c_int
    lib.orc_threads.restype = ctypes.c_int
    lib.orc_d64.restype = ctypes.c_double
    lib.orc_d64.argtypes = [_f32p, _f32p, ctypes.c_int64]
    lib.orc_e64.restype = ctypes.c_double
    lib.orc_e64.argtypes = [ctypes.c_double]
    lib.orc_join_rows.restype = ctypes.c_int
    lib.orc_join_rows.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_double, _i64p, ctypes.c_int64, _u64p, _u32p, _u64p]
    lib.orc_semijoin_rows.restype = ctypes.c_int
    lib.orc_semijoin_rows.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int64, _f32p, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_double, _i64p,
                                      ctypes.c_int64, _u64p, _u32p, _u64p]
    lib.orc_band_count.restype = ctypes.c_int64
    lib.orc_band_count.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_double, ctypes.c_double, _i64p, ctypes.c_int64]
    lib.orc_mix64.restype = ctypes.c_uint64
    lib.orc_mix64.argtypes = [ctypes.c_uint64]
    lib.orc_digest_rows.restype = ctypes.c_int
    lib.orc_digest_rows.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                    ctypes.c_double, _i64p, ctypes.c_int64, _u32p, _u64p, _u32p]
    lib.orc_digest_all.restype = ctypes.c_int
    lib.orc_digest_all.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                   ctypes.c_double, _u32p, _u64p, _u32p]
    lib.orc_knn.restype = ctypes.c_int
    lib.orc_knn.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int64, _f32p, ctypes.c_int64,
                            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _i64p, ctypes.c_int64,
                            _u32p, _dblp]
    lib.orc_calibrate.restype = ctypes.c_int
    lib.orc_calibrate.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _dblp, _dblp]
    _lib = lib
    return lib


def available() -> bool:
    try:
        _load()
        return True
    except OSError:
        return False


def version() -> int:
    return _load().orc_version()


def threads() -> int:
    return _load().orc_threads()


def _as_x(X):
    X = np.asarray(X)
    if X.dtype != np.float32 or X.ndim != 2:
        raise TypeError("X must be a 2-D float32 array")
    if not X.flags.c_contiguous:
        X = np.ascontiguousarray(X)
    return X


def _ptr(a, t):
    return a.ctypes.data_as(t)


def d64(a, b) -> float:
    """Canonical squared distance of two float32 vectors (binary64, no FMA)."""
    a = np.ascontiguousarray(a, dtype=np.float32).ravel()
    b = np.ascontiguousarray(b, dtype=np.float32).ravel()
    if a.shape != b.shape:
        raise ValueError("shape mismatch")
    return _load().orc_d64(_ptr(a, _f32p), _ptr(b, _f32p), a.size)


def e64(eps: float) -> float:
    return _load().orc_e64(float(eps))


def _rows_arg(rows):
    if rows is None:
        return None, None
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, _ptr(r, _i64p)


def join_rows(X, eps, rows=None):
    """Neighbour lists of ``rows`` (all rows if None) as CSR (colptr, cols).

    cols are point ids in ascending order within each row.
    """
    X = _as_x(X)
    n, d = X.shape
    lib = _load()
    r, rp = _rows_arg(rows)
    nrows = n if r is None else r.size
    counts = np.zeros(nrows, dtype=np.uint64)
    rc = lib.orc_join_rows(_ptr(X, _f32p), n, d, d, float(eps), rp, nrows,
                           _ptr(counts, _u64p), None, None)
    if rc != 0:
        raise ValueError(f"oracle rejected the input (code {rc})")
    colptr = np.zeros(nrows + 1, dtype=np.uint64)
    np.cumsum(counts, out=colptr[1:])
    cols = np.empty(int(colptr[-1]), dtype=np.uint32)
    if cols.size:
        rc = lib.orc_join_rows(_ptr(X, _f32p), n, d, d, float(eps), rp, nrows,
                               None, _ptr(cols, _u32p), _ptr(colptr, _u64p))
        if rc != 0:
            raise ValueError(f"oracle rejected the input (code {rc})")
    return colptr, cols


def semijoin_rows(Q, X, eps, rows=None):
    """Neighbour lists in X of the query rows ``rows`` of Q (all if None), as
    CSR (colptr, cols); cols ascending.  RT-HiSS Sec. II-A, the semi-join."""
    Q = _as_x(Q)
    X = _as_x(X)
    nq, d = Q.shape
    n, dx = X.shape
    if d != dx:
        raise ValueError("Q and X differ in dimension")
    lib = _load()
    r, rp = _rows_arg(rows)
    nrows = nq if r is None else r.size
    counts = np.zeros(nrows, dtype=np.uint64)
    rc = lib.orc_semijoin_rows(_ptr(Q, _f32p), nq, d, _ptr(X, _f32p), n, d, d, float(eps), rp, nrows,
                               _ptr(counts, _u64p), None, None)
    if rc != 0:
        raise ValueError(f"oracle rejected the input (code {rc})")
    colptr = np.zeros(nrows + 1, dtype=np.uint64)
    np.cumsum(counts, out=colptr[1:])
    cols = np.empty(int(colptr[-1]), dtype=np.uint32)
    if cols.size:
        rc = lib.orc_semijoin_rows(_ptr(Q, _f32p), nq, d, _ptr(X, _f32p), n, d, d, float(eps), rp, nrows,
                                   None, _ptr(cols, _u32p), _ptr(colptr, _u64p))
        if rc != 0:
            raise ValueError(f"oracle rejected the input (code {rc})")
    return colptr, cols


def semijoin_pairs(Q, X, eps):
    """All (j, i) with D64(q_j, x_i) <= fl(eps*eps) (query id, point id), uint32 [|R|, 2], sorted."""
    colptr, cols = semijoin_rows(Q, X, eps)
    counts = np.diff(colptr).astype(np.int64)
    q = np.repeat(np.arange(counts.size, dtype=np.uint32), counts)
    return np.stack([q, cols], axis=1)


def selfjoin_pairs(X, eps):
    """All (i, j) with D64(x_i, x_j) <= fl(eps*eps), as uint32 [|R|, 2], sorted."""
    colptr, cols = join_rows(X, eps)
    counts = np.diff(colptr).astype(np.int64)
    q = np.repeat(np.arange(counts.size, dtype=np.uint32), counts)
    return np.stack([q, cols], axis=1)


def knn_rows(Q, X, k: int, rows=None):
    """Exact k nearest neighbours in X of the query rows ``rows`` of Q (all if
    None), RT-HiSS Sec. VI: every point ranked by (D64, point id) ascending,
    the first k.  Returns (ids uint32 [nrows, k], d64 float64 [nrows, k])."""
    Q = _as_x(Q)
    X = _as_x(X)
    nq, d = Q.shape
    n, dx = X.shape
    if d != dx:
        raise ValueError("Q and X differ in dimension")
    r, rp = _rows_arg(rows)
    nrows = nq if r is None else r.size
    ids = np.zeros((nrows, int(k)), dtype=np.uint32)
    dist = np.zeros((nrows, int(k)), dtype=np.float64)
    rc = _load().orc_knn(_ptr(Q, _f32p), nq, d, _ptr(X, _f32p), n, d, d, int(k), rp, nrows,
                         _ptr(ids, _u32p), _ptr(dist, _dblp))
    if rc != 0:
        raise ValueError(f"oracle rejected the input (code {rc})")
    return ids, dist


def knn(X, k: int, rows=None):
    """Self kNN: the query rows are the points themselves (each its own first
    neighbour unless an identical point has a smaller id)."""
    return knn_rows(X, X, k, rows)


def band_count(X, eps, rel=1e-6, rows=None) -> int:
    """Ordered pairs (row, j) with |D64 - E64| <= rel * E64 over the selected
    rows (all if None): the pairs a reduced-precision classifier cannot
    decide without the exact binary64 test."""
    X = _as_x(X)
    n, d = X.shape
    r, rp = _rows_arg(rows)
    nrows = n if r is None else r.size
    v = _load().orc_band_count(_ptr(X, _f32p), n, d, d, float(eps), float(rel), rp, nrows)
    if v < 0:
        raise ValueError("oracle rejected the input")
    return int(v)


def mix64(j: int) -> int:
    """The splitmix64 output function of j (neighbour-list fingerprints)."""
    return int(_load().orc_mix64(int(j) & 0xffffffffffffffff))


def digest_rows(X, eps, rows=None, rel=1e-6):
    """Per selected row (all if None): (count, fingerprint, band) as uint32,
    uint64, uint32 arrays; fingerprint = sum of mix64(j) over the row's
    neighbours mod 2^64, band = points with |D64 - E64| <= rel * E64."""
    X = _as_x(X)
    n, d = X.shape
    r, rp = _rows_arg(rows)
    nrows = n if r is None else r.size
    cnt = np.zeros(nrows, dtype=np.uint32)
    dig = np.zeros(nrows, dtype=np.uint64)
    band = np.zeros(nrows, dtype=np.uint32)
    rc = _load().orc_digest_rows(_ptr(X, _f32p), n, d, d, float(eps), float(rel), rp, nrows,
                                 _ptr(cnt, _u32p), _ptr(dig, _u64p), _ptr(band, _u32p))
    if rc != 0:
        raise ValueError(f"oracle rejected the input (code {rc})")
    return cnt, dig, band


def digest_all(X, eps, rel=1e-6):
    """digest_rows for every row, each unordered pair evaluated once (mirrored)."""
    X = _as_x(X)
    n, d = X.shape
    cnt = np.zeros(n, dtype=np.uint32)
    dig = np.zeros(n, dtype=np.uint64)
    band = np.zeros(n, dtype=np.uint32)
    rc = _load().orc_digest_all(_ptr(X, _f32p), n, d, d, float(eps), float(rel),
                                _ptr(cnt, _u32p), _ptr(dig, _u64p), _ptr(band, _u32p))
    if rc != 0:
        raise ValueError(f"oracle rejected the input (code {rc})")
    return cnt, dig, band


def calibrate_bounds(X, nq: int, k: int):
    """(a, b): the K-th and (K+1)-th smallest non-self D64 over queries 0..nq-1, K = nq*k."""
    X = _as_x(X)
    n, d = X.shape
    lib = _load()
    m = max(4 * k, 64)
    while True:
        a = ctypes.c_double()
        b = ctypes.c_double()
        rc = lib.orc_calibrate(_ptr(X, _f32p), n, d, d, int(nq), int(k), int(m),
                               ctypes.byref(a), ctypes.byref(b))
        if rc == 0:
            return a.value, b.value
        if rc != 1:
            raise ValueError(f"oracle rejected the input (code {rc})")
        if m >= n - 1:
            raise RuntimeError("calibration did not converge")
        m = min(n - 1, 4 * m)


def calibrate_eps(X, nq: int, k: int):
    """epsilon with exactly nq*k non-self neighbours over queries 0..nq-1.

    Returns (eps, a, b) with a <= fl(eps*eps) < b.  eps starts at the root of
    the midpoint of [a, b) and is stepped one ulp at a time into the interval.
    """
    a, b = calibrate_bounds(X, nq, k)
    if not a < b:
        raise RuntimeError("tied distances at the calibration point; no epsilon gives the target")
    eps = math.sqrt(0.5 * (a + b))
    for _ in range(256):
        s = e64(eps)
        if s < a:
            eps = math.nextafter(eps, math.inf)
        elif s >= b:
            eps = math.nextafter(eps, 0.0)
        else:
            return eps, a, b
    raise RuntimeError("no binary64 epsilon squares into [a, b)")
