"""Exact epsilon-distance self-join on AMD Instinct MI355X (gfx950).

Thin ctypes binding of ``libersj.so`` (C ABI in ``include/ersj.h``).  The
functions carry the C names without the ``ersj_`` prefix and only marshal
arguments: every step of the join runs in the library's HIP kernels.
PyTorch supplies device memory (input and output tensors) and the stream.

The operation ("RT-HiSS: Ray Tracing Accelerated High Dimensional Vector
Similarity Searches", Sec. II-A): all ordered pairs (i, j) of rows of ``x``
with Euclidean distance at most ``eps``, self pairs included.
"""
import ctypes
import os

import torch  # loads the HIP runtime the library must share with torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# ERSJ_LIBRARY selects another build of the same library (for example the
# host-sanitized one that exact_range_similarity_amd.build makes on request)
LIB_PATH = os.environ.get("ERSJ_LIBRARY") or os.path.join(_HERE, "libersj.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_STATE = -2
ERR_HIP = -3
ERR_OOM = -4
ERR_BUDGET = -5
ERR_CAPACITY = -6
ERR_SCRATCH = -7
ERR_INTERNAL = -8

REFINE_AUTO = 0
REFINE_DIRECT = 1
REFINE_MFMA = 2
REFINE_MFMA16 = 3

_NAMES = {0: "OK", -1: "INVALID_ARG", -2: "STATE", -3: "HIP", -4: "OOM", -5: "BUDGET",
          -6: "CAPACITY", -7: "SCRATCH", -8: "INTERNAL"}

# ERSJ_NOALLOC_SCRATCH_BYTES / ERSJ_NOALLOC_MASK_BUDGET of include/ersj.h
NOALLOC_SCRATCH_BYTES = 64 << 20
NOALLOC_MASK_BUDGET = 48 << 20


class ErsjError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


class Options(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("refine_kernel", ctypes.c_int32),
                ("cell_width_scale", ctypes.c_double), ("max_device_bytes", ctypes.c_uint64),
                ("boundary_capacity", ctypes.c_uint64), ("timing", ctypes.c_int32),
                ("grid_reach", ctypes.c_int32), ("block_prune", ctypes.c_int32),
                ("cell_order", ctypes.c_int32), ("mfma_products", ctypes.c_int32),
                ("filter_bits", ctypes.c_int32)]


class Stats(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("d", ctypes.c_int32), ("index_dims", ctypes.c_int32 * 3),
                ("grid", ctypes.c_int32 * 3), ("refine_kernel", ctypes.c_int32),
                ("cells", ctypes.c_int64), ("tiles", ctypes.c_int64),
                ("total_candidates", ctypes.c_uint64), ("total_mask_words", ctypes.c_uint64),
                ("n_batches", ctypes.c_int32), ("last_batch", ctypes.c_int32),
                ("max_batch_words", ctypes.c_uint64), ("last_batch_candidates", ctypes.c_uint64),
                ("last_batch_pairs", ctypes.c_uint64), ("last_boundary_pairs", ctypes.c_uint64),
                ("last_recheck_in", ctypes.c_uint64), ("device_bytes", ctypes.c_uint64),
                ("build_ms", ctypes.c_double), ("count_ms", ctypes.c_double),
                ("plan_ms", ctypes.c_double), ("refine_ms", ctypes.c_double),
                ("recheck_ms", ctypes.c_double), ("expand_ms", ctypes.c_double),
                ("refine_launches", ctypes.c_int64), ("refined_candidates", ctypes.c_uint64),
                ("n_queries", ctypes.c_int64), ("last_skipped", ctypes.c_uint64),
                ("skipped_candidates", ctypes.c_uint64), ("mfma_products", ctypes.c_int32),
                ("last_partial", ctypes.c_uint64), ("partial_candidates", ctypes.c_uint64),
                ("last_filtered", ctypes.c_int32), ("filter_bits", ctypes.c_int32)]

    def as_dict(self):
        out = {}
        for name, _ in self._fields_:
            v = getattr(self, name)
            out[name] = list(v) if isinstance(v, ctypes.Array) else v
        return out


_lib = None
KNN_MAX_ROUNDS = 41


class KnnInfo(ctypes.Structure):
    _fields_ = [("rounds", ctypes.c_int32), ("refine_kernel", ctypes.c_int32),
                ("eps", ctypes.c_double * KNN_MAX_ROUNDS), ("queries", ctypes.c_int64 * KNN_MAX_ROUNDS),
                ("candidates", ctypes.c_uint64 * KNN_MAX_ROUNDS),
                ("dim_estimate", ctypes.c_double * KNN_MAX_ROUNDS),
                ("total_candidates", ctypes.c_uint64), ("index_ms", ctypes.c_double),
                ("refine_ms", ctypes.c_double), ("recheck_ms", ctypes.c_double),
                ("select_ms", ctypes.c_double), ("refine_launches", ctypes.c_int64),
                ("computed_candidates", ctypes.c_uint64)]

    def as_dict(self):
        r = min(self.rounds, KNN_MAX_ROUNDS)
        return {"rounds": self.rounds, "refine_kernel": self.refine_kernel, "eps": list(self.eps[:r]), "queries": list(self.queries[:r]),
                "candidates": list(self.candidates[:r]), "dim_estimate": list(self.dim_estimate[:r]),
                "total_candidates": self.total_candidates, "index_ms": self.index_ms,
                "refine_ms": self.refine_ms, "recheck_ms": self.recheck_ms, "select_ms": self.select_ms,
                "refine_launches": self.refine_launches,
                "computed_candidates": self.computed_candidates}


SYMBOLS = ("ersj_default_options", "ersj_build_index", "ersj_set_queries", "ersj_count_pass",
           "ersj_plan_batches", "ersj_fill_pass", "ersj_fill_pass_host", "ersj_fill_pass_noalloc",
           "ersj_host_sync",
           "ersj_batch_info", "ersj_get_stats", "ersj_free", "ersj_release_cached", "ersj_last_error", "ersj_knn")


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(python -m exact_range_similarity_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64, dbl = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                              ctypes.c_double)
    L.ersj_default_options.argtypes = [ctypes.POINTER(Options)]
    L.ersj_default_options.restype = None
    L.ersj_build_index.argtypes = [vp, i64, i32, i64, dbl, ctypes.POINTER(Options), vp,
                                   ctypes.POINTER(vp)]
    L.ersj_set_queries.argtypes = [vp, vp, i64, i64, vp]
    L.ersj_count_pass.argtypes = [vp, ctypes.POINTER(u64), vp]
    L.ersj_plan_batches.argtypes = [vp, u64, ctypes.POINTER(i32), vp]
    L.ersj_fill_pass.argtypes = [vp, i32, vp, u64, ctypes.POINTER(u64), vp]
    L.ersj_fill_pass_host.argtypes = [vp, i32, vp, u64, ctypes.POINTER(u64), vp]
    L.ersj_fill_pass_noalloc.argtypes = [vp, i32, vp, u64, ctypes.POINTER(u64), vp]
    L.ersj_host_sync.argtypes = [vp]
    L.ersj_batch_info.argtypes = [vp, i32, ctypes.POINTER(u64), ctypes.POINTER(u64),
                                  ctypes.POINTER(u64)]
    L.ersj_get_stats.argtypes = [vp, ctypes.POINTER(Stats)]
    L.ersj_free.argtypes = [vp]
    L.ersj_release_cached.argtypes = [i32, ctypes.POINTER(u64)]
    L.ersj_knn.argtypes = [vp, i64, i32, i64, vp, i64, i64, i32, dbl, dbl, ctypes.POINTER(Options),
                           vp, vp, ctypes.POINTER(KnnInfo), vp]
    L.ersj_free.restype = None
    L.ersj_last_error.argtypes = []
    L.ersj_last_error.restype = ctypes.c_char_p
    for f in ("ersj_build_index", "ersj_set_queries", "ersj_count_pass", "ersj_plan_batches",
              "ersj_fill_pass", "ersj_fill_pass_host", "ersj_fill_pass_noalloc", "ersj_host_sync",
              "ersj_batch_info",
              "ersj_get_stats"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def _check(rc):
    if rc != OK:
        raise ErsjError(rc, lib().ersj_last_error().decode(errors="replace"))


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def default_options(**kw) -> Options:
    o = Options()
    lib().ersj_default_options(ctypes.byref(o))
    for k, v in kw.items():
        setattr(o, k, v)
    return o


class Index:
    """Owner of an ``ersj_index*``; ``free()`` (or garbage collection) releases it."""

    def __init__(self, handle, n, d):
        self.handle = ctypes.c_void_p(handle)
        self.n, self.d = n, d

    def free(self):
        if self.handle and self.handle.value:
            lib().ersj_free(self.handle)
            self.handle = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def build_index(x: torch.Tensor, eps: float, options: Options = None, stream=None) -> Index:
    """``ersj_build_index`` on a float32 [n, d] CUDA tensor (rows may be strided)."""
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.dim() != 2:
        raise TypeError("x must be a 2-D torch.float32 tensor")
    if not x.is_cuda:
        raise TypeError("x must live on the GPU")
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous (stride(1) == 1)")
    n, d = x.shape
    out = ctypes.c_void_p()
    opt = ctypes.byref(options) if options is not None else None
    _check(lib().ersj_build_index(ctypes.c_void_p(x.data_ptr()), n, d, x.stride(0), float(eps), opt,
                                  _stream(stream), ctypes.byref(out)))
    return Index(out.value, n, d)


def _rows_tensor(x, what):
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or x.dim() != 2:
        raise TypeError(f"{what} must be a 2-D torch.float32 tensor")
    if not x.is_cuda:
        raise TypeError(f"{what} must live on the GPU")
    if x.stride(1) != 1:
        raise ValueError(f"{what} rows must be contiguous (stride(1) == 1)")


def set_queries(h: Index, q: torch.Tensor, stream=None):
    """``ersj_set_queries``: make the float32 [nq, d] CUDA tensor ``q`` the query
    rows of a semi-join against the indexed points."""
    _rows_tensor(q, "q")
    if q.shape[1] != h.d:
        raise ValueError(f"q has {q.shape[1]} columns, the index {h.d}")
    _check(lib().ersj_set_queries(h.handle, ctypes.c_void_p(q.data_ptr()), q.shape[0], q.stride(0),
                                  _stream(stream)))


def count_pass(h: Index, stream=None) -> int:
    total = ctypes.c_uint64()
    _check(lib().ersj_count_pass(h.handle, ctypes.byref(total), _stream(stream)))
    return total.value


def plan_batches(h: Index, budget_bytes: int = 0, stream=None) -> int:
    nb = ctypes.c_int32()
    _check(lib().ersj_plan_batches(h.handle, int(budget_bytes), ctypes.byref(nb), _stream(stream)))
    return nb.value


def _capacity_error(rc: int, required: int) -> ErsjError:
    # built here, not in the raising frame: an exception held in a local of
    # the frame that raises it forms a reference cycle through its traceback,
    # which would keep the caller's frames (and their output tensors) alive
    # until the garbage collector runs
    err = ErsjError(rc, lib().ersj_last_error().decode(errors="replace"))
    err.required = required
    return err


def fill_pass(h: Index, batch: int, pairs: torch.Tensor = None, capacity: int = None,
              stream=None) -> int:
    """Run ``ersj_fill_pass``; returns the batch's pair count.

    ``pairs`` is an int32 CUDA tensor viewed as [capacity, 2] uint32 ids.
    Raises ErsjError(CAPACITY) with ``.required`` when it is too small.
    """
    npairs = ctypes.c_uint64()
    if pairs is None:
        ptr, cap = None, 0
    else:
        if pairs.dtype != torch.int32 or not pairs.is_cuda or not pairs.is_contiguous():
            raise TypeError("pairs must be a contiguous int32 CUDA tensor")
        ptr = ctypes.c_void_p(pairs.data_ptr())
        cap = pairs.numel() // 2 if capacity is None else int(capacity)
        if cap * 2 > pairs.numel():
            raise ValueError("capacity exceeds the tensor")
    rc = lib().ersj_fill_pass(h.handle, int(batch), ptr, cap, ctypes.byref(npairs), _stream(stream))
    if rc == ERR_CAPACITY:
        raise _capacity_error(rc, npairs.value)
    _check(rc)
    return npairs.value


def fill_pass_noalloc(h: Index, batch: int, pairs: torch.Tensor = None, capacity: int = None,
                      stream=None) -> int:
    """``ersj_fill_pass_noalloc``: ``fill_pass`` with the batch's working memory
    taken from the library's fixed device scratch (no device allocation).
    Raises ErsjError(SCRATCH) when the batch does not fit it, and
    ErsjError(CAPACITY) with ``.required`` when ``pairs`` is too small."""
    npairs = ctypes.c_uint64()
    if pairs is None:
        ptr, cap = None, 0
    else:
        if pairs.dtype != torch.int32 or not pairs.is_cuda or not pairs.is_contiguous():
            raise TypeError("pairs must be a contiguous int32 CUDA tensor")
        ptr = ctypes.c_void_p(pairs.data_ptr())
        cap = pairs.numel() // 2 if capacity is None else int(capacity)
        if cap * 2 > pairs.numel():
            raise ValueError("capacity exceeds the tensor")
    rc = lib().ersj_fill_pass_noalloc(h.handle, int(batch), ptr, cap, ctypes.byref(npairs), _stream(stream))
    if rc == ERR_CAPACITY:
        raise _capacity_error(rc, npairs.value)
    _check(rc)
    return npairs.value


def fill_pass_host(h: Index, batch: int, pairs: torch.Tensor = None, capacity: int = None,
                   stream=None) -> int:
    """``ersj_fill_pass_host``: refine batch ``batch`` and start copying its pairs
    into ``pairs``, an int32 CPU tensor (pinned for an asynchronous copy) viewed
    as [capacity, 2] uint32 ids.  The pairs are there after ``host_sync``.
    Raises ErsjError(CAPACITY) with ``.required`` when it is too small."""
    npairs = ctypes.c_uint64()
    if pairs is None:
        ptr, cap = None, 0
    else:
        if pairs.dtype != torch.int32 or pairs.is_cuda or not pairs.is_contiguous():
            raise TypeError("pairs must be a contiguous int32 CPU tensor")
        ptr = ctypes.c_void_p(pairs.data_ptr())
        cap = pairs.numel() // 2 if capacity is None else int(capacity)
        if cap * 2 > pairs.numel():
            raise ValueError("capacity exceeds the tensor")
    rc = lib().ersj_fill_pass_host(h.handle, int(batch), ptr, cap, ctypes.byref(npairs), _stream(stream))
    if rc == ERR_CAPACITY:
        raise _capacity_error(rc, npairs.value)
    _check(rc)
    return npairs.value


def host_sync(h: Index):
    _check(lib().ersj_host_sync(h.handle))


def join_to_host(h: Index, n_batches: int, out: torch.Tensor = None, stream=None):
    """Deliver every batch into host memory, each batch's copy overlapping the
    next batch's refinement.  ``out``: an int32 CPU tensor [capacity, 2],
    pinned, filled batch after batch (allocated, pinned, when None; it must
    hold all pairs).  Returns the [|R|, 2] view of it with the pairs."""
    counts, at = [], 0
    if out is None:
        parts = []
        for b in range(n_batches):
            try:
                m = fill_pass_host(h, b, None, 0, stream)
            except ErsjError as e:
                if e.code != ERR_CAPACITY:
                    raise
                m = e.required
            buf = torch.empty((m, 2), dtype=torch.int32, pin_memory=True)
            if m:
                fill_pass_host(h, b, buf, m, stream)
            parts.append(buf)
        host_sync(h)
        if not parts:
            return torch.empty((0, 2), dtype=torch.int32)
        return parts[0] if len(parts) == 1 else torch.cat(parts)
    for b in range(n_batches):
        view = out[at:]
        m = fill_pass_host(h, b, view, view.shape[0], stream)
        counts.append(m)
        at += m
    host_sync(h)
    return out[:at]


def batch_info(h: Index, batch: int):
    a, b, c = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().ersj_batch_info(h.handle, int(batch), ctypes.byref(a), ctypes.byref(b),
                                 ctypes.byref(c)))
    return a.value, b.value, c.value


def get_stats(h: Index) -> dict:
    st = Stats()
    _check(lib().ersj_get_stats(h.handle, ctypes.byref(st)))
    return st.as_dict()


def free(h: Index):
    h.free()


def release_cached(device: int = -1) -> int:
    """Return the device memory the library keeps for reuse to the HIP runtime;
    the bytes freed."""
    out = ctypes.c_uint64()
    _check(lib().ersj_release_cached(device, ctypes.byref(out)))
    return out.value


def _empty_pairs(m: int, dev):
    # memory the library keeps for reuse is invisible to torch's allocator:
    # give it back once before failing
    try:
        return torch.empty((m, 2), dtype=torch.int32, device=dev)
    except torch.OutOfMemoryError:
        release_cached(dev.index if dev.index is not None else -1)
        return torch.empty((m, 2), dtype=torch.int32, device=dev)


def iter_batches(h: Index, n_batches: int, stream=None):
    """Yield each batch's pairs as an int32 CUDA tensor [m, 2] (uint32 ids)."""
    dev = torch.device("cuda", torch.cuda.current_device())
    for b in range(n_batches):
        try:
            m = fill_pass(h, b, None, 0, stream)
        except ErsjError as e:
            if e.code != ERR_CAPACITY:
                raise
            m = e.required
        out = _empty_pairs(m, dev)
        if m:
            fill_pass(h, b, out, m, stream)
        yield out


def self_join(x: torch.Tensor, eps: float, budget_bytes: int = 0, options: Options = None,
              stream=None, return_index: bool = False):
    """All pairs within eps of the rows of ``x``: list of per-batch [m, 2] int32 tensors."""
    h = build_index(x, eps, options, stream)
    try:
        count_pass(h, stream)
        nb = plan_batches(h, budget_bytes, stream)
        parts = list(iter_batches(h, nb, stream))
    except Exception:
        h.free()
        raise
    if return_index:
        return parts, h
    h.free()
    return parts


def semi_join(q: torch.Tensor, x: torch.Tensor, eps: float, budget_bytes: int = 0,
              options: Options = None, stream=None, return_index: bool = False):
    """All (query row of ``q``, row of ``x``) pairs within eps: list of per-batch
    [m, 2] int32 tensors (RT-HiSS Sec. II-A, the semi-join)."""
    h = build_index(x, eps, options, stream)
    try:
        set_queries(h, q, stream)
        count_pass(h, stream)
        nb = plan_batches(h, budget_bytes, stream)
        parts = list(iter_batches(h, nb, stream))
    except Exception:
        h.free()
        raise
    if return_index:
        return parts, h
    h.free()
    return parts


def knn(x: torch.Tensor, k: int, eps0: float, q: torch.Tensor = None, growth: float = 0.0,
        options: Options = None, stream=None, with_dist: bool = True):
    """Exact k nearest neighbours (``ersj_knn``; RT-HiSS Sec. VI, growing
    similarity searches): for each row of ``q`` (the rows of ``x`` when None),
    the k rows of ``x`` with the smallest canonical binary64 squared distance,
    ties to the smaller row.  Returns (ids int32 [nq, k] holding uint32 row
    numbers, D64 float64 [nq, k] or None, info dict)."""
    _rows_tensor(x, "x")
    nq, ldq, qp = 0, 0, None
    if q is not None:
        _rows_tensor(q, "q")
        if q.shape[1] != x.shape[1]:
            raise ValueError(f"q has {q.shape[1]} columns, x {x.shape[1]}")
        nq, ldq, qp = q.shape[0], q.stride(0), ctypes.c_void_p(q.data_ptr())
    rows = nq if q is not None else x.shape[0]
    ids = torch.empty((rows, int(k)), dtype=torch.int32, device=x.device)
    dist = torch.empty((rows, int(k)), dtype=torch.float64, device=x.device) if with_dist else None
    info = KnnInfo()
    _check(lib().ersj_knn(ctypes.c_void_p(x.data_ptr()), x.shape[0], x.shape[1], x.stride(0), qp, nq, ldq,
                          int(k), float(eps0), float(growth),
                          ctypes.byref(options) if options is not None else None,
                          ctypes.c_void_p(ids.data_ptr()),
                          ctypes.c_void_p(dist.data_ptr()) if dist is not None else None,
                          ctypes.byref(info), _stream(stream)))
    return ids, dist, info.as_dict()


def pairs_to_numpy(parts):
    """Concatenate per-batch tensors into a host uint32 [|R|, 2] array."""
    import numpy as np
    if not parts:
        return np.zeros((0, 2), dtype=np.uint32)
    arrs = [p.cpu().numpy().view(np.uint32) for p in parts]
    return np.concatenate(arrs, axis=0) if len(arrs) > 1 else arrs[0]
