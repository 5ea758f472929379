"""C ABI checks that need no GPU: the library loads, exports every entry point
of include/ersj.h, and rejects bad arguments before making any HIP call."""
import ctypes
import math
import os
import re

import pytest

import exact_range_similarity_amd as ersj

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "ersj.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(ersj_[a-z_]+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert set(header_functions()) == set(ersj.SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = ersj.lib()
    for name in header_functions():
        assert hasattr(L, name), name


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def build(ptr=FAKE, n=10, d=4, ld=4, eps=1.0, opt=None):
    out = ctypes.c_void_p(12345)
    rc = ersj.lib().ersj_build_index(ptr, n, d, ld, eps, opt, None, ctypes.byref(out))
    return rc, out


@pytest.mark.parametrize("kw", [
    dict(ptr=ctypes.c_void_p(None)), dict(n=0), dict(n=-5), dict(n=2 ** 32), dict(d=0),
    dict(d=4097), dict(ld=3), dict(eps=-1.0), dict(eps=float("nan")), dict(eps=-math.inf),
])
def test_build_rejects_bad_arguments(kw):
    rc, out = build(**kw)
    assert rc == ersj.ERR_INVALID_ARG
    assert out.value is None
    assert ersj.lib().ersj_last_error().decode()


def test_build_rejects_bad_options():
    o = ersj.default_options()
    assert o.struct_size == ctypes.sizeof(ersj.Options)
    o.refine_kernel = 9
    assert build(opt=ctypes.byref(o))[0] == ersj.ERR_INVALID_ARG
    o = ersj.default_options(struct_size=3)
    assert build(opt=ctypes.byref(o))[0] == ersj.ERR_INVALID_ARG
    o = ersj.default_options(cell_width_scale=float("nan"))
    assert build(opt=ctypes.byref(o))[0] == ersj.ERR_INVALID_ARG
    for reach in (-1, 3):
        o = ersj.default_options(grid_reach=reach)
        assert build(opt=ctypes.byref(o))[0] == ersj.ERR_INVALID_ARG
    for order in (-1, 4):
        o = ersj.default_options(cell_order=order)
        assert build(opt=ctypes.byref(o))[0] == ersj.ERR_INVALID_ARG
        assert "cell_order" in ersj.lib().ersj_last_error().decode()
    for products in (-1, 2, 4):
        o = ersj.default_options(mfma_products=products)
        assert build(opt=ctypes.byref(o))[0] == ersj.ERR_INVALID_ARG
        assert "mfma_products" in ersj.lib().ersj_last_error().decode()


def test_null_handle_paths():
    L = ersj.lib()
    u = ctypes.c_uint64()
    i = ctypes.c_int32()
    assert L.ersj_count_pass(None, ctypes.byref(u), None) == ersj.ERR_INVALID_ARG
    assert L.ersj_plan_batches(None, 0, ctypes.byref(i), None) == ersj.ERR_INVALID_ARG
    assert L.ersj_fill_pass(None, 0, None, 0, ctypes.byref(u), None) == ersj.ERR_INVALID_ARG
    assert L.ersj_fill_pass_noalloc(None, 0, None, 0, ctypes.byref(u), None) == ersj.ERR_INVALID_ARG
    assert L.ersj_batch_info(None, 0, None, None, None) == ersj.ERR_INVALID_ARG
    assert L.ersj_get_stats(None, None) == ersj.ERR_INVALID_ARG
    assert L.ersj_set_queries(None, FAKE, 10, 4, None) == ersj.ERR_INVALID_ARG
    L.ersj_free(None)


@pytest.mark.parametrize("kw", [
    dict(x=None), dict(ids=None), dict(n=0), dict(d=0), dict(ld=2), dict(k=0), dict(k=11),
    dict(k=1025, n=2000), dict(eps0=0.0), dict(eps0=-1.0), dict(eps0=float("nan")),
    dict(growth=1.0), dict(growth=0.5), dict(growth=float("inf")), dict(q=FAKE, nq=0),
    dict(q=FAKE, nq=5, ldq=2),
])
def test_knn_rejects_bad_arguments(kw):
    a = dict(x=FAKE, n=10, d=3, ld=3, q=None, nq=0, ldq=0, k=3, eps0=1.0, growth=0.0, ids=FAKE)
    a.update(kw)
    info = ersj.KnnInfo()
    rc = ersj.lib().ersj_knn(a["x"], a["n"], a["d"], a["ld"], a["q"], a["nq"], a["ldq"], a["k"],
                             a["eps0"], a["growth"], None, a["ids"], None, ctypes.byref(info), None)
    assert rc == ersj.ERR_INVALID_ARG
    assert ersj.lib().ersj_last_error()


def test_release_cached_rejects_a_missing_device():
    L = ersj.lib()
    out = ctypes.c_uint64(7)
    assert L.ersj_release_cached(-2, ctypes.byref(out)) == ersj.ERR_INVALID_ARG
    assert out.value == 0
    assert L.ersj_release_cached(1 << 20, None) == ersj.ERR_INVALID_ARG
    assert "not a HIP device" in L.ersj_last_error().decode()


def test_error_message_is_per_call():
    rc, _ = build(d=0)
    assert rc == ersj.ERR_INVALID_ARG
    assert "d = 0" in ersj.lib().ersj_last_error().decode()


def test_hip_failure_without_a_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this checks the no-device error path")
    rc, out = build()
    assert rc in (ersj.ERR_HIP, ersj.ERR_OOM)
    assert out.value is None


def test_capacity_error_leaves_no_reference_cycle(monkeypatch):
    # A CAPACITY result raises ErsjError with .required; the exception must
    # not form a cycle that keeps the caller's frame (and the output tensors
    # it holds) alive until a garbage collection.
    import gc
    import weakref

    class FakeLib:
        def ersj_fill_pass(self, handle, batch, ptr, cap, npairs_ref, stream):
            npairs_ref._obj.value = 12345
            return ersj.ERR_CAPACITY

        def ersj_last_error(self):
            return b"capacity"

    class FakeIndex:
        handle = None

    class Sentinel:
        pass

    monkeypatch.setattr(ersj, "lib", lambda: FakeLib())
    monkeypatch.setattr(ersj, "_stream", lambda stream: None)

    def caller():
        held = Sentinel()
        ref = weakref.ref(held)
        try:
            ersj.fill_pass(FakeIndex(), 0, None, 0)
        except ersj.ErsjError as e:
            assert e.code == ersj.ERR_CAPACITY and e.required == 12345
        return ref

    gc.disable()
    try:
        ref = caller()
        assert ref() is None
    finally:
        gc.enable()
