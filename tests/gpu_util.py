"""Helpers shared by the GPU tests: run the HIP path, compare pair sets."""
import sys

import numpy as np
import torch

import exact_range_similarity_amd as ersj
import oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def keys_of(P):
    P = np.asarray(P, dtype=np.uint32)
    return (P[:, 0].astype(np.uint64) << np.uint64(32)) | P[:, 1].astype(np.uint64)


def gpu_pairs(X, eps, budget=0, options=None, ld=None):
    """Pairs from the HIP path for host array X (copied to the GPU)."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    if ld is not None and ld != X.shape[1]:
        buf = np.zeros((X.shape[0], ld), dtype=np.float32)
        buf[:, :X.shape[1]] = X
        xt = torch.from_numpy(buf).cuda()[:, :X.shape[1]]
    else:
        xt = torch.from_numpy(X).cuda()
    parts = ersj.self_join(xt, eps, budget, options)
    torch.cuda.synchronize()
    return ersj.pairs_to_numpy(parts)


def assert_same_pairs(X, eps, got, want, label=""):
    kg = keys_of(got)
    kw = keys_of(want)
    sg = np.sort(kg)
    assert np.unique(sg).size == sg.size, f"{label}: duplicate pairs in GPU output"
    sw = np.sort(kw)
    if sg.size == sw.size and np.array_equal(sg, sw):
        return
    extra = np.setdiff1d(sg, sw)[:10]
    missing = np.setdiff1d(sw, sg)[:10]
    e2 = oracle.e64(eps)
    lines = []
    for tag, arr in (("extra", extra), ("missing", missing)):
        for k in arr:
            i, j = int(k >> np.uint64(32)), int(k & np.uint64(0xffffffff))
            d = oracle.d64(X[i], X[j])
            lines.append(f"{tag} ({i},{j}) D64={d!r} E64={e2!r} rel={(d - e2) / e2 if e2 else d}")
    raise AssertionError(f"{label}: |gpu|={sg.size} |oracle|={sw.size}\n" + "\n".join(lines))


KERNELS = (ersj.REFINE_DIRECT, ersj.REFINE_MFMA, ersj.REFINE_MFMA16)


def check_against_oracle(X, eps, label="", kernels=KERNELS, **kw):
    """Both refinement kernels must return exactly the oracle's pair set."""
    want = oracle.selfjoin_pairs(X, eps)
    got = None
    base = kw.pop("options", None)
    for k in kernels:
        say(f"[gpu] {label}: n={X.shape[0]} d={X.shape[1]} eps={eps!r} kernel={k}")
        opts = ersj.Options.from_buffer_copy(base) if base is not None else ersj.default_options()
        opts.refine_kernel = k
        got = gpu_pairs(X, eps, options=opts, **kw)
        assert_same_pairs(X, eps, got, want, f"{label} kernel={k}")
    return got
