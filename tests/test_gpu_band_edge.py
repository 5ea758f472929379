"""Pairs placed at the edges of the refinement kernels' bands.

Every refinement kernel decides a pair from a rounded squared distance and
sends it to the binary64 re-check when that value is within its error bound
of the threshold; outside the bound it decides alone.  A bound that is too
narrow would show as a pair just outside it decided the wrong way.  Here
pairs are built at squared distance fl(eps^2) (1 + m w) for m in +-0.5,
+-1, +-2, +-4 and for the half-width w of each kernel:

* split-fp16 MFMA form: K16 (Nq + Nx) / E, with K16 = 4 (d_pad + 8) u +
  3 * 2^-22 + 36 u * 3 * ceil(d_pad / 16) * 1.01;
* its high-parts-only form (above 64 dimensions): Khh (Nq + Nx) / E, with
  Khh = 4 (d_pad + 8) u + 2^-10 (1 + 2^-12) + 36 u * 2 ceil(ns / 2) * 1.01,
  ns = ceil(d_pad / 16);
* fp32 MFMA form: K32 (Nq + Nx) / E, with K32 = 4 (d_pad + 8) u;
* direct form: 2 (gamma(d_pad + 2) at u = 2^-24 + gamma(d + 2) at 2^-53),

where Nq and Nx are the squared norms of the query and the candidate about
the reference point (the row tile's up to 64 dimensions, the mean of all
points above; the cases above 64 dimensions place every point around one
centre, so that the two are close).  The pairs lie far from that point (the tile
is mostly a tight cluster near the origin of dimensions 3..d-1, the pairs
sit at about 1.2 eps from it in every one of those dimensions, with random
signs), so Nq + Nx is about 100 E and the distance comes out of a dot
product with heavy cancellation.  One case adds a large common offset, so
that the absolute part of the split form's bound matters too.  Each kernel
must return exactly the oracle's pair set (the result of "RT-HiSS: Ray
Tracing Accelerated High Dimensional Vector Similarity Searches",
Sec. II-A)."""
import math

import numpy as np
import pytest
import torch

import exact_range_similarity_amd as ersj
import oracle

from gpu_util import KERNELS, assert_same_pairs, gpu_pairs, say

pytestmark = pytest.mark.gpu
U32, U64 = 2.0 ** -24, 2.0 ** -53


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ersj.lib()


def gamma(n, u):
    return n * u / (1 - n * u)


def widths(d, phi):
    """Half-widths (relative to E) of the kernels' bands for Nq + Nx = phi E."""
    nb = (d + 3) // 4
    dpad = 4 * nb
    nslab = (nb + 3) // 4
    k32 = 4 * (dpad + 8) * U32
    k16 = k32 + 3 * 2.0 ** -22 + 36 * U32 * 3 * nslab * 1.01
    khh = k32 + 2.0 ** -10 * (1 + 2.0 ** -12) + 36 * U32 * 2 * ((nslab + 1) // 2) * 1.01
    direct = 2 * (gamma(dpad + 2, U32) + gamma(d + 2, U64))
    return {"mfma16": k16 * phi, "mfma16_hh": khh * phi, "mfma": k32 * phi, "direct": direct}


MULTS = (-4, -2, -1, -0.5, 0.5, 1, 2, 4)


def build(d, offset, seed, cells=12, home=96, eps=0.25, phi=100.0):
    rng = np.random.default_rng(seed)
    E = eps * eps
    F = math.sqrt(phi / 2 * E / (d - 3))   # |q - r|^2 ~ |x - r|^2 ~ phi E / 2
    w = widths(d, phi)
    rows, targets = [], []
    for c in range(cells):
        corner = np.array([5.0 * eps * c, 5.0 * eps * ((7 * c) % cells), 5.0 * eps * ((5 * c) % cells)])
        H = np.zeros((home, d))
        H[:, :3] = corner + rng.random((home, 3)) * 0.3 * eps
        H[:, 3:] = rng.normal(0.0, 0.02 * eps, (home, d - 3))
        rows.append(H)
        for kern, wk in w.items():
            for m in MULTS:
                q = np.zeros(d)
                q[:3] = corner + rng.random(3) * 0.3 * eps
                q[3:] = F * rng.choice((-1.0, 1.0), d - 3) + rng.normal(0.0, 0.01 * eps, d - 3)
                v = rng.normal(0.0, 1.0, d)
                v[:3] *= 0.1
                v *= math.sqrt(E * (1 + m * wk)) / np.linalg.norm(v)
                rows.append(np.stack([q, q + v]))
                targets.append((kern, m))
    X = (np.concatenate(rows) + offset).astype(np.float32)
    return X, eps, targets, home


@pytest.mark.parametrize("d,offset,cells", [(18, 0.0, 12), (40, 0.0, 12), (40, 64.0, 12), (100, 0.0, 12),
                                            (100, 0.0, 1), (129, 0.0, 1), (384, 0.0, 1)])
def test_pairs_at_the_band_edges(d, offset, cells):
    X, eps, targets, home = build(d, offset, seed=d + int(offset) + cells, cells=cells)
    E = oracle.e64(eps)
    w = widths(d, 100.0)
    kinds = len(w)
    # where the constructed pairs landed, in units of each kernel's half-width
    per_cell = home + 2 * kinds * len(MULTS)
    hit = {k: 0 for k in w}
    for c in range(cells):
        base = c * per_cell + home
        for t in range(kinds * len(MULTS)):
            kern, m = targets[c * kinds * len(MULTS) + t]
            i = base + 2 * t
            rel = (oracle.d64(X[i], X[i + 1]) - E) / E
            if 0.25 * abs(m) <= abs(rel) / w[kern] <= 2 * abs(m) and math.copysign(1, rel) == math.copysign(1, m):
                hit[kern] += 1
    say(f"[gpu] band edges d={d} offset={offset}: n={X.shape[0]} pairs placed within 2x of target: {hit}")
    # (with the large offset, fp32 coordinates cannot resolve the direct
    # form's width: its pairs land anywhere within a few E 1e-5 of E)
    need = [k for k in w if offset == 0.0 or k != "direct"]
    assert all(hit[k] >= cells * len(MULTS) // 2 for k in need), hit
    want = oracle.selfjoin_pairs(X, eps)
    runs = [(k, 0) for k in KERNELS]
    if d > 64:
        runs.append((ersj.REFINE_MFMA16, 3))  # the three-product form beside the default
    for k, products in runs:
        opts = ersj.default_options(refine_kernel=k, mfma_products=products)
        try:
            got = gpu_pairs(X, eps, options=opts)
        except ersj.ErsjError as e:
            # the fp32 MFMA form does not take every width (its query tile
            # must fit the LDS); the split form and the direct form always run
            assert k == ersj.REFINE_MFMA and e.code == ersj.ERR_INVALID_ARG, e
            say(f"[gpu] d={d}: kernel {k} not usable here: {e}")
            continue
        say(f"[gpu] band edges d={d} offset={offset} cells={cells} kernel={k} products={products}: "
            f"{len(got)} pairs")
        assert_same_pairs(X, eps, got, want, f"band edges d={d} offset={offset} kernel={k} products={products}")
