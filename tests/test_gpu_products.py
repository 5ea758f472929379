"""The split-fp16 form above 64 dimensions with one or three products per slab.

The high-parts-only form (mfma_products = 1, the default there) sums the
high-half products alone and widens its band by the dropped terms' bound;
the three-product form (3) keeps hi.lo and lo.hi.  Both must return exactly
the oracle's pair set (RT-HiSS Sec. II-A), for the self-join and the
semi-join, on an odd slab count (a zero-padded slab), ragged sizes and the
d = 384 workload's shape; the wider band sends at least as many pairs to the
binary64 re-check.  The partial test (a 32 x 32 block whose pairs are all
farther than the band over the first 64 dimensions of the variance order is
settled there) is checked with pairs whose difference lies in those 64
dimensions alone, at the band's edges.""" 
import math

import numpy as np
import pytest
import torch

import exact_range_similarity_amd as ersj
import oracle
from workloads import make_config, make_queries

from gpu_util import assert_same_pairs, keys_of, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ersj.lib()


def _join_stats(X, eps, products, bits=0):
    opts = ersj.default_options(refine_kernel=ersj.REFINE_MFMA16, mfma_products=products, filter_bits=bits)
    h = ersj.build_index(torch.from_numpy(X).cuda(), eps, opts)
    ersj.count_pass(h)
    nb = ersj.plan_batches(h, 0)
    parts = list(ersj.iter_batches(h, nb))
    st = ersj.get_stats(h)
    h.free()
    return ersj.pairs_to_numpy(parts), st


@pytest.mark.parametrize("bits", [8, 16])
@pytest.mark.parametrize("name,n,d", [("c5", 6000, None), ("rand", 3001, 129), ("rand", 700, 68),
                                      ("rand", 1500, 200)])
def test_both_forms_match_the_oracle(name, n, d, bits):
    if name == "rand":
        rng = np.random.default_rng(n + d)
        X = rng.random((n, d), dtype=np.float32)
        eps = 0.33 * math.sqrt(d / 6.0)
    else:
        X = make_config(name, n)
        eps, _, _ = oracle.calibrate_eps(X, min(1000, n), 50)
    want = oracle.selfjoin_pairs(X, eps)
    band = {}
    for products in (1, 3):
        say(f"[gpu] products={products} {name} n={n} d={X.shape[1]} eps={eps!r}")
        got, st = _join_stats(X, eps, products, bits)
        assert st["mfma_products"] == products and st["filter_bits"] == bits
        assert_same_pairs(X, eps, got, want, f"{name} products={products}")
        band[products] = st["last_boundary_pairs"]
        say(f"[gpu] {name} products={products}: {st['last_partial']} comparisons settled from the first "
            f"64 dimensions")
        if name == "c5":  # clusters far apart: most blocks are settled early
            assert st["last_partial"] > 0
    say(f"[gpu] {name}: band pairs {band}")
    assert band[1] >= band[3]


def test_default_is_high_parts_above_64_dimensions():
    rng = np.random.default_rng(5)
    for d, expect in ((64, 3), (65, 1), (384, 1)):
        X = rng.random((300, d), dtype=np.float32)
        h = ersj.build_index(torch.from_numpy(X).cuda(), 0.5,
                             ersj.default_options(refine_kernel=ersj.REFINE_MFMA16))
        st = ersj.get_stats(h)
        h.free()
        assert st["mfma_products"] == expect, (d, st["mfma_products"])


@pytest.mark.parametrize("products", [1, 3])
@pytest.mark.parametrize("nq,n,d", [(600, 900, 100), (257, 1300, 133)])
def test_semi_join_both_forms(nq, n, d, products):
    rng = np.random.default_rng(nq + n + d)
    X = rng.random((n, d), dtype=np.float32)
    Q = np.concatenate([rng.random((nq - 40, d), dtype=np.float32),
                        X[:40] + np.float32(0.01)])
    eps = 0.33 * math.sqrt(d / 6.0)
    want = np.sort(keys_of(oracle.semijoin_pairs(Q, X, eps)))
    opts = ersj.default_options(refine_kernel=ersj.REFINE_MFMA16, mfma_products=products)
    parts = ersj.semi_join(torch.from_numpy(Q).cuda(), torch.from_numpy(X).cuda(), eps, 0, opts)
    got = np.sort(keys_of(ersj.pairs_to_numpy(parts)))
    say(f"[gpu] semi-join products={products} nq={nq} n={n} d={d}: {got.size} pairs")
    assert np.array_equal(got, want)


def test_c5_shape_semijoin_queries_from_the_same_centres():
    X = make_config("c5", 5000)
    Q = make_queries("c5", 1500, 9, 5000)
    eps, _, _ = oracle.calibrate_eps(X, 1000, 50)
    want = np.sort(keys_of(oracle.semijoin_pairs(Q, X, eps)))
    for products in (1, 3):
        opts = ersj.default_options(refine_kernel=ersj.REFINE_MFMA16, mfma_products=products)
        parts = ersj.semi_join(torch.from_numpy(Q).cuda(), torch.from_numpy(X).cuda(), eps, 0, opts)
        got = np.sort(keys_of(ersj.pairs_to_numpy(parts)))
        assert np.array_equal(got, want), products


@pytest.mark.parametrize("bits", [8, 16])
@pytest.mark.parametrize("products", [1, 3])
def test_partial_test_with_differences_in_the_leading_dimensions(products, bits):
    # dimensions 0..63 spread widely (they lead the variance order), the rest
    # nearly constant; each pair differs in dimensions 0..63 only, so its
    # distance over them is its full distance, placed around eps^2 at
    # relative offsets from 1e-6 to 1e-1 on both sides
    rng = np.random.default_rng(77 + products)
    d, eps = 100, 0.5
    E = eps * eps
    base = np.zeros((3000, d))
    base[:, :64] = rng.random((3000, 64)) * 4.0
    base[:, 64:] = rng.normal(0.0, 0.01, (3000, d - 64))
    rows = [base]
    for rel in (1e-6, 1e-5, 1e-4, 1e-3, 3e-3, 1e-2, 1e-1):
        for sgn in (-1.0, 1.0):
            for _ in range(6):
                q = base[rng.integers(0, 3000)].copy()
                v = np.zeros(d)
                v[:64] = rng.normal(0.0, 1.0, 64)
                v *= np.sqrt(E * (1.0 + sgn * rel)) / np.linalg.norm(v)
                rows.append(np.stack([q, q + v]))
    X = np.concatenate(rows).astype(np.float32)
    want = oracle.selfjoin_pairs(X, eps)
    got, st = _join_stats(X, eps, products, bits)
    say(f"[gpu] leading-dimension pairs products={products} filter bits={bits}: {len(got)} pairs, "
        f"{st['last_partial']} comparisons settled from the first 64 dimensions")
    assert st["last_partial"] > 0 and st["filter_bits"] == bits
    assert_same_pairs(X, eps, got, want, f"leading-dimension pairs products={products} bits={bits}")


def test_dense_steps_continue_in_place():
    # about a tenth of all pairs are neighbours, so nearly every 32 x 32
    # block is still live after the first 64 dimensions: a step with more
    # live blocks than it may hand to the second kernel finishes them itself
    rng = np.random.default_rng(91)
    n, d = 12000, 96
    X = rng.random((n, d), dtype=np.float32)
    eps, _, _ = oracle.calibrate_eps(X, 500, 1200)
    want = oracle.selfjoin_pairs(X, eps)
    for products in (1, 3):
        got, st = _join_stats(X, eps, products)
        say(f"[gpu] dense d={d} products={products}: {len(got)} pairs, {st['last_partial']} settled early")
        assert_same_pairs(X, eps, got, want, f"dense d={d} products={products}")


def test_more_live_blocks_than_the_hand_on_list_holds():
    # equal spread in all 160 dimensions and a radius for a few neighbours
    # per point: the distance over the first 64 dimensions settles almost no
    # block, so the 1.2 M blocks of this join overflow the hand-on list
    # (2^20 entries at this size) and the batch is refined again by the
    # tiled kernel
    rng = np.random.default_rng(97)
    n, d = 36000, 160
    X = rng.random((n, d), dtype=np.float32)
    eps, _, _ = oracle.calibrate_eps(X, 300, 4)
    want = oracle.selfjoin_pairs(X, eps)
    got, st = _join_stats(X, eps, 0)
    say(f"[gpu] overflowing hand-on list n={n} d={d}: {len(got)} pairs, {st['last_partial']} settled early")
    assert_same_pairs(X, eps, got, want, f"overflowing hand-on list n={n} d={d}")


def _coherent_semijoin_case(seed=3):
    # Every coordinate of the first 64 dimensions is 4 m + 1.75 or 4 m + 2.25
    # (m an integer, 1024 <= m < 2048) after the kernels' scaling by 2^14
    # (the largest magnitude, below 0.5, sets that scale; the points are
    # mirrored so that their mean, the reference, is exactly 0).  fp16 has
    # spacing 4 there, so every high half rounds down by 1.75 (or up by
    # 1.75) in all 64 dimensions of both rows of a pair: the dropped
    # low-half products add up instead of cancelling, and the high-half dot
    # product is off by about 0.6 E, most of the high-half band 2^-10 (Nq + Nx)
    # and far beyond the three-product band.  Each query has one partner, at
    # S = E (1 + rho) for rho from -0.3 to 0.3; a semi-join, so that no
    # zero-distance self pair keeps a block live.
    rng = np.random.default_rng(seed)
    d, scale, Es = 100, 16384.0, 4.0e6
    Q, X = [], []
    for off in (1.75, 2.25):
        for rho in (-0.3, -0.1, -0.03, -0.01, -0.001, 0.001, 0.01, 0.03, 0.1, 0.3):
            a = rng.integers(0, 600, 64)
            base = rng.random(64) + 0.5
            j = np.round(math.sqrt(Es * (1 + rho) / 16 / np.sum(base ** 2)) * base).astype(np.int64)
            q, x = np.zeros(d), np.zeros(d)
            q[:64] = (4 * (1024 + a) + off) / scale
            x[:64] = (4 * (1024 + a + j) + off) / scale
            Q.append(q)
            X.append(x)
    Q = np.array(Q, dtype=np.float32)
    X = np.array(X, dtype=np.float32)
    assert np.abs(X).max() < 0.5 and np.abs(Q).max() < 0.5 and np.abs(X).max() >= 0.25
    Q = np.concatenate([Q, -Q])
    X = np.concatenate([X, -X])
    return Q, X, math.sqrt(Es) / scale


@pytest.mark.parametrize("products", [1, 3])
@pytest.mark.parametrize("tiled", [False, True])
def test_high_halves_that_all_round_one_way(products, tiled):
    Q, X, eps = _coherent_semijoin_case()
    want = np.sort(keys_of(oracle.semijoin_pairs(Q, X, eps)))
    assert want.size == 20  # the ten pairs below eps and their mirror images
    # a device-memory cap keeps the hand-on list unallocated: the tiled kernel
    opts = ersj.default_options(refine_kernel=ersj.REFINE_MFMA16, mfma_products=products,
                                max_device_bytes=(1 << 34) if tiled else 0)
    parts, h = ersj.semi_join(torch.from_numpy(Q).cuda(), torch.from_numpy(X).cuda(), eps, 0, opts,
                              return_index=True)
    st = ersj.get_stats(h)
    h.free()
    got = np.sort(keys_of(ersj.pairs_to_numpy(parts)))
    say(f"[gpu] coherent rounding products={products} tiled={tiled}: {got.size} pairs, "
        f"filtered={st['last_filtered']}, band pairs {st['last_boundary_pairs']}")
    assert st["last_filtered"] == (0 if tiled else 1)
    assert np.array_equal(got, want)


def _int8_coherent_case(f, rhos, seed=5):
    # The int8 filter centres on the mean (exactly 0: the points are
    # mirrored) and scales by S = 127 / (M (1 + 2^-20)), M the largest
    # coordinate of the first 64 dimensions.  Every such coordinate here is
    # (a_i + f) / S with a_i an integer: each rounds to a_i, off by f / S
    # in the same direction in all 64 dimensions of both rows of a pair, so
    # the dropped parts add up and the test's bound is nearly tight.  One
    # partner per query, differing in those dimensions by integer steps j_i,
    # at S^2 |x - q|^2 = sum j_i^2 around E S^2 (1 + rho), every pair of a case
    # at one rho, so that a block holding a pair just inside the radius holds
    # no other kind; a semi-join, so no self pair keeps a block live.  Pairs
    # of different queries lie about 1.8 E apart, mirror images far apart.
    # Dimensions 64..99 are 0.
    rng = np.random.default_rng(seed)
    d, M = 100, np.float32(0.4375)
    S = 127.0 / (float(M) * (1.0 + 2.0 ** -20))
    eps = 0.5
    E = eps * eps
    Q, X = [], []
    for rho in rhos:
        for _ in range(40):
            a = rng.integers(10, 50, 64)  # one sign: the rounding errors' products add up too
            j = rng.normal(0.0, 1.0, 64)
            j = np.round(j * math.sqrt(E * S * S * (1 + rho) / np.sum(j * j))).astype(np.int64)
            j = np.clip(j, -100 - a, 110 - a)
            q, x = np.zeros(d), np.zeros(d)
            q[:64] = (a + f) / S
            x[:64] = (a + j + f) / S
            Q.append(q)
            X.append(x)
    edge = np.zeros(d)
    edge[0] = M  # sets the scale
    Q, X = np.array(Q + [edge]), np.array(X + [edge])
    Q = np.concatenate([Q, -Q]).astype(np.float32)
    X = np.concatenate([X, -X]).astype(np.float32)
    assert np.abs(Q).max() == M and np.abs(X).max() == M
    return Q, X, eps


@pytest.mark.parametrize("rho", [-0.05, -0.01, -0.002, 0.3])
@pytest.mark.parametrize("f", [0.499, -0.499, 0.25])
def test_int8_filter_with_rounding_all_one_way(f, rho):
    Q, X, eps = _int8_coherent_case(f, (rho,))
    want = np.sort(keys_of(oracle.semijoin_pairs(Q, X, eps)))
    assert want.size >= (0 if rho > 0 else 40)
    for bits in (8, 16):
        opts = ersj.default_options(refine_kernel=ersj.REFINE_MFMA16, filter_bits=bits)
        parts, h = ersj.semi_join(torch.from_numpy(Q).cuda(), torch.from_numpy(X).cuda(), eps, 0, opts,
                                  return_index=True)
        st = ersj.get_stats(h)
        h.free()
        got = np.sort(keys_of(ersj.pairs_to_numpy(parts)))
        say(f"[gpu] int8 rounding one way f={f} bits={bits}: {got.size} pairs (oracle {want.size}), "
            f"filtered={st['last_filtered']}, settled early {st['last_partial']}")
        assert st["filter_bits"] == bits and st["last_filtered"] == 1
        if rho > 0:
            assert st["last_partial"] > 0  # the bound settles blocks here
        assert np.array_equal(got, want), (f, rho, bits)


@pytest.mark.parametrize("case", ["eps0_duplicates", "eps_inf", "one_far_outlier", "constant_leading_dims"])
def test_int8_filter_degenerate_inputs(case):
    # eps = 0 with repeated rows (only exact duplicates pair up), eps = inf
    # (every row start clamped: nothing settled), one row far from all others
    # (it sets the int8 scale, so the others' integers are small and the
    # bound wide), and 70 of 80 dimensions constant (the variance order puts
    # the 10 that vary first, so the filter's 64 dimensions are mostly
    # zero after centring); both filter forms against the oracle
    rng = np.random.default_rng(len(case))
    d = 80
    if case == "eps0_duplicates":
        base = rng.random((300, d), dtype=np.float32)
        X = base[rng.integers(0, 300, 900)]
        eps = 0.0
    elif case == "eps_inf":
        X = rng.random((400, d), dtype=np.float32)
        eps = math.inf
    elif case == "one_far_outlier":
        X = rng.random((2000, d), dtype=np.float32)
        X[17] += np.float32(500.0)
        eps = 0.33 * math.sqrt(d / 6.0)
    else:
        X = np.full((1500, d), np.float32(0.25))
        X[:, 70:] = rng.random((1500, 10), dtype=np.float32)
        eps = 0.4
    want = oracle.selfjoin_pairs(X, eps)
    for bits in (8, 16):
        got, st = _join_stats(X, eps, 0, bits)
        say(f"[gpu] int8 degenerate {case} bits={bits}: {len(got)} pairs (oracle {len(want)}), "
            f"filter bits used {st['filter_bits']}, settled early {st['last_partial']}")
        assert_same_pairs(X, eps, got, want, f"{case} bits={bits}")
