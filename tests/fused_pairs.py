"""Pairs of float32 vectors whose canonical binary64 squared distance (every
difference, square and sum rounded separately, the definition the join and
the kNN are specified by) differs from the value a fused multiply-add
accumulation gives, each with an eps whose fl(eps^2) equals the smaller of
the two: such a pair is a neighbour under one computation and not under the
other.  Pure python: float arithmetic is binary64 with round-to-nearest, and
the fused step is rounded once from the exact rational value.

The difference of two float32 values of similar magnitude is exact in
binary64 with at most about 26 significant bits, so its square is exact and
fusing changes nothing; the pairs therefore mix coordinates near 1 with
coordinates 2^-12 .. 2^-40 in size, whose differences carry up to 53 bits."""
import math
from fractions import Fraction

import numpy as np


def canonical_d64(a, b):
    s = 0.0
    for x, y in zip(a.tolist(), b.tolist()):
        t = float(x) - float(y)
        s = s + t * t
    return s


def fused_d64(a, b):
    s = 0.0
    for x, y in zip(a.tolist(), b.tolist()):
        t = float(x) - float(y)
        s = float(Fraction(t) * Fraction(t) + Fraction(s))
    return s


def eps_squaring_to(e):
    """An eps with eps * eps == e exactly in binary64, or None."""
    r = math.sqrt(e)
    for _ in range(2):
        r = math.nextafter(r, 0.0)
    for _ in range(5):
        if r * r == e:
            return r
        r = math.nextafter(r, math.inf)
    return None


def discriminating_pairs(count, d, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        a = (1.0 + rng.random(d)).astype(np.float32)
        b = (rng.random(d) * np.exp2(-rng.integers(12, 41, d))).astype(np.float32)
        c, f = canonical_d64(a, b), fused_d64(a, b)
        if c == f:
            continue
        eps = eps_squaring_to(min(c, f))
        if eps is None:
            continue
        out.append((a, b, eps, c <= eps * eps))
    return out
