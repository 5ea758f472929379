"""The binary64 re-check and the kNN ranking compute the canonical D64
(difference, square and sum each rounded on their own, no fused
multiply-add): pairs built so that a fused accumulation lands on the other
side of fl(eps^2) must be decided as the canonical value says, by both
refinement kernels, and the kNN must report the canonical D64."""
import numpy as np
import pytest
import torch

import exact_range_similarity_amd as ersj
from fused_pairs import canonical_d64, discriminating_pairs

from gpu_util import KERNELS, gpu_pairs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ersj.lib()


@pytest.mark.parametrize("d", [7, 33])
def test_join_decides_with_the_canonical_d64(d):
    pairs = discriminating_pairs(24, d, 100 + d)
    say(f"[gpu] {len(pairs)} fused/unfused discriminating pairs, d={d}")
    for k in KERNELS:
        for a, b, eps, inside in pairs:
            X = np.stack([a, b])
            got = {tuple(p) for p in gpu_pairs(X, eps, options=ersj.default_options(refine_kernel=k)).tolist()}
            assert got >= {(0, 0), (1, 1)}
            assert ((0, 1) in got) == inside and ((1, 0) in got) == inside, (k, eps, inside)


def test_knn_reports_the_canonical_d64():
    pairs = discriminating_pairs(16, 9, 7)
    for a, b, eps, _ in pairs:
        X = torch.from_numpy(np.stack([a, b])).cuda()
        ids, dist, _ = ersj.knn(X, 2, 1.0)
        assert dist[0, 1].item() == canonical_d64(a, b) == dist[1, 1].item()
