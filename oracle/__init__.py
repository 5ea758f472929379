"""CPU oracle for the exact epsilon-distance self-join, semi-join and kNN.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check
and by the benchmark's ``cpu_baseline`` leg, never by the product path.  It
shares no code with the GPU library.
"""
from .oracle import (  # noqa: F401
    available, d64, e64, join_rows, selfjoin_pairs, semijoin_rows, semijoin_pairs, band_count,
    calibrate_bounds, knn_rows, knn, mix64, digest_rows, digest_all,
    calibrate_eps, version, threads,
)
