"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle scripts.

This package only draws coordinates.  It holds none of the join's arithmetic
(no distance, no epsilon, no grid), so the GPU path and the CPU oracle can
both consume its arrays without sharing any code of the method.
"""
from .synth import (  # noqa: F401
    CONFIGS, ConfigSpec, make_config, make_config_labels, make_queries, config_spec, lattice, fig3_points, fig5_points,
    x_digest,
)
