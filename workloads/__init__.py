"""Seeded synthetic DNA workloads shared by the tests, the benchmark and the smoke check.

This package only draws sequences. It holds none of the hit-discovery, gating or
extension arithmetic: no seed keys, no scores, no X-drop. Both the HIP path and the
CPU oracle receive the same ASCII bytes from here and compute everything else on
their own.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    HOXD70,
    SEED_PATTERN,
    Workload,
    build,
    random_pair,
    reverse_complement_ascii,
)
