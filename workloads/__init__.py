"""Seeded synthetic workloads for the ReplaySSM decode path.

This package only *draws inputs*: shapes, seeds and the random recipe of each
workload. It holds none of the method's arithmetic (no decay, no state update,
no output formula). It is the one module both the fp64 oracle's tests and the
HIP library's tests/benchmark use, so that both sides see exactly the same bits.
"""
from .shapes import Workload, WORKLOADS, get  # noqa: F401
from . import synth  # noqa: F401
