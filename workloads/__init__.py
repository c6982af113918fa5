"""Seeded synthetic workloads for the paged decode path.

This package only draws random numbers and describes workload shapes; it
contains no step of the attention or block-bookkeeping arithmetic.  Both the
HIP path (through the Python binding) and the CPU oracle consume what it
produces, so it is the single source of inputs for parity tests and the bench.
"""
from .configs import WORKLOADS, Workload, Instance, get  # noqa: F401
