"""Seeded synthetic workloads for the CSA/HCA layer path.

This package holds only shapes and random draws; it contains none of the
method's arithmetic (no compression, scoring, selection or attention), so both
the CPU oracle and the HIP path can be fed from it without sharing any
computation.
"""
from .configs import WORKLOADS, Workload, workload  # noqa: F401
from .inputs import make_inputs, draw_lengths  # noqa: F401
