"""fp64 CPU oracle of the CSA/HCA layer path -- test infrastructure only.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library.
"""
from . import csa_oracle  # noqa: F401
