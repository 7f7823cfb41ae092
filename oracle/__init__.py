"""CPU oracle of the CSA/HCA attention path (float64 numpy, plus a scalar
brute-force twin for tiny inputs).

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the library or its binding.
"""
from . import lca_oracle, brute, workloads  # noqa: F401
