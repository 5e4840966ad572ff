"""fp64 CPU oracle of the CRISP sparse prefill path.

Test infrastructure only: imported by the test suite, the package smoke check
and the benchmark's CPU-baseline leg, never by the product path.
"""
from .crisp_oracle import *  # noqa: F401,F403
