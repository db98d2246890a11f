"""fp64 CPU oracle of the CRISP sparse-attention prefill.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's CPU
baseline leg import this package.  The GPU library never does.
"""
from . import crisp_oracle  # noqa: F401
from .crisp_oracle import *  # noqa: F401,F403
