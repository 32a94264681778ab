"""CPU oracle for the POET-X layer (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The HIP library never calls it and shares no code
with it.
"""
from .poetx_oracle import *  # noqa: F401,F403
