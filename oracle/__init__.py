"""CPU oracle (test infrastructure only).

Used by the tests, by the package's smoke check and by the benchmark's CPU
baseline leg.  The HIP library never imports it.
"""
from .sda_oracle import *  # noqa: F401,F403
