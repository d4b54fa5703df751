"""CPU oracle of routed block-sparse attention -- test infrastructure only.

Only the tests, the package's smoke check and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the HIP library.
"""
from .sol_oracle import *  # noqa: F401,F403
