"""Seeded synthetic inputs for the paged decode path.

This package draws random numbers, rounds them to storage dtypes, places tokens into a scattered
block pool through the host block manager, and fills unused memory with poison. It holds none of
the method's arithmetic: no attention, no softmax, no copy-on-write execution. Both the HIP
library (through the tests and ``bench.py``) and the oracle read the same arrays it returns.
"""

from .synth import *  # noqa: F401,F403
