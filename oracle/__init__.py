"""fp64 CPU oracle of the ST-DiT attention block.  TEST INFRASTRUCTURE ONLY.

Importable from the tests, the smoke check and the benchmark's CPU-baseline leg,
never from the product path.  Shares no code with the HIP kernels.
"""
from .st_oracle import *  # noqa: F401,F403
from . import st_oracle  # noqa: F401
