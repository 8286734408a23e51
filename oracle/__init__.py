"""fp64 CPU oracle of DKV decode attention -- test infrastructure only.

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import it; the HIP library never does.
"""
from .dkv_oracle import *  # noqa: F401,F403
