"""CPU oracle -- TEST INFRASTRUCTURE, not part of the product path.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It is a plain float64 implementation of what the fused kernels
compute and shares no code with the HIP library.
"""
from .mk_oracle import *  # noqa: F401,F403
from .compare import *  # noqa: F401,F403
