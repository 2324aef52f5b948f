"""CPU oracle (test infrastructure only): plain float64 definitions of the
fused block's forward and backward, used to check the HIP path.  Only the
tests, the smoke check and the benchmark's CPU-baseline leg import it."""
from .coda_oracle import *  # noqa: F401,F403
from .coda_oracle import __all__  # noqa: F401
