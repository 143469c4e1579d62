"""CPU oracle of the flow-matching denoise loop. Test infrastructure only: imported by the
tests, the package smoke check and the benchmark's CPU-baseline leg, never by the product."""
from .fm_oracle import *  # noqa: F401,F403
