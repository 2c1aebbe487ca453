"""CPU oracle (numpy float64).  Test infrastructure only: imported by the
tests, the package smoke check and the benchmark's CPU-baseline leg, never by
the product path."""
from .lsi_oracle import *  # noqa: F401,F403
from .lsi_oracle import lse_merge, recall  # noqa: F401
