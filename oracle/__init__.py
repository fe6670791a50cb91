"""fp64 CPU oracle (test infrastructure only; never used by the product path)."""
from .lla_oracle import *  # noqa: F401,F403
