"""fp64 CPU oracle (test infrastructure only; see svg2_oracle)."""
from .svg2_oracle import *  # noqa: F401,F403
