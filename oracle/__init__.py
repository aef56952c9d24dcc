"""CPU oracle (test infrastructure only; see schnet_oracle)."""
from .schnet_oracle import *  # noqa: F401,F403
