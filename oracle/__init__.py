"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .h3k_oracle import *  # noqa: F401,F403
