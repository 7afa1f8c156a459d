"""CPU fp64 oracle of the fused chunked sparse-KL loss head (test infrastructure only)."""
from .kl_oracle import *  # noqa: F401,F403
