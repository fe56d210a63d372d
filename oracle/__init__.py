"""CPU oracle for the LLA latent-cache kernels (test infrastructure only; see lla_oracle.py)."""
from .lla_oracle import *  # noqa: F401,F403
