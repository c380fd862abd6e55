"""CPU oracle of the NSA forward pass (test infrastructure only; see nsa_oracle)."""
from .nsa_oracle import *  # noqa: F401,F403
