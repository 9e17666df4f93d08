"""CPU oracle of the SCOPE hot path (test infrastructure only; see scope_oracle)."""
from .scope_oracle import *  # noqa: F401,F403
