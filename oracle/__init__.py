"""CPU fp64 oracle of the LaCT fast-weight layer (test infrastructure only)."""
from .lact_oracle import *  # noqa: F401,F403
