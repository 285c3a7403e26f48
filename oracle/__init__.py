"""Plain fp64 CPU oracle (test infrastructure only; see evo_oracle)."""
from .evo_oracle import *  # noqa: F401,F403
