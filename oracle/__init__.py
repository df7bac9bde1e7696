"""CPU oracle for the MoGE layer (test infrastructure only; see moge_oracle)."""
from .moge_oracle import *  # noqa: F401,F403
from . import moge_oracle  # noqa: F401
