"""CPU oracle (test infrastructure only; see qmm_oracle's header)."""
from .qmm_oracle import *  # noqa: F401,F403
from . import qmm_oracle  # noqa: F401
