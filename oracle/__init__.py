"""CPU oracle (test infrastructure only; see qsa_oracle's header)."""

from .qsa_oracle import *  # noqa: F401,F403
from .qsa_oracle import BLOCK, BUDGET_TOKENS, TOP_K_BLOCKS  # noqa: F401
