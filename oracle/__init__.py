"""Float64 CPU oracle (test infrastructure only; see hs2_oracle's header)."""
from .hs2_oracle import *  # noqa: F401,F403
from .hs2_oracle import BLOCK, K_GLOBAL, WINDOW  # noqa: F401
