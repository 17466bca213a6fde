"""CPU oracle (test infrastructure only; see lrkv_oracle's header)."""
from .lrkv_oracle import *  # noqa: F401,F403
