"""CPU oracle for the ZAYA1 decoder block (test infrastructure only; see zaya_oracle)."""
from .zaya_oracle import *  # noqa: F401,F403
