"""CPU oracle (test infrastructure only; see ref.py)."""
from .ref import *  # noqa: F401,F403
