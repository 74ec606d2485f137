"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .llatte_oracle import *  # noqa: F401,F403
from . import llatte_oracle, brute  # noqa: F401
