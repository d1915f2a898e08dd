"""f64 CPU oracle (test infrastructure only; never used by the product path)."""
from .mel_oracle import *  # noqa: F401,F403
from . import mel_oracle  # noqa: F401
