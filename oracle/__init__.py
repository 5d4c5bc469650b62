"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .lychee_oracle import *  # noqa: F401,F403
from .lychee_oracle import decode_step_f64  # noqa: F401
