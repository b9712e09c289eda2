"""Float64 CPU oracle (test infrastructure only; see opd_oracle for the rules of its use)."""

from .opd_oracle import *  # noqa: F401,F403
from .opd_oracle import __all__  # noqa: F401
