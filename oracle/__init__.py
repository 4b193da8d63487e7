"""fp64 CPU oracle (test infrastructure only; see losa_oracle's header)."""
from .losa_oracle import *  # noqa: F401,F403
from .losa_oracle import __all__  # noqa: F401
