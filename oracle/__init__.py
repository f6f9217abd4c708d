"""CPU oracle (test infrastructure only; see armt_oracle's docstring)."""
from .armt_oracle import *  # noqa: F401,F403
from .armt_oracle import __all__  # noqa: F401
