"""CPU oracle (test infrastructure only; see tp_oracle.py)."""
from .tp_oracle import *  # noqa: F401,F403
from .tp_oracle import Cfg, Local  # noqa: F401
