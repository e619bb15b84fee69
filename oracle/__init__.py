"""fp64 CPU oracle (test infrastructure only; see oracle/oracle.py)."""
from .oracle import *  # noqa: F401,F403
from .oracle import KV_CHUNK  # noqa: F401
