"""BitDelta CPU oracle -- test infrastructure only (see oracle.py)."""
from .oracle import *  # noqa: F401,F403
from .oracle import build, load, PER_MATRIX, PER_ROW  # noqa: F401
