"""fp64 CPU oracle (test infrastructure only; see oracle.py)."""
from . import oracle  # noqa: F401
