"""Plain fp64 CPU oracle (test infrastructure; see oracle.py)."""
