"""fp64 CPU oracle (test infrastructure only; see lp_oracle.py).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg import
this package.  The library never does.
"""
from .lp_oracle import *  # noqa: F401,F403
