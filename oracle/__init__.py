"""NABLA oracle (test infrastructure only): plain float64 CPU reference.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.
"""
from .nabla_oracle import *  # noqa: F401,F403
from .nabla_oracle import __all__  # noqa: F401
