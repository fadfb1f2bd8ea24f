"""CPU oracle (test infrastructure only): see rd_oracle for what it computes.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.
"""
from .rd_oracle import *  # noqa: F401,F403
