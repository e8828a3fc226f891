"""CPU oracle for Sparse Gated Attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The GPU library and its binding never import it.
"""
from .sga_oracle import *  # noqa: F401,F403
