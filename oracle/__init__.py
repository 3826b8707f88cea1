"""fp64 CPU oracle of the NAtS-L hybrid layer.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it.  The HIP library never uses it.
"""
from .natsl_oracle import *  # noqa: F401,F403
from .natsl_oracle import SM, LIN, CHUNK  # noqa: F401
