"""CPU oracle for the Sparse-BitLinear forward path (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package; the HIP library never does.
"""
from .sbl_oracle import *  # noqa: F401,F403
