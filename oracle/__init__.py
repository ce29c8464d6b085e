"""CPU oracle for the W4A16 weight-only linear layer (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package; the HIP library and its binding never do.
"""
from .w4a16_ref import *  # noqa: F401,F403
