"""fp64 CPU oracle for the BEAM masked-MoE layer (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The HIP library and its Python binding never do.
"""
from .beam_oracle import *  # noqa: F401,F403
from .beam_oracle import __all__  # noqa: F401
