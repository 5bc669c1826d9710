"""fp64 CPU oracle for the AKV hot path -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this package.  The product path never imports it and has no CPU fallback.
"""
from .akv_oracle import *  # noqa: F401,F403
from .akv_oracle import __all__  # noqa: F401
