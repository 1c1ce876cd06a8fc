"""fp64 CPU oracle of the In-Place TTT layer, forward and backward (test
infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it.
"""
from .ipttt_oracle import *  # noqa: F401,F403
from .ipttt_oracle import __all__  # noqa: F401
