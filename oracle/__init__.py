"""CPU oracle of the routed MoE expert layer (test infrastructure only).

Importable only from tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg.  It shares no code with the GPU library.
"""
from .moe_oracle import *  # noqa: F401,F403
