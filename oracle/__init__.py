"""CPU oracle of the MoE layer forward (test infrastructure only).

Imported only by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
leg. Nothing on the product path may import it.
"""
from . import moe_oracle
from .moe_oracle import *  # noqa: F401,F403
