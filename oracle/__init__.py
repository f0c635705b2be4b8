"""CPU oracle of the routed MoE layer -- test infrastructure only.

Imported only by the tests, the smoke check and the bench's CPU-baseline leg.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import LRUCache, CapacityError  # noqa: F401
from . import kv_oracle  # noqa: F401  (the KV tier)
