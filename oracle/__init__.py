"""CPU oracle of the routed-experts MoE layer (test infrastructure only).

Only tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package; the product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
