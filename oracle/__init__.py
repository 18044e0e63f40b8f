"""CPU oracle of the capacity-limited MoE layer forward pass (test infrastructure only).

Only the test suite, the entry module's smoke check and the benchmark's CPU-baseline
leg may import this package; the product library never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
