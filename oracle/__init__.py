"""CPU oracle of the NanoColibri MoE layer (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package; the GPU library never does.
"""
from .moe_oracle import *  # noqa: F401,F403
