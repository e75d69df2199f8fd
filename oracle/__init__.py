"""CPU oracle of the DeepSeekMoE layer forward — test infrastructure only.

Importable from the tests, the smoke check and the benchmark's CPU-baseline
leg; never from the library.  See moe_oracle.py.
"""
from .moe_oracle import *  # noqa: F401,F403
from . import moe_oracle  # noqa: F401
