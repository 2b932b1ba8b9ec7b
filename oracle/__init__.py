"""Plain fp64 CPU oracle for WaterSIC layer quantization.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this package: only the
test suite, the smoke check and the benchmark's CPU-baseline leg use it.
"""
from .watersic import *  # noqa: F401,F403
