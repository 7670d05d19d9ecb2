"""Seeded synthetic workloads shared by the oracle and the GPU path.

Holds shapes, seeded draws and storage encodings only; no attention or
allocation arithmetic.
"""
from .workloads import *  # noqa: F401,F403
from .workloads import (C1, C2, C3, C4, C5, CONFIGS, DecodeConfig, SamplingConfig,  # noqa: F401
                        PoolPlan)
