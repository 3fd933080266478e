"""Seeded synthetic inputs shared by the CPU oracle, the tests and the bench.

Nothing here computes any step of the MoE routing method: the module only
draws random numbers (numpy PCG64) and rounds them to storage formats.
"""
from .gen import *  # noqa: F401,F403
