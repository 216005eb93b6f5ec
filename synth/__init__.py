"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the benchmark.

This package holds input construction only (random draws, index lists, tree
shapes, planted logits).  It computes no attention, no softmax and no
acceptance: the oracle and the HIP library each do that on their own.
"""
from .generators import *  # noqa: F401,F403
