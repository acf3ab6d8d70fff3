"""Seeded synthetic inputs shared by the tests, the bench and the oracle's sample runs.

This package draws random numbers and lays them out in the shapes of the
workloads; it holds none of the attention method's arithmetic (no RoPE, no
compression, no scoring, no quantisation).
"""
from .rng import bits64, uniform, normal, normal_bf16, permutation, stream_key  # noqa: F401
from . import workloads  # noqa: F401
