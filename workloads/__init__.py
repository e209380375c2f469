"""Seeded synthetic inputs for the KDA hot path.

This package draws random tensors in the shapes and distributions of the five
workloads and casts them to their storage dtypes.  It holds none of the
method's arithmetic: the tests, the smoke check and the benchmark feed the
same stored tensors to the HIP library and to the oracle.
"""
from .configs import CONFIGS, Config
from .gen import chunk_inputs, decode_inputs, draw_chunk

__all__ = ["CONFIGS", "Config", "chunk_inputs", "decode_inputs", "draw_chunk"]
