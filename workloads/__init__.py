"""Seeded synthetic KV-cache workloads (input generation only).

This package draws the arrays that both the library and the test oracle
consume.  It holds none of the coding arithmetic: no symbol mapping, no
tables, no entropy coding.
"""
from .gen import CONFIGS, Config, dckv_draw, residual_slab, channel_sigma  # noqa: F401
