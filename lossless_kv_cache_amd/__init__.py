"""Lossless KV-cache coding on MI355X: residual against a predictor cache,
per-channel discretized-Laplace tables, 32-lane interleaved rANS in HIP.

The C ABI lives in ``include/skv.h`` (``libskv.so``); ``skv`` is its thin
ctypes binding.
"""
from . import skv  # noqa: F401
from .skv import (BF16, CHECKERBOARD, E4M3, INT16, RESIDUAL, Encoder, SkvError, Tables,  # noqa: F401
                  decode, decode_into, encode, fit_tables, load_tables, make_shape)
