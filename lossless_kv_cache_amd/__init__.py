"""Lossless KV-cache coding on MI355X: residual against a predictor cache,
per-channel discretized-Laplace tables, 32-lane interleaved rANS in HIP.

The C ABI lives in ``include/skv.h`` (``libskv.so``); ``skv`` is its thin
ctypes binding.
"""
from . import skv  # noqa: F401
from .skv import (BF16, CHECKERBOARD, CHECKERBOARD_MAP, E4M3, INT16, RESIDUAL, RESIDUAL_EXP, Encoder,  # noqa: F401
                  SkvError, Store, Tables, block_hashes, decode, decode_into, decode_range, encode, encode_noalloc, encode_workspace,
                  fit_tables, fit_tables_map, load_tables, make_shape, transfer)
