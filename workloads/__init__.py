"""Seeded synthetic inputs for quantized sparse shared-KV MLA attention.

This package holds only input generation: shapes, lengths, block tables,
sparse index draws, random values and their fp8 e4m3 quantisation.  It holds
none of the attention arithmetic, so both the CPU oracle (``oracle/``) and the
HIP path can consume the same bytes without sharing any method code.
"""
from .gen import Inputs, make_config, make_custom, redraw_query_side, CONFIG_NAMES, quantize_rows_e4m3  # noqa: F401
