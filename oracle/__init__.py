"""CPU oracle for quantized sparse shared-KV MLA attention and for the
lightning-indexer top-k that feeds it (test infrastructure).

This package is TEST INFRASTRUCTURE ONLY.  It is a plain, slow, float64
NumPy restatement of what the pages define, used to check the HIP path.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The library under ``sparse_compressed_mla_amd/``
never imports it and never falls back to it.

``oracle.indexer`` holds the indexer oracle.  Every function is pinned by
``tests/test_oracle_*.py`` against something other
than itself (library routines, closed forms, brute-force masks, invariants).
"""
from .fp8 import decode_e4m3, E4M3_LUT  # noqa: F401
from .attention import (  # noqa: F401
    OracleResult, oracle_forward, attend_rows, merge_partials,
    batch_lengths, ori_window, cmp_visible, token_rows, token_table,
)
