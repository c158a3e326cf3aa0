"""Quantized sparse shared-KV MLA attention for AMD MI355X (gfx950).

The compute path is the HIP library libcsmla.so (C ABIs: include/csmla.h for
the attention, include/csmla_indexer.h for the indexer top-k that feeds it);
this package is its thin ctypes binding.  There is no CPU fallback: the
binding raises if the library is missing.
"""
from .binding import (  # noqa: F401
    CsmlaProblem, CsmlaHostLengths, CsmlaTensors, CsmlaError, Plan,
    csmla_abi_version, csmla_status_string, csmla_last_error, csmla_metadata_words,
    csmla_validate, csmla_plan, csmla_plan_check, csmla_forward, csmla_forward_noalloc, csmla_debug_resolve, csmla_debug_resolve_whole_token,
    problem_from, host_lengths_from, tensors_from, forward, debug_resolve, load, LIB_PATH,
    CsmlaIndexerProblem, CsmlaIndexerHostLengths, CsmlaIndexerTensors, IndexerPlan,
    csmla_indexer_metadata_words, csmla_indexer_validate, csmla_indexer_plan, csmla_indexer_forward,
    indexer_problem_from, indexer_host_lengths_from, indexer_tensors_from, indexer_forward,
)
