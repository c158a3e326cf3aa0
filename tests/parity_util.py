"""Comparison helpers for GPU-vs-oracle parity (shared by the GPU tests,
smoke() and bench.py's parity precheck).

Tolerance (from the benchmark spec's numeric target): every bf16 output
element satisfies |gpu - ref| <= 1e-2 + 1e-2*|ref| and every lse element
|gpu - ref| <= 1e-3; -inf must match -inf exactly.
"""
import sys

import numpy as np

ATOL, RTOL, LSE_ATOL = 1e-2, 1e-2, 1e-3


def compare(out_gpu, ref_out, tokens, lse_gpu=None, ref_lse=None, name="", verbose=True):
    """out_gpu: np.float32 [T1, N1, D] (bf16 upcast); ref_out: oracle float64.
    Returns a dict of error figures; raises AssertionError past tolerance."""
    toks = np.asarray(tokens, dtype=np.int64)
    g = out_gpu[toks].astype(np.float64)
    r = ref_out[toks]
    assert np.all(np.isfinite(r)), f"{name}: oracle produced non-finite values"
    assert np.all(np.isfinite(g)), f"{name}: GPU produced non-finite values at {np.argwhere(~np.isfinite(g))[:5]}"
    err = np.abs(g - r)
    bound = ATOL + RTOL * np.abs(r)
    bad = err > bound
    stats = dict(max_abs=float(err.max(initial=0.0)),
                 max_rel=float((err / np.maximum(np.abs(r), 1e-3)).max(initial=0.0)),
                 norm_rel=float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)),
                 n=int(g.size))
    if lse_gpu is not None and ref_lse is not None:
        lg = lse_gpu[toks].astype(np.float64)
        lr = ref_lse[toks]
        both_inf = np.isneginf(lg) & np.isneginf(lr)
        assert np.array_equal(np.isneginf(lg), np.isneginf(lr)), f"{name}: lse -inf pattern differs"
        le = np.abs(np.where(both_inf, 0.0, lg - lr))
        stats["lse_max_abs"] = float(le.max(initial=0.0))
        assert np.all(le <= LSE_ATOL), f"{name}: lse error {le.max()} > {LSE_ATOL}"
    if verbose:
        print(f"[parity] {name}: " + " ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}"
                                             for k, v in stats.items()), flush=True)
        sys.stdout.flush()
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{name}: {int(bad.sum())} elements past tolerance; first {idx.tolist()}, "
                             f"gpu {g[bad][:5]}, ref {r[bad][:5]}, stats {stats}")
    return stats
