"""CPU oracle for the lightning-indexer top-k (TEST INFRASTRUCTURE ONLY).

Restates the QuantLightningIndexerV2 page (功能说明 formula and steps,
参数说明, 约束说明) for quant_mode 1: fp8 e4m3 query and key, fp32 dequant
scales, fp32 weights.  For query token t of batch b with g index heads,

    score[t, s] = sum_h  W[t, h] * ReLU((scale_q[t, h] * scale_k[s]) * (q[t, h, :] . k[s, :]))

for each compressed index key s that the token may see, and the output is the
topk key positions with the largest scores, -1 padded.

Readings where the page is silent (each one is listed in the design notes):
  * D = 128, the index head width; the key has one head (约束说明).
  * Which keys a token sees follows the attention page's rule for cmp_kv:
    restored length L = n * cmp_ratio + cmp_residual_k, token i of the batch's
    S1 sits at position p = L - S1 + i, and mask_mode 3 lets it see
    floor((p + 1) / cmp_ratio) keys (clamped to [0, n]); mask_mode 0 sees all n.
  * Equal scores: the lower key position wins.  The chosen positions are
    written in ascending order, then -1 up to topk.
  * Query rows past seqused_q (TND or BSND padding) get -1 everywhere, as the
    page's TND padding constraint says for invalid rows.

Precision: the ranking is decided on float32 scores, the precision the HIP
kernel ranks in.  The dot products are formed exactly (float64 holds every
sum of 128 products of e4m3 values) and rounded once to float32; the scale
product, the ReLU, the weights and the sum over heads (in head order) are
float32 operations in the formula's order.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline
may import this module; the library never does.
"""
from typing import Iterable, Optional

import numpy as np

from .fp8 import decode_e4m3


def _np(x):
    if x is None:
        return None
    return x.detach().cpu().numpy() if hasattr(x, "detach") else np.asarray(x)


def index_scores(q_codes, q_scale, weights, k_codes, k_scale) -> np.ndarray:
    """Scores of one query token against n keys (功能说明, steps 1-3 before Top-k).

    q_codes [g, d] uint8, q_scale [g] f32, weights [g] f32, k_codes [n, d] uint8,
    k_scale [n] f32  ->  float32 [n]."""
    q = decode_e4m3(q_codes)                                  # [g, d] exact values
    k = decode_e4m3(k_codes)                                  # [n, d]
    dots = (q @ k.T).astype(np.float32)                       # step 1: Q K^T, [g, n]
    scale = np.asarray(q_scale, np.float32)[:, None] * np.asarray(k_scale, np.float32)[None, :]  # Scale_Q Scale_K^T
    rel = np.maximum(scale * dots, np.float32(0.0))           # step 2: dequantise, ReLU
    weighted = np.asarray(weights, np.float32)[:, None] * rel  # step 3: (W 1) ⊙ ...
    out = np.zeros(weighted.shape[1], dtype=np.float32)
    for h in range(weighted.shape[0]):                        # 1_{1×g} @ ...: sum over heads
        out = out + weighted[h]
    return out


def topk_positions(scores: np.ndarray, k: int) -> np.ndarray:
    """Top-k of one score row: the k highest scores, ties to the lower position,
    returned as ascending positions padded with -1 to length k."""
    n = int(scores.shape[0])
    ranked = sorted(range(n), key=lambda s: (-float(scores[s]), s))
    chosen = sorted(ranked[:k])
    out = np.full(k, -1, dtype=np.int32)
    out[:len(chosen)] = chosen
    return out


def visible_keys(p: int, n: int, ratio: int, mask_mode: int) -> int:
    """Leading compressed keys a row at restored position p sees."""
    if mask_mode == 0:
        return n
    if mask_mode == 3:
        return max(0, min(n, (p + 1) // ratio))
    raise ValueError(f"mask_mode {mask_mode}")


def token_context(inp, t: int):
    """(batch, row in batch, rows used in batch S1, keys n, visible keys) of query row t;
    visible is -1 for a padding row (past seqused_q)."""
    if inp.layout_q == "TND":
        cu = _np(inp.cu_seqlens_q)
        b = int(np.searchsorted(cu, t, side="right") - 1)
        i, span = t - int(cu[b]), int(cu[b + 1] - cu[b])
    else:
        b, i, span = t // inp.q_s, t % inp.q_s, inp.q_s
    s1 = span if inp.seqused_q is None else int(_np(inp.seqused_q)[b])
    if inp.layout_k == "TND":
        cuk = _np(inp.cu_seqlens_k)
        n = int(cuk[b + 1] - cuk[b])
    elif inp.seqused_k is not None:
        n = int(_np(inp.seqused_k)[b])
    else:
        n = int(inp.key.shape[1])                               # BSND: S
    res = 0 if inp.cmp_residual_k is None else int(_np(inp.cmp_residual_k)[b])
    if i >= s1:
        return b, i, s1, n, -1
    p = n * inp.cmp_ratio + res - s1 + i
    return b, i, s1, n, visible_keys(p, n, inp.cmp_ratio, inp.mask_mode)


def key_rows(inp, b: int, count: int):
    """(codes [count, d], scales [count]) of the batch's first `count` keys."""
    key, ks = _np(inp.key), _np(inp.key_scale)
    pos = np.arange(count)
    if inp.layout_k == "PA_BBND":
        bs = key.shape[1]
        blk = _np(inp.block_table)[b, pos // bs].astype(np.int64)
        return key[blk, pos % bs, 0], ks[blk, pos % bs]
    if inp.layout_k == "TND":
        r0 = int(_np(inp.cu_seqlens_k)[b])
        return key[r0 + pos, 0], ks[r0 + pos]
    return key[b, pos, 0], ks[b, pos]


def oracle_scores(inp, t: int) -> Optional[np.ndarray]:
    """float32 scores of row t over its visible keys (None for a padding row)."""
    b, _, _, _, vis = token_context(inp, t)
    if vis < 0:
        return None
    kc, ks = key_rows(inp, b, vis)
    return index_scores(_np(inp.q)[t], _np(inp.q_scale)[t], _np(inp.weights)[t], kc, ks)


def oracle_indexer(inp, tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """sparse_indices as int32 [T1, topk] (rows not in `tokens` stay -1)."""
    T1 = int(inp.q.shape[0])
    out = np.full((T1, inp.topk), -1, dtype=np.int32)
    for t in (range(T1) if tokens is None else tokens):
        sc = oracle_scores(inp, t)
        if sc is not None and sc.shape[0] > 0:
            out[t] = topk_positions(sc, inp.topk)
    return out
