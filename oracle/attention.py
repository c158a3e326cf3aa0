"""Float64 CPU oracle for quantized sparse shared-KV MLA attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py; never by the library.

What is computed (QuantSparseFlashMla page, 功能说明 formula, with the sink
logit of the benchmark spec added to the softmax):

    O = softmax(Q K~^T * softmax_scale  (+ sink logit))  V~,    K~ = V~

K~ is the concatenation of
  * the ori_kv rows visible to the query row under ori_mask_mode and the
    window (QuantSparseFlashMla, 参数说明: ori_mask_mode, ori_win_left/right),
  * the cmp_kv rows: every causally visible compressed token (HCA), or the
    valid entries of cmp_sparse_indices (CSA)  (QuantSparseFlashMla,
    功能说明: the three computation modes).

Readings of points the pages leave open:
  R1 sink: an extra logit sinks[h] with a zero value row; not multiplied by
     softmax_scale or any descale.  lse includes it.
  R2 ori band / causal masks are bottom-right aligned: query row i of a batch
     with S1 query rows and S2 kv tokens sits at position p = S2 - S1 + i
     (fused infer-attention page, 约束说明: the row-exclusion rules of
     sparse_mode 3 and 4).  Band: p-left <= j <= p+right; -1 = unbounded.
     RightDownCausal: j <= p.
  R3 cmp causal mask: compressed token c covers original tokens
     [c*r, c*r + r - 1]; it is visible to a row at restored position
     p_cmp = L - S1 + i (L = cmp_len*cmp_ratio + residual,
     QuantSparseFlashMla, 约束说明: cmp_residual_kv) iff c < floor((p_cmp+1)/r).
  R4 cmp_len default: seqused_cmp_kv, else cu_seqlens_cmp_kv difference, else
     the BSND shape, else floor(S2/cmp_ratio) for paged KV; residual default 0.
  R5 an index value is a logical compressed-token position within its batch;
     -1 anywhere, values < 0 and values >= the visible count are skipped;
     duplicates are kept (each listed entry is one key).  Only the first
     cmp_topk_length[t] slots are read when that tensor is given.
  R6 q_descale is one fp32 per (token, head) row, or one per token.
  R7 V uses the same rows and descales as K (K~ = V~).
  R8 no row visible: O = 0 and lse = sink (or -inf without sinks).
  R9 query rows at or past seqused_q inside a cu_seqlens_q span are padding:
     O = 0, lse = -inf.
  R10 bf16 q with packed 640-byte KV rows (KvQuantSparseAttnSharedkv): q's
     512 columns pair with the row's logical columns in storage order, the
     64 rope columns first, then the 448 nope columns; the output keeps that
     order.  There are no q or KV descales: the nope scales live in the row.
  R11 bf16 q and bf16 KV (SparseCompressedFlashAttention): values as stored.
  R12 ori_sparse_indices (QuantSparseFlashMla, 参数说明: indices into ori_kv,
     -1 invalid; ori_topk_length: the slots in effect): when given, the ori
     part of K~ is the listed logical positions in slot order (duplicates
     kept, -1 and out-of-range entries skipped) that the ori mask and window
     also admit, the same rule as for the compressed side (R5); without them
     it is the whole window.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from .fp8 import decode_e4m3
from .formats import decode_bf16, decode_packed640

TILE = 64
KIND_ORI = 0
KIND_CMP = 1


def _np(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        return x.detach().cpu().numpy()
    return np.asarray(x)


# ---------------------------------------------------------------------------
# lengths and positions
# ---------------------------------------------------------------------------

def batch_lengths(inp, b: int) -> Dict[str, int]:
    """Per-batch lengths (QuantSparseFlashMla, 参数说明 cu_seqlens_* / seqused_* /
    cmp_residual_kv; 约束说明 on seqused_cmp_kv and cmp_residual_kv)."""
    if inp.layout_q == "TND":
        cu = _np(inp.cu_seqlens_q)
        q0, span = int(cu[b]), int(cu[b + 1] - cu[b])
    else:
        q0, span = b * inp.q_s, inp.q_s
    s1 = span
    if inp.seqused_q is not None:
        s1 = min(span, int(_np(inp.seqused_q)[b]))
    # ori length
    if inp.seqused_ori_kv is not None:
        s2 = int(_np(inp.seqused_ori_kv)[b])
    elif inp.cu_seqlens_ori_kv is not None:
        cu = _np(inp.cu_seqlens_ori_kv)
        s2 = int(cu[b + 1] - cu[b])
    else:
        s2 = int(inp.ori_kv.shape[1])  # BSND shape
    kv0 = int(_np(inp.cu_seqlens_ori_kv)[b]) if inp.layout_kv == "TND" else 0
    r = int(inp.cmp_ratio)
    c, cmp0 = 0, 0
    if inp.cmp_kv is not None:
        if inp.seqused_cmp_kv is not None:
            c = int(_np(inp.seqused_cmp_kv)[b])
        elif inp.cu_seqlens_cmp_kv is not None:
            cu = _np(inp.cu_seqlens_cmp_kv)
            c = int(cu[b + 1] - cu[b])
        elif inp.layout_kv == "BSND":
            c = int(inp.cmp_kv.shape[1])
        else:
            c = s2 // r
        if inp.layout_kv == "TND":
            cmp0 = int(_np(inp.cu_seqlens_cmp_kv)[b])
    res = int(_np(inp.cmp_residual_kv)[b]) if inp.cmp_residual_kv is not None else 0
    return dict(q0=q0, span=span, s1=s1, s2=s2, c=c, res=res, L=c * r + res, kv0=kv0, cmp0=cmp0)


def ori_window(p: int, s2: int, mode: int, left: int, right: int) -> Tuple[int, int]:
    """Visible ori positions [lo, hi) for a row at position p (R2).

    mode 0: no mask; 3: j <= p; 4: p-left <= j <= p+right (-1 unbounded)."""
    if mode == 0:
        return 0, s2
    if mode == 3:
        return 0, max(0, min(s2, p + 1))
    if mode == 4:
        lo = 0 if left < 0 else max(0, p - left)
        hi = s2 if right < 0 else max(0, min(s2, p + right + 1))
        return lo, max(lo, hi)
    raise ValueError(f"ori_mask_mode {mode}")


def cmp_visible(p_cmp: int, c: int, r: int, mode: int) -> int:
    """Number of leading compressed tokens visible to a row at restored
    position p_cmp (R3): mode 0 -> all c; mode 3 -> clamp(floor((p+1)/r), 0, c)."""
    if mode == 0:
        return c
    if mode == 3:
        return max(0, min(c, (p_cmp + 1) // r))  # Python // floors negatives
    raise ValueError(f"cmp_mask_mode {mode}")


def token_table(inp) -> List[Tuple[int, int]]:
    """(batch, row-in-batch) for every flattened query token t (padding rows
    included, marked by row >= s1 in batch_lengths)."""
    out = []
    for b in range(inp.batch):
        bl = batch_lengths(inp, b)
        for i in range(bl["span"]):
            out.append((b, i))
    assert len(out) == inp.t1, (len(out), inp.t1)
    return out


def _phys_row(inp, which: str, b: int, j: int, bl) -> int:
    """Row of the flattened cache that holds logical token j of batch b."""
    if inp.layout_kv == "PA_BBND":
        table = _np(inp.ori_block_table if which == "ori" else inp.cmp_block_table)
        bs = int((inp.ori_kv if which == "ori" else inp.cmp_kv).shape[1])
        return int(table[b, j // bs]) * bs + j % bs
    if inp.layout_kv == "TND":
        return (bl["kv0"] if which == "ori" else bl["cmp0"]) + j
    smax = int((inp.ori_kv if which == "ori" else inp.cmp_kv).shape[1])
    return b * smax + j


def token_rows(inp, t: int, tt=None) -> List[Tuple[int, int]]:
    """The resolved key list of query token t, in order: ori band positions
    ascending, then cmp entries (HCA: [0, vis); CSA: index slots in order).
    Each entry is (kind, physical row)."""
    tt = tt or token_table(inp)
    b, i = tt[t]
    bl = batch_lengths(inp, b)
    if i >= bl["s1"]:
        return []
    rows = []
    p = bl["s2"] - bl["s1"] + i
    lo, hi = ori_window(p, bl["s2"], inp.ori_mask_mode, inp.ori_win_left, inp.ori_win_right)
    ori_idx = getattr(inp, "ori_sparse_indices", None)
    if ori_idx is None:
        ori_cand = range(lo, hi)
    else:
        slots = _np(ori_idx)[t, 0]
        k1 = len(slots)
        if getattr(inp, "ori_topk_length", None) is not None:
            k1 = max(0, min(k1, int(_np(inp.ori_topk_length)[t])))
        ori_cand = [int(x) for x in slots[:k1] if lo <= int(x) < hi]
    for j in ori_cand:
        rows.append((KIND_ORI, _phys_row(inp, "ori", b, j, bl)))
    if inp.cmp_kv is not None:
        p_cmp = bl["L"] - bl["s1"] + i
        vis = cmp_visible(p_cmp, bl["c"], int(inp.cmp_ratio), inp.cmp_mask_mode)
        if inp.cmp_sparse_indices is None:
            cand = range(vis)
        else:
            slots = _np(inp.cmp_sparse_indices)[t, 0]
            k = len(slots)
            if inp.cmp_topk_length is not None:
                k = max(0, min(k, int(_np(inp.cmp_topk_length)[t])))
            cand = [int(x) for x in slots[:k] if 0 <= int(x) < vis]
        for j in cand:
            rows.append((KIND_CMP, _phys_row(inp, "cmp", b, j, bl)))
    return rows


# ---------------------------------------------------------------------------
# dequantisation and dense softmax attention
# ---------------------------------------------------------------------------

def _bits16(x) -> np.ndarray:
    """Bit patterns of a 16-bit (bf16) tensor as uint16."""
    import torch
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _flat_cache(kv, ds, per_tile, fmt: str = "fp8"):
    """The cache as rows: fp8 codes with descales, bf16 bit patterns, or
    packed 640-byte rows (no descales for the last two)."""
    if fmt == "bf16":
        bits = _bits16(kv)
        return bits.reshape(-1, bits.shape[-1]), None, "bf16"
    d = kv.shape[-1]
    codes = _np(kv).reshape(-1, d)
    if fmt == "packed640":
        return codes, None, "packed640"
    dsn = _np(ds)
    return codes, dsn.reshape(codes.shape[0], -1) if per_tile else dsn.reshape(-1), per_tile


def dequant_rows(codes: np.ndarray, ds: np.ndarray, per_tile, rows: Sequence[int]) -> np.ndarray:
    """Rows of a cache as float64 values.  fp8: code * descale, with one
    descale per row or one per 64-wide tile of D (KvQuantSparseAttnSharedkv,
    参数说明: kv_quant_mode / tile_size); bf16: the stored values
    (SparseCompressedFlashAttention); packed640: rope then scaled nope
    (KvQuantSparseAttnSharedkv, 约束说明: the 640-wide row)."""
    rows = np.asarray(rows, dtype=np.int64)
    if per_tile == "bf16":
        return decode_bf16(codes[rows])
    if per_tile == "packed640":
        return decode_packed640(codes[rows])
    vals = decode_e4m3(codes[rows])
    if per_tile:
        return vals * np.repeat(ds[rows].astype(np.float64), TILE, axis=-1)
    return vals * ds[rows].astype(np.float64)[:, None]


def attend_rows(Q: np.ndarray, K: np.ndarray, scale: float, sinks: Optional[np.ndarray]):
    """Dense softmax attention of Q [N1, D] over keys K [n, D] (values = K),
    with an optional per-head sink logit (R1).  Returns (O, lse, lse_nosink)."""
    n1, d = Q.shape
    sig = np.full(n1, -np.inf) if sinks is None else np.asarray(sinks, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros((n1, d)), sig.copy(), np.full(n1, -np.inf)
    s = (Q @ K.T) * float(scale)
    m = np.maximum(s.max(axis=1), sig)
    e = np.exp(s - m[:, None])
    l_keys = e.sum(axis=1)
    l = l_keys + np.exp(sig - m)
    O = (e @ K) / l[:, None]
    return O, m + np.log(l), m + np.log(l_keys)


def merge_partials(parts, sinks: Optional[np.ndarray]):
    """Merge sink-free partial states of one query token over disjoint key
    subsets.  Each part is (m [N1], l [N1], acc [N1, D]) with
    acc = sum_j exp(s_j - m) v_j and l = sum_j exp(s_j - m); the sink logit is
    added once here.  (lse as the merge quantity: fused infer-attention page,
    输出说明 softmaxLse.)"""
    n1 = parts[0][0].shape[0]
    sig = np.full(n1, -np.inf) if sinks is None else np.asarray(sinks, dtype=np.float64)
    M = np.maximum(np.max([p[0] for p in parts], axis=0), sig)
    empty = ~np.isfinite(M)
    Ms = np.where(empty, 0.0, M)
    L = np.zeros(n1)
    acc = np.zeros_like(parts[0][2])
    for m, l, a in parts:
        w = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0.0) - Ms), 0.0)
        L += w * l
        acc += w[:, None] * a
    L += np.where(np.isfinite(sig), np.exp(np.where(np.isfinite(sig), sig, 0.0) - Ms), 0.0)
    O = np.where(L[:, None] > 0, acc / np.where(L > 0, L, 1.0)[:, None], 0.0)
    lse = np.where(L > 0, Ms + np.log(np.where(L > 0, L, 1.0)), -np.inf)
    return O, lse


@dataclass
class OracleResult:
    out: np.ndarray            # float64 [T1, N1, D]; rows not computed are NaN
    lse: np.ndarray            # float64 [T1, N1]  (includes the sink, R1)
    lse_nosink: np.ndarray     # float64 [T1, N1]
    rows: Dict[int, List[Tuple[int, int]]] = field(default_factory=dict)
    tokens: List[int] = field(default_factory=list)


def oracle_forward(inp, tokens: Optional[Sequence[int]] = None) -> OracleResult:
    """Reference result for the listed query tokens (all by default)."""
    T1, n1, d = inp.t1, inp.n1, inp.d
    tt = token_table(inp)
    toks = list(range(T1)) if tokens is None else [int(t) for t in tokens]
    q_bf16 = getattr(inp, "q_format", "fp8") == "bf16"
    fmt = getattr(inp, "kv_format", "fp8")
    q = (_bits16(inp.q) if q_bf16 else _np(inp.q)).reshape(T1, n1, d)
    qds = None if q_bf16 else _np(inp.q_descale).astype(np.float64)
    sinks = None if inp.sinks is None else _np(inp.sinks).astype(np.float64)
    per_tile = inp.kv_scale_mode == 1
    ori_codes, ori_ds, ori_tile = _flat_cache(inp.ori_kv, inp.ori_kv_descale, per_tile, fmt)
    if inp.cmp_kv is not None:
        cmp_codes, cmp_ds, cmp_tile = _flat_cache(inp.cmp_kv, inp.cmp_kv_descale, per_tile, fmt)
    out = np.full((T1, n1, d), np.nan)
    lse = np.full((T1, n1), np.nan)
    lse_ns = np.full((T1, n1), np.nan)
    res_rows = {}
    for t in toks:
        b, i = tt[t]
        rows = token_rows(inp, t, tt)
        res_rows[t] = rows
        if i >= batch_lengths(inp, b)["s1"]:
            out[t] = 0.0
            lse[t] = -np.inf
            lse_ns[t] = -np.inf
            continue
        if q_bf16:
            Q = decode_bf16(q[t])
        else:
            qs = qds[t] if qds.ndim == 2 else np.full(n1, qds[t])
            Q = decode_e4m3(q[t]) * qs[:, None]
        ori_r = [r for k, r in rows if k == KIND_ORI]
        cmp_r = [r for k, r in rows if k == KIND_CMP]
        parts = [dequant_rows(ori_codes, ori_ds, ori_tile, ori_r)]
        if cmp_r:
            parts.append(dequant_rows(cmp_codes, cmp_ds, cmp_tile, cmp_r))
        K = np.concatenate(parts, axis=0) if parts else np.zeros((0, d))
        O, l1, l2 = attend_rows(Q, K, inp.softmax_scale, sinks)
        out[t], lse[t], lse_ns[t] = O, l1, l2
    return OracleResult(out=out, lse=lse, lse_nosink=lse_ns, rows=res_rows, tokens=toks)


def work_counts(inp, rows: Dict[int, List[Tuple[int, int]]]) -> Dict[str, float]:
    """Algorithmic work of the listed tokens: (token, key) pairs, rows unique
    per batch, and the fp8 KV bytes those unique rows hold (row + descales)."""
    tt = token_table(inp)
    pairs = sum(len(v) for v in rows.values())
    per_batch: Dict[int, set] = {}
    for t, v in rows.items():
        per_batch.setdefault(tt[t][0], set()).update(v)
    uniq = sum(len(s) for s in per_batch.values())
    fmt = getattr(inp, "kv_format", "fp8")
    if fmt == "bf16":
        row_bytes = 2 * inp.d
    elif fmt == "packed640":
        row_bytes = 640
    else:
        row_bytes = inp.d + (4 * (inp.d // TILE) if inp.kv_scale_mode == 1 else 4)
    return dict(pairs=pairs, unique_rows=uniq, kv_bytes=uniq * row_bytes,
                flops=4.0 * inp.n1 * inp.d * pairs)
