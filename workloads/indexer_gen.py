"""Seeded synthetic inputs for the lightning-indexer top-k (QuantLightningIndexerV2
page, quant_mode 1: fp8 e4m3 query and key with fp32 dequant scales, fp32
weights).  Input construction only: lengths, paged key caches, block tables,
N(0,1) values and their e4m3 quantisation (descale = amax / 448).  Nothing
here computes scores or selects indices.

The index head width is 128 and there are 64 index heads by default; the
workloads reuse the lengths of the attention workloads, the compressed key
count of a batch being the compressed length of its KV (ratio 4).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Sequence

import numpy as np
import torch

from .gen import _contig_cache, _cu, _paged_cache, _randn, quantize_rows_e4m3

D_INDEX = 128
G_INDEX = 64


@dataclass
class IndexerInputs:
    """Every input of one indexer call, in the page's layouts.

    q            uint8 [T1, g, D]  (TND, or BSND flattened as t = b*S1 + s)
    q_scale      f32   [T1, g]     (query_dequant_scale, shaped like weights)
    weights      f32   [T1, g]
    key          uint8 PA_BBND [blocks, block_size, 1, D] | TND [rows, 1, D] | BSND [B, S, 1, D]
    key_scale    f32   the key's shape without (1, D)
    """
    layout_q: str
    layout_k: str
    batch: int
    q_s: int
    q: torch.Tensor
    q_scale: torch.Tensor
    weights: torch.Tensor
    key: torch.Tensor
    key_scale: torch.Tensor
    block_table: Optional[torch.Tensor] = None
    cu_seqlens_q: Optional[torch.Tensor] = None
    seqused_q: Optional[torch.Tensor] = None
    cu_seqlens_k: Optional[torch.Tensor] = None
    seqused_k: Optional[torch.Tensor] = None
    cmp_residual_k: Optional[torch.Tensor] = None
    topk: int = 512
    mask_mode: int = 3
    cmp_ratio: int = 4
    name: str = ""

    @property
    def t1(self) -> int:
        return int(self.q.shape[0])

    @property
    def g(self) -> int:
        return int(self.q.shape[1])

    @property
    def block_size(self) -> int:
        return int(self.key.shape[1]) if self.layout_k == "PA_BBND" else 0

    def to(self, device) -> "IndexerInputs":
        kw = {k: v.to(device) for k, v in self.__dict__.items() if isinstance(v, torch.Tensor)}
        return replace(self, **kw)


def make_indexer(*, seed: int, q_lens: Sequence[int], k_lens: Sequence[int],
                 layout_q: str = "TND", layout_k: str = "PA_BBND", g: int = G_INDEX, d: int = D_INDEX,
                 block_size: int = 128, spare_blocks: int = 3, table_cols: Optional[int] = None,
                 cmp_ratio: int = 4, residual: Optional[Sequence[int]] = None, topk: int = 512,
                 mask_mode: int = 3, seqused_q: Optional[Sequence[int]] = None,
                 weight_scale: Optional[float] = None, device="cpu", name: str = "indexer") -> IndexerInputs:
    """q_lens: query rows per batch (TND span; BSND: S1 for every batch);
    k_lens: compressed index keys per batch."""
    np_rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(2_000_029 * seed + 5)
    B = len(k_lens)
    assert len(q_lens) == B
    if layout_q == "BSND":
        assert len(set(q_lens)) == 1
        q_s = int(q_lens[0])
    else:
        q_s = 0
    T1 = int(sum(q_lens))
    q_codes, q_scale = quantize_rows_e4m3(_randn(gen, (T1, g, d), device))
    ws = g ** -0.5 if weight_scale is None else weight_scale
    weights = (_randn(gen, (T1, g), device) * ws).contiguous()
    out = dict(layout_q=layout_q, layout_k=layout_k, batch=B, q_s=q_s, q=q_codes.contiguous(),
               q_scale=q_scale.contiguous(), weights=weights, topk=int(topk), mask_mode=int(mask_mode),
               cmp_ratio=int(cmp_ratio), name=name)
    if layout_q == "TND":
        out["cu_seqlens_q"] = _cu(q_lens).to(device)
    if seqused_q is not None:
        out["seqused_q"] = torch.as_tensor(np.asarray(seqused_q, dtype=np.int32), device=device)
    if layout_k == "PA_BBND":
        key, ks, tab = _paged_cache(np_rng, gen, k_lens, block_size, d, False, spare_blocks, table_cols, device)
        out.update(key=key, key_scale=ks, block_table=tab)
        out["seqused_k"] = torch.as_tensor(np.asarray(k_lens, dtype=np.int32), device=device)
    else:
        bs_len = max(max(k_lens), 1) if layout_k == "BSND" else None
        key, ks = _contig_cache(gen, k_lens, d, False, device, bs_len)
        out.update(key=key, key_scale=ks)
        if layout_k == "TND":
            out["cu_seqlens_k"] = _cu(k_lens).to(device)
        else:
            out["seqused_k"] = torch.as_tensor(np.asarray(k_lens, dtype=np.int32), device=device)
    if residual is not None:
        out["cmp_residual_k"] = torch.as_tensor(np.asarray(residual, dtype=np.int32), device=device)
    return IndexerInputs(**out)


# ---------------------------------------------------------------------------
# workloads shaped like the CSA attention cases (index keys = compressed KV)
# ---------------------------------------------------------------------------

def _idx_tiny(seed, device):
    return make_indexer(seed=seed, q_lens=[4, 4], k_lens=[75, 50], residual=[0, 0], topk=32,
                        layout_q="TND", device=device, name="idx_tiny")


def _idx_decode(seed, device, batch=32, s2=8192, topk=512):
    ratio = 4
    return make_indexer(seed=seed, q_lens=[1] * batch, k_lens=[s2 // ratio] * batch, residual=[0] * batch,
                        layout_q="BSND", cmp_ratio=ratio, topk=topk, spare_blocks=8, device=device,
                        name="idx_csa_decode")


def _idx_mtp(seed, device, batch=64, lo=65536, hi=131072, topk=512):
    rng = np.random.default_rng(20_000 + seed)
    ratio = 4
    lens = rng.integers(lo, hi + 1, size=batch)
    return make_indexer(seed=seed, q_lens=[2] * batch, k_lens=[int(x) // ratio for x in lens],
                        residual=[int(x) % ratio for x in lens], layout_q="BSND", cmp_ratio=ratio, topk=topk,
                        table_cols=hi // ratio // 128, spare_blocks=8, device=device, name="idx_csa_mtp_long")


def _idx_prefill(seed, device, batch=4, s=4096, topk=512):
    ratio = 4
    return make_indexer(seed=seed, q_lens=[s] * batch, k_lens=[s // ratio] * batch, residual=[0] * batch,
                        layout_q="TND", cmp_ratio=ratio, topk=topk, spare_blocks=4, device=device,
                        name="idx_csa_prefill")


INDEXER_WORKLOADS = {"idx_tiny": _idx_tiny, "idx_csa_decode": _idx_decode, "idx_csa_mtp_long": _idx_mtp,
                     "idx_csa_prefill": _idx_prefill}


def make_indexer_workload(name: str, seed: int = 7, device="cpu", **kw) -> IndexerInputs:
    return INDEXER_WORKLOADS[name](seed, device, **kw)
