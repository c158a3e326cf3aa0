"""Seeded synthetic workloads shaped like the cases on the QuantSparseFlashMla /
KvQuantSparseAttnSharedkv / SparseCompressedFlashAttention pages.

Only input construction lives here: lengths, paged caches, block tables,
top-k index draws, N(0,1) values and their fp8 e4m3 quantisation with
``descale = amax / 448``.  Nothing here computes attention.

All tensors are ``torch`` tensors on the requested device (CPU by default);
fp8 data is stored as raw ``uint8`` codes (OCP e4m3fn), descales as float32.
Unused cache slots (positions past a batch's length, spare blocks) are filled
with the e4m3 NaN code 0x7F and a NaN descale, so that any read of a slot the
method does not visit poisons the output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Callable, List, Optional, Sequence

import numpy as np
import torch

E4M3_MAX = 448.0
NAN_CODE = 0x7F
N1_DEFAULT = 64
D_DEFAULT = 512
TILE = 64  # per-tile descale granularity along D (KvQuantSparseAttnSharedkv, tile_size)

CONFIG_NAMES = {
    1: "swa_tiny",
    2: "csa_decode",
    3: "hca_decode",
    4: "csa_mtp_long",
    5: "csa_prefill",
}


@dataclass
class Inputs:
    """Every input of one call, in the layouts the pages give.

    q                 uint8  [T1, N1, D]   (TND, or BSND flattened as t = b*Q_S + s); bf16 with q_format "bf16"
    q_descale         f32    [T1, N1]      (None with bf16 q)
    kv_format "bf16": ori_kv / cmp_kv are bf16 [..., D]; "packed640": uint8 [..., 640] rows
    (bf16 rope 64 | e4m3 nope 448 | 7 e8m0 scales | pad); descales None for both
    ori_kv            uint8  [blocks, block_size, 1, D] (PA_BBND) | [T_kv, 1, D] (TND) | [B, S2, 1, D] (BSND)
    ori_kv_descale    f32    same leading dims as ori_kv without (1, D); a trailing [D/64] for per-tile scales
    cmp_kv, cmp_kv_descale   as above, or None (SWA)
    cmp_sparse_indices int32 [T1, 1, K2] or None (HCA / SWA)
    """
    layout_q: str
    layout_kv: str
    batch: int
    q_s: int
    q: torch.Tensor
    q_descale: torch.Tensor
    ori_kv: torch.Tensor
    ori_kv_descale: torch.Tensor
    cmp_kv: Optional[torch.Tensor] = None
    cmp_kv_descale: Optional[torch.Tensor] = None
    cmp_sparse_indices: Optional[torch.Tensor] = None
    ori_sparse_indices: Optional[torch.Tensor] = None   # int32 [T1, 1, K1]: listed ori positions (-1 invalid)
    ori_topk_length: Optional[torch.Tensor] = None      # int32 [T1]
    ori_block_table: Optional[torch.Tensor] = None
    cmp_block_table: Optional[torch.Tensor] = None
    cu_seqlens_q: Optional[torch.Tensor] = None
    cu_seqlens_ori_kv: Optional[torch.Tensor] = None
    cu_seqlens_cmp_kv: Optional[torch.Tensor] = None
    seqused_q: Optional[torch.Tensor] = None
    seqused_ori_kv: Optional[torch.Tensor] = None
    seqused_cmp_kv: Optional[torch.Tensor] = None
    cmp_residual_kv: Optional[torch.Tensor] = None
    cmp_topk_length: Optional[torch.Tensor] = None
    sinks: Optional[torch.Tensor] = None
    softmax_scale: float = 1.0 / math.sqrt(D_DEFAULT)
    cmp_ratio: int = 1
    ori_mask_mode: int = 4
    cmp_mask_mode: int = 3
    ori_win_left: int = 127
    ori_win_right: int = 0
    kv_scale_mode: int = 0          # 0: one descale per KV row; 1: one per 64-wide D tile
    q_format: str = "fp8"           # "fp8" (e4m3 codes + q_descale) or "bf16" (q_descale None)
    kv_format: str = "fp8"          # "fp8" (codes + descales), "bf16" or "packed640" (descales None)
    return_lse: bool = False
    name: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def t1(self) -> int:
        return int(self.q.shape[0])

    @property
    def n1(self) -> int:
        return int(self.q.shape[1])

    @property
    def d(self) -> int:
        return int(self.q.shape[2])

    @property
    def topk(self) -> int:
        return 0 if self.cmp_sparse_indices is None else int(self.cmp_sparse_indices.shape[-1])

    def to(self, device) -> "Inputs":
        kw = {}
        for k, v in self.__dict__.items():
            if isinstance(v, torch.Tensor):
                kw[k] = v.to(device)
        return replace(self, **kw)


# ---------------------------------------------------------------------------
# quantisation of synthetic values (input construction: descale = amax / 448,
# cast to OCP e4m3fn with round-to-nearest-even)
# ---------------------------------------------------------------------------

def quantize_rows_e4m3(x: torch.Tensor, tile: Optional[int] = None):
    """Quantise the last dim of ``x`` (float32) to e4m3 codes.

    tile=None: one descale per row; tile=t: one descale per t-wide slice.
    Returns (uint8 codes with x's shape, float32 descale).
    """
    x = x.float()
    if tile is None:
        amax = x.abs().amax(dim=-1, keepdim=True)
    else:
        xs = x.unflatten(-1, (x.shape[-1] // tile, tile))
        amax = xs.abs().amax(dim=-1, keepdim=True)
    ds = amax / E4M3_MAX
    ds = torch.where(ds > 0, ds, torch.ones_like(ds))
    if tile is None:
        codes = (x / ds).to(torch.float8_e4m3fn).view(torch.uint8)
        return codes, ds.squeeze(-1).contiguous()
    codes = (xs / ds).to(torch.float8_e4m3fn).view(torch.uint8).flatten(-2)
    return codes.contiguous(), ds.squeeze(-1).contiguous()


PACKED_ROW = 640
ROPE = 64
BF16_NAN = 0x7FC0


def pack_rows_640(x: torch.Tensor) -> torch.Tensor:
    """Rows of 512 float32 values as 640-byte packed rows: the first 64 values
    as bf16 (round to nearest even), the other 448 as e4m3 codes with one
    e8m0 scale per 64-wide tile, E = ceil(log2(amax / 448)) + 127 (so every
    value / 2^(E - 127) lies within e4m3's range; E = 127 for an all-zero
    tile), then 57 zero pad bytes."""
    n = x.shape[0]
    out = torch.zeros((n, PACKED_ROW), dtype=torch.uint8, device=x.device)
    out[:, :2 * ROPE] = x[:, :ROPE].to(torch.bfloat16).contiguous().view(torch.uint8).reshape(n, 2 * ROPE)
    nope = x[:, ROPE:].float().unflatten(-1, (7, 64))
    amax = nope.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.ceil(torch.log2(amax / E4M3_MAX)), torch.zeros_like(amax))
    e = e.clamp(-127, 127)
    codes = (nope / torch.pow(2.0, e)[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).flatten(-2)
    out[:, 2 * ROPE:2 * ROPE + 448] = codes
    out[:, 2 * ROPE + 448:2 * ROPE + 455] = (e + 127).to(torch.uint8)
    return out


def _poison_rows(n: int, d: int, kv_format: str, device) -> torch.Tensor:
    """Rows that decode to NaN in every format (unused cache slots)."""
    if kv_format == "bf16":
        return torch.full((n, d), BF16_NAN, dtype=torch.int16, device=device).view(torch.bfloat16)
    if kv_format == "packed640":
        r = torch.full((n, PACKED_ROW), NAN_CODE, dtype=torch.uint8, device=device)
        r[:, 0:2 * ROPE:2] = 0xC0
        r[:, 1:2 * ROPE:2] = 0x7F
        r[:, 2 * ROPE + 448:2 * ROPE + 455] = 0xFF
        r[:, 2 * ROPE + 455:] = 0
        return r
    return torch.full((n, d), NAN_CODE, dtype=torch.uint8, device=device)


def _encode_rows(vals: torch.Tensor, kv_format: str, per_tile: bool):
    """(rows in the cache's storage type, descales or None)."""
    if kv_format == "bf16":
        return vals.to(torch.bfloat16), None
    if kv_format == "packed640":
        return pack_rows_640(vals), None
    return quantize_rows_e4m3(vals, TILE if per_tile else None)


def _randn(gen: torch.Generator, shape, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _paged_cache(np_rng, gen, lengths: Sequence[int], block_size: int, d: int,
                 per_tile: bool, spare_blocks: int, table_cols: Optional[int], device, kv_format: str = "fp8"):
    """Build a paged cache [blocks, block_size, 1, row] holding N(0,1) rows for
    positions [0, len_b) of each batch, with a random permutation of physical
    block ids.  Unused table slots point at a NaN-poisoned spare block."""
    nblk = [(int(s) + block_size - 1) // block_size for s in lengths]
    used = sum(nblk)
    spare_blocks = max(1, spare_blocks)
    total = used + spare_blocks
    perm = np_rng.permutation(total).astype(np.int64)
    cols = max(max(nblk) if nblk else 1, 1) if table_cols is None else table_cols
    assert cols >= max(nblk + [0])
    spare_id = int(perm[used])
    table = np.full((len(lengths), cols), spare_id, dtype=np.int32)
    poison = _poison_rows(total * block_size, d, kv_format, device)
    width = poison.shape[-1]
    pool = poison.view(total, block_size, 1, width)
    pool_ds = None
    if kv_format == "fp8":
        ds_shape = (total, block_size, d // TILE) if per_tile else (total, block_size)
        pool_ds = torch.full(ds_shape, float("nan"), dtype=torch.float32, device=device)
    off = 0
    for b, s in enumerate(lengths):
        ids = perm[off:off + nblk[b]]
        off += nblk[b]
        table[b, :nblk[b]] = ids
        if s == 0:
            continue
        vals = _randn(gen, (int(s), d), device)
        rows, ds = _encode_rows(vals, kv_format, per_tile)
        pad = nblk[b] * block_size - int(s)
        ids_t = torch.as_tensor(ids, device=device)
        if pad:
            rows = torch.cat([rows, _poison_rows(pad, d, kv_format, device)])
            if ds is not None:
                ds = torch.cat([ds, torch.full((pad,) + tuple(ds.shape[1:]), float("nan"), device=device)])
        pool[ids_t] = rows.view(nblk[b], block_size, 1, width)
        if ds is not None:
            pool_ds[ids_t] = ds.view((nblk[b], block_size) + tuple(ds.shape[1:]))
    return pool, pool_ds, torch.as_tensor(table, device=device)


def _contig_cache(gen, lengths, d, per_tile, device, bsnd_len: Optional[int], kv_format: str = "fp8"):
    """TND ([sum len, 1, row]) or BSND ([B, S2max, 1, row]) contiguous cache."""
    if bsnd_len is None:
        total = int(sum(lengths))
        vals = _randn(gen, (max(total, 1), d), device)[:total]
        rows, ds = _encode_rows(vals, kv_format, per_tile)
        return rows.view(total, 1, rows.shape[-1]), ds
    B = len(lengths)
    poison = _poison_rows(B * bsnd_len, d, kv_format, device)
    width = poison.shape[-1]
    codes = poison.view(B, bsnd_len, 1, width)
    dsall = None
    if kv_format == "fp8":
        ds_shape = (B, bsnd_len, d // TILE) if per_tile else (B, bsnd_len)
        dsall = torch.full(ds_shape, float("nan"), dtype=torch.float32, device=device)
    for b, s in enumerate(lengths):
        if s:
            c, ds = _encode_rows(_randn(gen, (int(s), d), device), kv_format, per_tile)
            codes[b, :s, 0] = c
            if ds is not None:
                dsall[b, :s] = ds
    return codes, dsall


def _cu(lengths) -> torch.Tensor:
    return torch.as_tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))


def make_custom(*, seed: int, q_lens: Sequence[int], ori_lens: Sequence[int],
                layout_q: str = "TND", layout_kv: str = "PA_BBND",
                cmp_lens: Optional[Sequence[int]] = None, cmp_ratio: int = 1,
                residual: Optional[Sequence[int]] = None,
                indices: Optional[np.ndarray] = None,
                topk_length: Optional[Sequence[int]] = None,
                seqused_q: Optional[Sequence[int]] = None,
                block_size: int = 128, spare_blocks: int = 3, table_cols: Optional[int] = None,
                cmp_block_size: Optional[int] = None,
                kv_scale_mode: int = 0, with_sinks: bool = True,
                softmax_scale: float = 1.0 / math.sqrt(D_DEFAULT),
                ori_mask_mode: int = 4, cmp_mask_mode: int = 3,
                win_left: int = 127, win_right: int = 0,
                return_lse: bool = False, device="cpu",
                n1: int = N1_DEFAULT, d: int = D_DEFAULT,
                pass_seqused_cmp: bool = True, pass_residual: bool = True,
                q_descale_per_head: bool = True, q_format: str = "fp8", kv_format: str = "fp8",
                ori_indices: Optional[np.ndarray] = None, ori_topk_length: Optional[Sequence[int]] = None,
                name: str = "custom") -> Inputs:
    """General builder: explicit per-batch lengths, modes and (optional) index array.

    q_lens: per-batch query rows (TND span, or Q_S for every batch in BSND).
    indices: int32 [T1, K2] or None; cmp_lens None means SWA (no cmp_kv).
    """
    np_rng = np.random.default_rng(seed)
    gen = torch.Generator(device=device)
    gen.manual_seed(1_000_003 * seed + 17)
    B = len(ori_lens)
    per_tile = kv_scale_mode == 1
    if layout_q == "BSND":
        assert len(set(q_lens)) == 1
        q_s = int(q_lens[0])
    else:
        q_s = 0
    T1 = int(sum(q_lens))
    qv = _randn(gen, (T1, n1, d), device)
    q_codes, q_ds = quantize_rows_e4m3(qv)
    if q_format == "bf16":
        q_codes, q_ds = qv.to(torch.bfloat16), None
    elif not q_descale_per_head:
        # one descale per token: re-quantise each token with its global amax
        amax = qv.abs().amax(dim=(1, 2))
        ds = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
        q_codes = (qv / ds[:, None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
        q_ds = ds.contiguous()

    sinks = _randn(gen, (n1,), device) if with_sinks else None
    out = dict(layout_q=layout_q, layout_kv=layout_kv, batch=B, q_s=q_s, sinks=sinks,
               q=q_codes.contiguous(), q_descale=None if q_ds is None else q_ds.contiguous(),
               softmax_scale=float(softmax_scale), cmp_ratio=int(cmp_ratio),
               ori_mask_mode=ori_mask_mode, cmp_mask_mode=cmp_mask_mode,
               ori_win_left=win_left, ori_win_right=win_right,
               kv_scale_mode=kv_scale_mode, q_format=q_format, kv_format=kv_format,
               return_lse=return_lse, name=name)
    if layout_q == "TND":
        out["cu_seqlens_q"] = _cu(q_lens).to(device)
    if seqused_q is not None:
        out["seqused_q"] = torch.as_tensor(np.asarray(seqused_q, dtype=np.int32), device=device)
    if ori_indices is not None:
        out["ori_sparse_indices"] = torch.as_tensor(np.asarray(ori_indices, dtype=np.int32).reshape(T1, 1, -1),
                                                    device=device)
    if ori_topk_length is not None:
        out["ori_topk_length"] = torch.as_tensor(np.asarray(ori_topk_length, dtype=np.int32), device=device)

    if layout_kv == "PA_BBND":
        kv, kds, tab = _paged_cache(np_rng, gen, ori_lens, block_size, d, per_tile, spare_blocks, table_cols, device,
                                    kv_format)
        out.update(ori_kv=kv, ori_kv_descale=kds, ori_block_table=tab)
        out["seqused_ori_kv"] = torch.as_tensor(np.asarray(ori_lens, dtype=np.int32), device=device)
    else:
        bs_len = max(ori_lens) if layout_kv == "BSND" else None
        kv, kds = _contig_cache(gen, ori_lens, d, per_tile, device, bs_len, kv_format)
        out.update(ori_kv=kv, ori_kv_descale=kds)
        if layout_kv == "TND":
            out["cu_seqlens_ori_kv"] = _cu(ori_lens).to(device)
        else:
            out["seqused_ori_kv"] = torch.as_tensor(np.asarray(ori_lens, dtype=np.int32), device=device)

    if cmp_lens is not None:
        cbs = cmp_block_size or block_size
        if layout_kv == "PA_BBND":
            ckv, cds, ctab = _paged_cache(np_rng, gen, cmp_lens, cbs, d, per_tile, spare_blocks, None, device,
                                          kv_format)
            out.update(cmp_kv=ckv, cmp_kv_descale=cds, cmp_block_table=ctab)
        else:
            bs_len = max(max(cmp_lens), 1) if layout_kv == "BSND" else None
            ckv, cds = _contig_cache(gen, cmp_lens, d, per_tile, device, bs_len, kv_format)
            out.update(cmp_kv=ckv, cmp_kv_descale=cds)
            if layout_kv == "TND":
                out["cu_seqlens_cmp_kv"] = _cu(cmp_lens).to(device)
        if pass_seqused_cmp:
            out["seqused_cmp_kv"] = torch.as_tensor(np.asarray(cmp_lens, dtype=np.int32), device=device)
        if pass_residual and residual is not None:
            out["cmp_residual_kv"] = torch.as_tensor(np.asarray(residual, dtype=np.int32), device=device)
        if indices is not None:
            idx = np.asarray(indices, dtype=np.int32).reshape(T1, 1, -1)
            out["cmp_sparse_indices"] = torch.as_tensor(idx, device=device)
        if topk_length is not None:
            out["cmp_topk_length"] = torch.as_tensor(np.asarray(topk_length, dtype=np.int32), device=device)
    return Inputs(**out)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def _uniform_draw(rng, hi: int, k: int) -> np.ndarray:
    """k distinct integers drawn uniformly from [0, hi), shuffled."""
    if k <= 0:
        return np.zeros(0, dtype=np.int32)
    return rng.choice(hi, size=k, replace=False).astype(np.int32)


def _fmt(kw):
    """The q / KV format keywords of a config (fp8 by default); the per-tile
    descale mode applies to fp8 rows only."""
    return dict(q_format=kw.get("q_format", "fp8"), kv_format=kw.get("kv_format", "fp8"))


def _swa_tiny(seed, device, **fmt):
    return make_custom(seed=seed, q_lens=[4, 4], ori_lens=[300, 200], layout_q="TND",
                       spare_blocks=3, return_lse=True, device=device, name="swa_tiny", **_fmt(fmt))


def _csa_decode_indices(rng, batch, c, topk):
    """One decode row per batch at position s2 - 1 sees every compressed token:
    topk distinct ones drawn uniformly."""
    return np.stack([_uniform_draw(rng, c, topk) for _ in range(batch)])


def _csa_decode(seed, device, batch=32, s2=8192, topk=512, layout_q="BSND", **fmt):
    rng = np.random.default_rng(10_000 + seed)
    ratio = 4
    c = s2 // ratio
    idx = _csa_decode_indices(rng, batch, c, topk)
    return make_custom(seed=seed, q_lens=[1] * batch, ori_lens=[s2] * batch, layout_q=layout_q,
                       cmp_lens=[c] * batch, cmp_ratio=ratio, residual=[0] * batch,
                       indices=idx, spare_blocks=8, device=device, name="csa_decode", **_fmt(fmt))


def _hca_decode(seed, device, batch=32, lo=32768, hi=65536, **fmt):
    rng = np.random.default_rng(10_000 + seed)
    ratio = 128
    lens = rng.integers(lo, hi + 1, size=batch)
    cmp = [int(x) // ratio for x in lens]
    res = [int(x) % ratio for x in lens]
    return make_custom(seed=seed, q_lens=[1] * batch, ori_lens=[int(x) for x in lens], layout_q="BSND",
                       cmp_lens=cmp, cmp_ratio=ratio, residual=res, indices=None,
                       table_cols=hi // 128, spare_blocks=8, device=device, name="hca_decode", **_fmt(fmt))


def _csa_mtp_indices(rng, lens, s_q, ratio, topk, recent):
    """Per query row: the `recent` most recent visible compressed tokens plus
    uniform draws from the older ones, shuffled, -1 padded."""
    rows = []
    for b in range(len(lens)):
        L = int(lens[b])
        for i in range(s_q):
            # compressed tokens whose whole span lies at or before this row's position
            vis = (L - s_q + i + 1) // ratio
            k_recent = min(recent, vis)
            near = np.arange(vis - k_recent, vis, dtype=np.int32)
            far = _uniform_draw(rng, vis - k_recent, min(topk - k_recent, vis - k_recent))
            sel = np.concatenate([near, far])
            rng.shuffle(sel)
            row = np.full(topk, -1, dtype=np.int32)
            row[:len(sel)] = sel
            rows.append(row)
    return np.stack(rows)


def _csa_mtp(seed, device, batch=64, lo=65536, hi=131072, topk=512, recent=256, **fmt):
    rng = np.random.default_rng(10_000 + seed)
    ratio = 4
    s_q = 2
    lens = rng.integers(lo, hi + 1, size=batch)
    cmp = [int(x) // ratio for x in lens]
    res = [int(x) % ratio for x in lens]
    rows = _csa_mtp_indices(rng, lens, s_q, ratio, topk, recent)
    return make_custom(seed=seed, q_lens=[s_q] * batch, ori_lens=[int(x) for x in lens], layout_q="BSND",
                       cmp_lens=cmp, cmp_ratio=ratio, residual=res, indices=rows,
                       table_cols=hi // 128, spare_blocks=8, device=device, name="csa_mtp_long", **_fmt(fmt))


def _csa_prefill(seed, device, batch=4, s=4096, topk=512, **fmt):
    rng = np.random.default_rng(10_000 + seed)
    ratio = 4
    c = s // ratio
    rows = np.full((batch * s, topk), -1, dtype=np.int32)
    for b in range(batch):
        for p in range(s):
            vis = (p + 1) // ratio
            k = min(topk, vis)
            rows[b * s + p, :k] = _uniform_draw(rng, vis, k)
    return make_custom(seed=seed, q_lens=[s] * batch, ori_lens=[s] * batch, layout_q="TND",
                       cmp_lens=[c] * batch, cmp_ratio=ratio, residual=[0] * batch, indices=rows,
                       kv_scale_mode=1 if _fmt(fmt)["kv_format"] == "fp8" else 0, spare_blocks=4,
                       return_lse=True, device=device, name="csa_prefill", **_fmt(fmt))


def redraw_query_side(inp: Inputs, k: int, draw: int) -> Inputs:
    """The same workload with a new draw of everything a model layer owns on
    the query side: q and its descales, and (for the CSA configs) the top-k
    index rows, by the config's own recipe.  The lengths, block tables,
    sinks and the caches' bytes are shared (the caller replaces the caches
    with copies of its own).  Tensors are made on inp's device."""
    dev = inp.q.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(7_000_003 * (draw + 1) + k)
    qv = _randn(gen, tuple(inp.q.shape), dev)
    if inp.q_format == "bf16":
        out = replace(inp, q=qv.to(torch.bfloat16).contiguous(), q_descale=None)
    else:
        q_codes, q_ds = quantize_rows_e4m3(qv)
        out = replace(inp, q=q_codes.contiguous(), q_descale=q_ds.contiguous())
    if inp.cmp_sparse_indices is None:
        return out
    rng = np.random.default_rng(20_000 + 1000 * k + draw)
    topk = inp.topk
    if k == 2:
        c = int(inp.seqused_cmp_kv[0])
        idx = _csa_decode_indices(rng, inp.batch, c, topk)
    elif k == 4:
        lens = inp.seqused_ori_kv.cpu().numpy()
        idx = _csa_mtp_indices(rng, lens, inp.q_s, inp.cmp_ratio, topk, 256)
    else:
        raise ValueError(f"no query-side redraw recipe for config {k}")
    out.cmp_sparse_indices = torch.as_tensor(idx.reshape(inp.t1, 1, topk), device=dev)
    return out


def make_config(k: int, seed: Optional[int] = None, device="cpu", **kw) -> Inputs:
    """Workload k (1..5) with seed k by default; keyword overrides shrink it."""
    seed = k if seed is None else seed
    fn = {1: _swa_tiny, 2: _csa_decode, 3: _hca_decode, 4: _csa_mtp, 5: _csa_prefill}[k]
    return fn(seed, device, **kw)
