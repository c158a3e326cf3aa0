"""Pins of the CPU oracle against things other than itself.

* fp8 decode vs torch.float8_e4m3fn and the OCP format points (golden)
* visible windows vs hand-worked cases and the fused infer-attention page's
  row-exclusion rules (golden)
* the whole forward vs a brute-force dense masked softmax built from
  per-cell predicates over logical caches (no use of the oracle's window or
  row code), and vs torch scaled_dot_product_attention in float64
* closed forms (one row, n identical rows, dominant sink) and invariants
  (lse identity, CSA(-1 everywhere) == SWA, CSA(permutation) == HCA, index
  order, block placement, split-merge algebra)
"""
import json
from dataclasses import replace
import math
import os

import numpy as np
import pytest
import torch

from oracle import (decode_e4m3, oracle_forward, attend_rows, merge_partials,
                    ori_window, cmp_visible, batch_lengths, token_table)
from oracle.attention import work_counts
from workloads import make_custom, make_config

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- fp8 decode

def test_fp8_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode_e4m3(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(got[~both_nan]))


def test_fp8_decode_golden_points():
    for pt in _gold("fp8_e4m3_points.json")["points"]:
        v = decode_e4m3(np.array([int(pt["code"], 16)]))[0]
        if pt["value"] == "nan":
            assert math.isnan(v)
        else:
            assert v == pt["value"] and math.copysign(1, v) == math.copysign(1, pt["value"])


# ---------------------------------------------------------------- windows

def test_band_window_golden():
    for c in _gold("band_window_worked.json")["cases"]:
        p = c["s2"] - c["s1"] + c["i"]
        assert ori_window(p, c["s2"], c["mode"], c["left"], c["right"]) == (c["lo"], c["hi"]), c


def test_mask_row_exclusion_golden():
    for c in _gold("mask_row_exclusion.json")["cases"]:
        empty = False
        for i in range(c["s_q"]):
            p = c["s_kv"] - c["s_q"] + i
            lo, hi = ori_window(p, c["s_kv"], c["mode"], c["pre"], c["next"])
            empty |= hi <= lo
        assert empty == c["has_empty_rows"], c


def test_cmp_visibility_golden():
    for c in _gold("cmp_visibility_worked.json")["cases"]:
        cl = c["s2"] // c["r"]
        assert cl == c["cmp_len"], c
        assert c["s2"] - cl * c["r"] == c["residual"], c
        L = cl * c["r"] + c["residual"]
        p = L - c["s1"] + c["i"]
        assert cmp_visible(p, cl, c["r"], 3) == c["vis"], c


# ---------------------------------------------------------------- brute force

def _dec_torch(codes):
    return codes.view(torch.float8_e4m3fn).to(torch.float64)


def _logical_cache(kv, ds, table, b, length, per_tile):
    """Logical rows [0, length) of batch b: concatenate its blocks in table order."""
    bs = kv.shape[1]
    if length == 0:
        return torch.zeros(0, kv.shape[-1], dtype=torch.float64)
    nb = (length + bs - 1) // bs
    blocks = table[b, :nb].long()
    codes = kv[blocks].reshape(nb * bs, -1)[:length]
    vals = _dec_torch(codes)
    if per_tile:
        sc = ds[blocks].reshape(nb * bs, -1)[:length].to(torch.float64)
        return vals * sc.repeat_interleave(64, dim=1)
    return vals * ds[blocks].reshape(-1)[:length].to(torch.float64)[:, None]


def _logical_rows(inp, which, b, length, per_tile):
    """Logical rows [0, length) of batch b's ori or cmp cache in any layout:
    paged (table order), TND (the batch's run of a [T, 1, D] cache, found by
    summing the earlier batches' lengths from the cu_seqlens input) or BSND
    (row b of a [B, S, 1, D] cache)."""
    kv = getattr(inp, f"{which}_kv")
    ds = getattr(inp, f"{which}_kv_descale")
    if inp.layout_kv == "PA_BBND":
        return _logical_cache(kv, ds, getattr(inp, f"{which}_block_table"), b, length, per_tile)
    if inp.layout_kv == "TND":
        cu = getattr(inp, f"cu_seqlens_{which}_kv")
        start = int(cu[b])
        codes, sc = kv[start:start + length, 0], ds[start:start + length]
    else:
        codes, sc = kv[b, :length, 0], ds[b, :length]
    vals = _dec_torch(codes)
    if per_tile:
        return vals * sc.to(torch.float64).repeat_interleave(64, dim=1)
    return vals * sc.to(torch.float64)[:, None]


def _brute_force(inp, s2_of=None, c_of=None, r_of=None):
    """Dense masked softmax over every logical row of the batch, with the mask
    written cell by cell from the alignment rules (last query row aligned with
    the last kv token / the last restored token).  Lengths come from
    seqused_ori_kv / seqused_cmp_kv / cmp_residual_kv, unless the caller
    states them (s2_of / c_of / r_of: per-batch lists)."""
    T1, n1, d = inp.t1, inp.n1, inp.d
    per_tile = inp.kv_scale_mode == 1
    out = torch.zeros(T1, n1, d, dtype=torch.float64)
    lse = torch.full((T1, n1), -math.inf, dtype=torch.float64)
    q_off = 0
    for b in range(inp.batch):
        if inp.layout_q == "TND":
            span = int(inp.cu_seqlens_q[b + 1] - inp.cu_seqlens_q[b])
        else:
            span = inp.q_s
        s1 = span if inp.seqused_q is None else min(span, int(inp.seqused_q[b]))
        s2 = int(inp.seqused_ori_kv[b]) if s2_of is None else int(s2_of[b])
        ori = _logical_rows(inp, "ori", b, s2, per_tile)
        r = inp.cmp_ratio
        if inp.cmp_kv is not None:
            C = int(inp.seqused_cmp_kv[b]) if c_of is None else int(c_of[b])
            if r_of is not None:
                R = int(r_of[b])
            else:
                R = int(inp.cmp_residual_kv[b]) if inp.cmp_residual_kv is not None else 0
            L = C * r + R
            cmp = _logical_rows(inp, "cmp", b, C, per_tile)
        for i in range(span):
            t = q_off + i
            if i >= s1:
                continue
            qs = inp.q_descale[t].to(torch.float64)
            Q = _dec_torch(inp.q[t]) * (qs[:, None] if qs.ndim == 1 else qs)
            keys, ok = [], []
            dq = i - (s1 - 1)          # offset of this row from the last query row
            ori_list = getattr(inp, "ori_sparse_indices", None)
            if ori_list is None:
                ori_cand = range(s2)
            else:   # the listed slots, each one key (checked against the mask below)
                ori_cand = [int(x) for x in ori_list[t, 0]]
                if getattr(inp, "ori_topk_length", None) is not None:
                    ori_cand = ori_cand[:max(0, int(inp.ori_topk_length[t]))]
            for j in ori_cand:
                dk = j - (s2 - 1)      # offset of kv token j from the last kv token
                m = inp.ori_mask_mode
                if m == 0:
                    vis = True
                elif m == 3:
                    vis = dk <= dq
                else:
                    vis = (inp.ori_win_left < 0 or dq - dk <= inp.ori_win_left) and \
                          (inp.ori_win_right < 0 or dk - dq <= inp.ori_win_right)
                vis = vis and 0 <= j < s2
                keys.append(ori[j] if 0 <= j < s2 else torch.zeros(d, dtype=torch.float64))
                ok.append(vis)
            if inp.cmp_kv is not None:
                def cvis(c):
                    if not (0 <= c < C):
                        return False
                    if inp.cmp_mask_mode == 0:
                        return True
                    last = c * r + r - 1          # last original token summarised by c
                    return last - (L - 1) <= dq
                if inp.cmp_sparse_indices is None:
                    cand = list(range(C))
                else:
                    cand = [int(x) for x in inp.cmp_sparse_indices[t, 0]]
                    if inp.cmp_topk_length is not None:
                        cand = cand[:max(0, int(inp.cmp_topk_length[t]))]
                for c in cand:
                    keys.append(cmp[c] if 0 <= c < C else torch.zeros(d, dtype=torch.float64))
                    ok.append(cvis(c))
            sig = inp.sinks.to(torch.float64) if inp.sinks is not None else torch.full((n1,), -math.inf,
                                                                                      dtype=torch.float64)
            if not any(ok):
                lse[t] = sig
                continue
            K = torch.stack(keys)
            s = (Q @ K.T) * inp.softmax_scale
            s[:, ~torch.tensor(ok)] = -math.inf
            logits = torch.cat([s, sig[:, None]], dim=1)
            w = torch.softmax(logits, dim=1)
            out[t] = w[:, :-1] @ K
            lse[t] = torch.logsumexp(logits, dim=1)
        q_off += span
    return out, lse


def _cmp_case(seed, **kw):
    rng = np.random.default_rng(seed)
    B = kw.pop("B", 2)
    q_lens = kw.pop("q_lens", [int(x) for x in rng.integers(1, 6, size=B)])
    ori = kw.pop("ori_lens", [int(x) for x in rng.integers(1, 300, size=B)])
    r = kw.pop("r", 4)
    res = [int(x) for x in rng.integers(0, r, size=B)] if kw.pop("use_res", True) else [0] * B
    cmp = [max(0, (o - rs) // r) for o, rs in zip(ori, res)]
    res = [o - c * r if c > 0 else min(rs, o) for o, c, rs in zip(ori, cmp, res)]
    k2 = kw.pop("k2", 16)
    idx = None
    if kw.pop("csa", True):
        idx = rng.integers(-2, max(cmp) + 3, size=(sum(q_lens), k2))
        idx[rng.random(idx.shape) < 0.2] = -1
        if idx.size:
            idx[0, :2] = idx[0, 0]   # a duplicate entry
    return make_custom(seed=seed, q_lens=q_lens, ori_lens=ori, cmp_lens=cmp, cmp_ratio=r,
                       residual=res, indices=idx, n1=kw.pop("n1", 4), d=kw.pop("d", 128),
                       block_size=kw.pop("block_size", 16), **kw)


def _assert_close(a, b, tol=1e-10):
    a, b = np.asarray(a), np.asarray(b)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin)
    assert np.array_equal(a[~fin], b[~fin])
    assert np.max(np.abs(a[fin] - b[fin]), initial=0.0) <= tol


@pytest.mark.parametrize("seed,kw", [
    (1, dict()),
    (2, dict(r=1)),
    (3, dict(r=7, ori_mask_mode=3)),
    (4, dict(r=2, win_left=-1, win_right=0)),
    (5, dict(r=4, win_left=5, win_right=3)),
    (6, dict(r=4, win_left=0, win_right=-1, cmp_mask_mode=0)),
    (7, dict(r=128, ori_lens=[290, 40])),
    (8, dict(csa=False, r=3)),
    (9, dict(csa=False, r=5, ori_mask_mode=0, cmp_mask_mode=0)),
    (10, dict(kv_scale_mode=1)),
    (11, dict(q_lens=[9, 2], ori_lens=[4, 200], r=2)),
    (12, dict(use_res=False, with_sinks=False)),
    (13, dict(layout_q="BSND", q_lens=[3, 3, 3], B=3)),
    (14, dict(topk_length=None, seqused_q=[2, 1], q_lens=[4, 3])),
])
def test_oracle_vs_brute_force(seed, kw):
    inp = _cmp_case(seed, **kw)
    res = oracle_forward(inp)
    out, lse = _brute_force(inp)
    _assert_close(res.out, out.numpy())
    _assert_close(res.lse, lse.numpy())


def test_oracle_vs_brute_force_topk_length_and_swa():
    inp = _cmp_case(21, topk_length=None)
    T1 = inp.t1
    inp.cmp_topk_length = torch.as_tensor(np.random.default_rng(0).integers(0, 20, size=T1).astype(np.int32))
    res = oracle_forward(inp)
    out, lse = _brute_force(inp)
    _assert_close(res.out, out.numpy())
    swa = make_custom(seed=22, q_lens=[3, 5], ori_lens=[70, 33], n1=4, d=128, block_size=16,
                      win_left=10, win_right=2, cmp_mask_mode=0)
    _assert_close(oracle_forward(swa).out, _brute_force(swa)[0].numpy())


@pytest.mark.parametrize("layout_kv,kw", [
    ("TND", dict(q_lens=[3, 1, 4], ori_lens=[150, 37, 260])),
    ("TND", dict(q_lens=[2, 5], ori_lens=[9, 300], kv_scale_mode=1)),
    ("BSND", dict(q_lens=[3, 3, 3], ori_lens=[150, 37, 260], layout_q="BSND")),
    ("BSND", dict(q_lens=[2, 2], ori_lens=[300, 120], layout_q="BSND", kv_scale_mode=1)),
    ("BSND", dict(q_lens=[2, 2], ori_lens=[203, 201], layout_q="BSND")),   # equal cmp lengths (50)
])
def test_oracle_vs_brute_force_contiguous_kv(layout_kv, kw):
    """Contiguous KV caches (QuantSparseFlashMla, 参数说明 layout_kv TND / BSND
    with cu_seqlens_ori_kv / cu_seqlens_cmp_kv): the TND case passes no
    seqused_ori_kv, so the ori length is the cu_seqlens difference; the brute
    force reads each batch's run of the cache itself and is told the lengths
    the cache was built with.  The caches' spare slots hold NaN, so a row
    read from the wrong batch or offset shows.  The compressed length comes
    from cu_seqlens_cmp_kv (TND), from seqused_cmp_kv (BSND, unequal
    lengths), or from the BSND shape when every batch has the same number."""
    kw = dict(kw)
    r = 4
    ori = kw.pop("ori_lens")
    res = [o % r for o in ori]
    cmp = [o // r for o in ori]
    rng = np.random.default_rng(sum(ori))
    T1 = sum(kw["q_lens"])
    idx = rng.integers(-2, max(cmp) + 3, size=(T1, 24))
    idx[rng.random(idx.shape) < 0.2] = -1
    by_shape = layout_kv == "BSND" and len(set(cmp)) == 1
    inp = make_custom(seed=len(ori) + ori[0], ori_lens=ori, cmp_lens=cmp, cmp_ratio=r, residual=res,
                      indices=idx, n1=4, d=128, layout_kv=layout_kv,
                      pass_seqused_cmp=(layout_kv == "BSND" and not by_shape), **kw)
    if layout_kv == "TND" or by_shape:
        assert inp.seqused_cmp_kv is None
    if layout_kv == "TND":
        assert inp.seqused_ori_kv is None and inp.cu_seqlens_ori_kv is not None
    got = oracle_forward(inp)
    out, lse = _brute_force(inp, s2_of=ori, c_of=cmp, r_of=res)
    _assert_close(got.out, out.numpy())
    _assert_close(got.lse, lse.numpy())


def _relayout(inp, layout_kv):
    """The same logical caches (the rows of each batch in order, and their
    descales) laid out as a TND ([T, 1, D] + cu_seqlens) or BSND
    ([B, S, 1, D], NaN past each batch's length) cache."""
    out = {}
    B = inp.batch
    s2 = [int(x) for x in inp.seqused_ori_kv]
    cl = [int(x) for x in inp.seqused_cmp_kv]
    for which, lens in (("ori", s2), ("cmp", cl)):
        kv = getattr(inp, f"{which}_kv")
        ds = getattr(inp, f"{which}_kv_descale")
        tab = getattr(inp, f"{which}_block_table")
        bs = kv.shape[1]
        rows_kv, rows_ds = [], []
        for b in range(B):
            nb = (lens[b] + bs - 1) // bs
            blocks = tab[b, :nb].long()
            rows_kv.append(kv[blocks].reshape(nb * bs, 1, -1)[:lens[b]])
            rows_ds.append(ds[blocks].reshape((nb * bs,) + tuple(ds.shape[2:]))[:lens[b]])
        if layout_kv == "TND":
            out[f"{which}_kv"] = torch.cat(rows_kv)
            out[f"{which}_kv_descale"] = torch.cat(rows_ds)
            out[f"cu_seqlens_{which}_kv"] = torch.as_tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
        else:
            S = max(lens)
            k = torch.full((B, S, 1, kv.shape[-1]), 0x7F, dtype=torch.uint8)
            d_ = torch.full((B, S) + tuple(ds.shape[2:]), float("nan"))
            for b in range(B):
                k[b, :lens[b]] = rows_kv[b]
                d_[b, :lens[b]] = rows_ds[b]
            out[f"{which}_kv"], out[f"{which}_kv_descale"] = k, d_
        out[f"{which}_block_table"] = None
    from dataclasses import replace
    return replace(inp, layout_kv=layout_kv, **out)


@pytest.mark.parametrize("kv_scale_mode", [0, 1])
def test_oracle_layouts_agree(kv_scale_mode):
    """One logical problem as paged, TND and BSND caches: the oracle's result
    is bit-identical (K~ depends only on the logical rows; QuantSparseFlashMla,
    参数说明 layout_kv).  A TND offset or a BSND batch stride that is off by
    one reads another row (or a NaN pad) and fails here."""
    inp = _cmp_case(71, q_lens=[3, 2, 4], ori_lens=[130, 61, 222], B=3, kv_scale_mode=kv_scale_mode)
    base = oracle_forward(inp)
    for lay in ("TND", "BSND"):
        alt = _relayout(inp, lay)
        res = oracle_forward(alt)
        assert np.array_equal(res.out, base.out), lay
        assert np.array_equal(res.lse, base.lse), lay


def test_default_cmp_length_and_residual():
    """Paged caches with neither seqused_cmp_kv nor cmp_residual_kv: the
    reading of QuantSparseFlashMla 约束说明 (the compressed length derived from
    the shapes) takes C = floor(S2 / cmp_ratio) and residual 0.  The brute
    force is told exactly those lengths; a batch whose S2 is not a multiple
    of the ratio makes the restored length L = C r differ from S2."""
    r = 4
    ori = [203, 130]
    cmp_true = [o // r for o in ori]
    rng = np.random.default_rng(5)
    idx = rng.integers(-1, max(cmp_true) + 2, size=(5, 20))
    idx[0:2, 0] = 49     # the last compressed token of batch 0: visible to its rows 0 and 1 only with residual 3
    inp = make_custom(seed=73, q_lens=[3, 2], ori_lens=ori, cmp_lens=cmp_true, cmp_ratio=r,
                      residual=[o % r for o in ori], indices=idx, n1=4, d=128, block_size=16,
                      pass_seqused_cmp=False, pass_residual=False, return_lse=True)
    assert inp.seqused_cmp_kv is None and inp.cmp_residual_kv is None
    got = oracle_forward(inp)
    for b in range(2):
        bl = batch_lengths(inp, b)
        assert (bl["c"], bl["res"], bl["L"]) == (ori[b] // r, 0, (ori[b] // r) * r)
    out, lse = _brute_force(inp, s2_of=ori, c_of=cmp_true, r_of=[0, 0])
    _assert_close(got.out, out.numpy())
    _assert_close(got.lse, lse.numpy())
    # the same problem with the residual passed: the cmp visibility moves for
    # batch 0 (203 = 50 * 4 + 3), so the results differ
    inp_r = make_custom(seed=73, q_lens=[3, 2], ori_lens=ori, cmp_lens=cmp_true, cmp_ratio=r,
                        residual=[o % r for o in ori], indices=idx, n1=4, d=128, block_size=16,
                        pass_seqused_cmp=False, pass_residual=True, return_lse=True)
    out_r, _ = _brute_force(inp_r, s2_of=ori, c_of=cmp_true)
    _assert_close(oracle_forward(inp_r).out, out_r.numpy())
    assert not np.allclose(got.out, oracle_forward(inp_r).out)


def test_oracle_vs_sdpa_float64():
    """No mask, no cmp, no sink: the oracle is softmax attention, which torch
    computes in float64 with scaled_dot_product_attention."""
    inp = make_custom(seed=31, q_lens=[5], ori_lens=[77], n1=8, d=128, block_size=16,
                      ori_mask_mode=0, win_left=-1, win_right=-1, with_sinks=False, cmp_mask_mode=0,
                      softmax_scale=0.07)
    res = oracle_forward(inp)
    K = _logical_cache(inp.ori_kv, inp.ori_kv_descale, inp.ori_block_table, 0, 77, False)
    Q = _dec_torch(inp.q) * inp.q_descale.to(torch.float64)[..., None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q.transpose(0, 1)[None], K[None, None], K[None, None], scale=0.07)[0].transpose(0, 1)
    _assert_close(res.out, ref.numpy(), 1e-12)


def test_sink_equals_sdpa_with_virtual_key():
    """A sink logit is one extra key with a fixed logit and a zero value row."""
    inp = make_custom(seed=32, q_lens=[3], ori_lens=[40], n1=8, d=128, block_size=16,
                      ori_mask_mode=0, win_left=-1, win_right=-1, cmp_mask_mode=0, softmax_scale=0.05)
    res = oracle_forward(inp)
    K = _logical_cache(inp.ori_kv, inp.ori_kv_descale, inp.ori_block_table, 0, 40, False)
    Q = _dec_torch(inp.q) * inp.q_descale.to(torch.float64)[..., None]
    Kx = torch.cat([K, torch.zeros(1, 128, dtype=torch.float64)])
    bias = torch.zeros(8, 3, 41, dtype=torch.float64)
    bias[:, :, 40] = inp.sinks.to(torch.float64)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q.transpose(0, 1), Kx[None].expand(8, -1, -1), Kx[None].expand(8, -1, -1),
        attn_mask=bias, scale=0.05).transpose(0, 1)
    _assert_close(res.out, ref.numpy(), 1e-12)
    from scipy.special import logsumexp
    s = torch.einsum("thd,jd->thj", Q, K).numpy() * 0.05
    lse_ref = logsumexp(np.concatenate([s, np.broadcast_to(inp.sinks.double().numpy()[None, :, None],
                                                           (3, 8, 1))], axis=2), axis=2)
    _assert_close(res.lse, lse_ref, 1e-12)


# ---------------------------------------------------------------- closed forms

def test_single_row_closed_form():
    rng = np.random.default_rng(5)
    Q = rng.standard_normal((4, 64))
    v = rng.standard_normal((1, 64))
    O, lse, _ = attend_rows(Q, v, 0.3, None)
    assert np.allclose(O, np.repeat(v, 4, axis=0), rtol=0, atol=1e-14)
    assert np.allclose(lse, 0.3 * Q @ v[0], atol=1e-14)


def test_identical_rows_closed_form():
    rng = np.random.default_rng(6)
    Q = rng.standard_normal((4, 64))
    v = rng.standard_normal(64)
    n = 7
    sig = rng.standard_normal(4)
    O, lse, _ = attend_rows(Q, np.tile(v, (n, 1)), 0.2, sig)
    s = 0.2 * Q @ v
    w = n * np.exp(s) / (n * np.exp(s) + np.exp(sig))
    assert np.allclose(O, w[:, None] * v[None], atol=1e-13)
    assert np.allclose(lse, np.log(n * np.exp(s) + np.exp(sig)), atol=1e-13)


def test_dominant_sink_closed_form():
    rng = np.random.default_rng(7)
    Q = rng.standard_normal((3, 32))
    K = rng.standard_normal((5, 32))
    O, lse, lns = attend_rows(Q, K, 0.1, np.full(3, 80.0))
    assert np.max(np.abs(O)) < 1e-30
    assert np.allclose(lse, 80.0)
    O2, lse2, _ = attend_rows(Q, np.zeros((0, 32)), 0.1, np.array([1.0, 2.0, -3.0]))
    assert np.all(O2 == 0) and np.array_equal(lse2, [1.0, 2.0, -3.0])
    _, lse3, _ = attend_rows(Q, np.zeros((0, 32)), 0.1, None)
    assert np.all(np.isneginf(lse3))


# ---------------------------------------------------------------- invariants

def test_lse_identity():
    inp = _cmp_case(41, n1=8)
    res = oracle_forward(inp)
    tt = token_table(inp)
    from oracle.attention import dequant_rows, _flat_cache
    codes, ds, _ = _flat_cache(inp.ori_kv, inp.ori_kv_descale, False)
    ccodes, cds, _ = _flat_cache(inp.cmp_kv, inp.cmp_kv_descale, False)
    for t in range(inp.t1):
        rows = res.rows[t]
        if not rows:
            continue
        K = np.concatenate([dequant_rows(codes, ds, False, [r for k, r in rows if k == 0]),
                            dequant_rows(ccodes, cds, False, [r for k, r in rows if k == 1])])
        Q = decode_e4m3(inp.q[t].numpy()) * inp.q_descale[t].double().numpy()[:, None]
        s = inp.softmax_scale * Q @ K.T
        w = np.exp(s - res.lse[t][:, None])
        sig = inp.sinks.double().numpy()
        assert np.allclose(w.sum(1) + np.exp(sig - res.lse[t]), 1.0, atol=1e-12)
        assert np.allclose(w @ K, res.out[t], atol=1e-12)


def test_csa_all_invalid_equals_swa():
    inp = make_config(1)  # SWA tiny, then add a cmp cache whose indices are all -1
    base = oracle_forward(inp)
    csa = make_custom(seed=1, q_lens=[4, 4], ori_lens=[300, 200], layout_q="TND", spare_blocks=3,
                      cmp_lens=[75, 50], cmp_ratio=4, residual=[0, 0],
                      indices=np.full((8, 16), -1), return_lse=True)
    # same q / ori cache bytes (same seed, same draw order), cmp never attended
    assert torch.equal(csa.q, inp.q) and torch.equal(csa.ori_kv, inp.ori_kv)
    res = oracle_forward(csa)
    _assert_close(res.out, base.out, 0.0)
    _assert_close(res.lse, base.lse, 0.0)


def test_csa_permutation_equals_hca():
    rng = np.random.default_rng(3)
    kw = dict(seed=51, q_lens=[3, 2], ori_lens=[250, 190], cmp_lens=[62, 47], cmp_ratio=4,
              residual=[2, 2], n1=4, d=128, block_size=16)
    hca = make_custom(indices=None, **kw)
    tt = None
    rows = []
    for t, (b, i) in enumerate(token_table(hca)):
        bl = batch_lengths(hca, b)
        vis = cmp_visible(bl["L"] - bl["s1"] + i, bl["c"], 4, 3)
        sel = rng.permutation(vis)
        row = np.full(70, -1)
        row[:vis] = sel
        rows.append(row)
    csa = make_custom(indices=np.stack(rows), **kw)
    a, b_ = oracle_forward(hca), oracle_forward(csa)
    _assert_close(a.out, b_.out, 1e-12)
    _assert_close(a.lse, b_.lse, 1e-12)


def test_index_order_and_block_placement_invariance():
    inp = _cmp_case(61, n1=4)
    base = oracle_forward(inp)
    rng = np.random.default_rng(0)
    idx = inp.cmp_sparse_indices.clone()
    for t in range(idx.shape[0]):
        idx[t, 0] = idx[t, 0][torch.as_tensor(rng.permutation(idx.shape[-1]))]
    inp.cmp_sparse_indices = idx
    _assert_close(oracle_forward(inp).out, base.out, 1e-12)
    # move every physical block to a new place and rewrite the tables
    for name, tname in (("ori", "ori_block_table"), ("cmp", "cmp_block_table")):
        kv = getattr(inp, f"{name}_kv")
        ds = getattr(inp, f"{name}_kv_descale")
        perm = torch.as_tensor(rng.permutation(kv.shape[0]))
        newkv = torch.empty_like(kv)
        newds = torch.empty_like(ds)
        newkv[perm] = kv
        newds[perm] = ds
        setattr(inp, f"{name}_kv", newkv)
        setattr(inp, f"{name}_kv_descale", newds)
        setattr(inp, tname, perm[getattr(inp, tname).long()].to(torch.int32))
    _assert_close(oracle_forward(inp).out, base.out, 1e-12)


def test_split_merge_algebra():
    rng = np.random.default_rng(8)
    Q = rng.standard_normal((6, 64))
    K = rng.standard_normal((40, 64))
    sig = rng.standard_normal(6)
    O, lse, _ = attend_rows(Q, K, 0.15, sig)
    for n_split in (1, 2, 3, 7):
        cuts = np.sort(rng.choice(np.arange(1, 40), size=n_split - 1, replace=False))
        parts = []
        for seg in np.split(np.arange(40), cuts):
            s = 0.15 * Q @ K[seg].T
            m = s.max(1)
            e = np.exp(s - m[:, None])
            parts.append((m, e.sum(1), e @ K[seg]))
        parts.append((np.full(6, -np.inf), np.zeros(6), np.zeros((6, 64))))  # an empty split
        O2, lse2 = merge_partials(parts, sig)
        assert np.allclose(O2, O, atol=1e-13) and np.allclose(lse2, lse, atol=1e-13)


def test_work_counts_cfg2_shape():
    """Unique rows of the CSA decode workload: 128 band + 512 cmp per batch."""
    inp = make_config(2, batch=2)
    res = oracle_forward(inp, tokens=[0, 1])
    wc = work_counts(inp, res.rows)
    assert wc["pairs"] == 2 * 640 and wc["unique_rows"] == 2 * 640
    assert wc["kv_bytes"] == 2 * 640 * 516


# ---------------------------------------------------------------- ori_sparse_indices

def _ori_idx_case(seed, k1=48, mode=4, wl=30, wr=5, with_len=True):
    rng = np.random.default_rng(seed)
    q_lens, ori = [3, 4], [260, 120]
    cmp = [o // 4 for o in ori]
    T1 = sum(q_lens)
    oidx = rng.integers(-3, max(ori) + 4, size=(T1, k1))
    oidx[rng.random(oidx.shape) < 0.15] = -1
    oidx[0, 1:4] = oidx[0, 0]                     # duplicates are separate keys
    cidx = rng.integers(-1, max(cmp) + 2, size=(T1, 16))
    return make_custom(seed=seed, q_lens=q_lens, ori_lens=ori, cmp_lens=cmp, cmp_ratio=4,
                       residual=[o % 4 for o in ori], indices=cidx, n1=4, d=128, block_size=16,
                       ori_mask_mode=mode, win_left=wl, win_right=wr, ori_indices=oidx,
                       ori_topk_length=rng.integers(0, k1 + 3, size=T1) if with_len else None, return_lse=True)


@pytest.mark.parametrize("seed,kw", [
    (91, dict()),
    (92, dict(mode=3, wl=-1, wr=-1)),
    (93, dict(mode=0, wl=-1, wr=-1, with_len=False)),
    (94, dict(mode=4, wl=-1, wr=0, k1=300)),
])
def test_ori_indices_vs_brute_force(seed, kw):
    """ori_sparse_indices (QuantSparseFlashMla, 参数说明; reading R12): the
    listed positions in slot order that the ori mask admits, -1 and
    out-of-range slots skipped, duplicates kept, the first ori_topk_length
    slots only; the brute force checks each listed slot against the mask
    cell by cell."""
    inp = _ori_idx_case(seed, **kw)
    res = oracle_forward(inp)
    out, lse = _brute_force(inp)
    _assert_close(res.out, out.numpy())
    _assert_close(res.lse, lse.numpy())


def test_ori_indices_listing_the_window_equals_no_indices():
    """Listing exactly the window's positions (in order, then -1) reproduces
    the window without indices; all -1 leaves only the compressed keys."""
    inp = _ori_idx_case(95, with_len=False)
    base = replace(inp, ori_sparse_indices=None, ori_topk_length=None)
    want = oracle_forward(base)
    tt = token_table(base)
    rows = []
    for t, (b, i) in enumerate(tt):
        bl = batch_lengths(base, b)
        lo, hi = ori_window(bl["s2"] - bl["s1"] + i, bl["s2"], base.ori_mask_mode, base.ori_win_left,
                            base.ori_win_right)
        r = np.full(80, -1)
        r[:hi - lo] = np.arange(lo, hi)
        rows.append(r)
    listed = replace(base, ori_sparse_indices=torch.as_tensor(np.stack(rows)[:, None, :].astype(np.int32)))
    got = oracle_forward(listed)
    _assert_close(got.out, want.out, 0.0)
    _assert_close(got.lse, want.lse, 0.0)
    none = replace(base, ori_sparse_indices=torch.full((base.t1, 1, 8), -1, dtype=torch.int32))
    r0 = oracle_forward(none)
    assert all(all(k == 1 for k, _ in r0.rows[t]) for t in range(base.t1))
