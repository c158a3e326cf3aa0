"""Pins of the oracle's bf16 / packed-640 paths (the KvQuantSparseAttnSharedkv
row format and the SparseCompressedFlashAttention bf16 variant) against
things other than themselves:

* the bf16 and e8m0 bit decoders against torch's float types on every code;
* a hand-worked packed row (tests/golden/packed640_row_worked.json);
* a packed problem whose values the fp8 per-tile path can hold exactly gives
  the fp8 path's result bit for bit (two independently written decoders);
* the forward against a brute-force dense masked softmax that decodes the
  caches with torch's own float types, and against torch SDPA in float64.
"""
import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

from oracle import oracle_forward
from oracle.formats import decode_bf16, decode_e8m0, decode_packed640
from workloads import make_custom
from workloads.gen import pack_rows_640
from tests.test_oracle_pins import _assert_close

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_decode_matches_torch_all_codes():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_e8m0_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = decode_e8m0(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)) and nan.sum() == 1 and nan[255]
    assert np.array_equal(ref[~nan], got[~nan])


def _gold_value(v):
    if isinstance(v, str):
        return {"2^-133": 2.0 ** -133, "2^118": 2.0 ** 118, "448 * 2^-27": 448 * 2.0 ** -27}[v]
    return float(v)


def test_packed_row_golden():
    g = json.load(open(os.path.join(GOLD, "packed640_row_worked.json")))
    row = np.zeros(640, dtype=np.uint8)
    row[576:583] = 127                      # unit scales unless the fixture sets them
    for b in g["bytes"]:
        row[b["offset"]] = b["value"]
    vals = decode_packed640(row[None])[0]
    assert vals.shape == (512,)
    for e in g["expected"]:
        assert vals[e["column"]] == _gold_value(e["value"]), e
    # every column not named decodes to zero (the pad byte is ignored)
    named = {e["column"] for e in g["expected"]}
    assert np.all(vals[[c for c in range(512) if c not in named]] == 0)


def test_pack_rows_640_round_trip():
    """The input builder's packing decodes (by the oracle) to the bf16 rope
    and to within e4m3's precision of the nope values, each tile's largest
    magnitude inside e4m3's range."""
    x = torch.randn(50, 512, generator=torch.Generator().manual_seed(3))
    x[3, 64:128] = 0.0                       # an all-zero tile
    rows = pack_rows_640(x).numpy()
    dec = decode_packed640(rows)
    assert np.array_equal(dec[:, :64], x[:, :64].to(torch.bfloat16).double().numpy())
    nope = x[:, 64:].double().numpy()
    scale = np.repeat(decode_e8m0(rows[:, 576:583]), 64, axis=1)
    assert np.all(np.abs(nope) / scale <= 448.0)
    # round to nearest: half a step of e4m3 (relative 2^-4 for normals, 2^-10 absolute below 2^-6)
    assert np.all(np.abs(dec[:, 64:] - nope) <= np.maximum(np.abs(nope) * 2.0 ** -4, scale * 2.0 ** -10))
    assert np.all(dec[3, 64:128] == 0)
    assert np.all(rows[:, 583:] == 0)


def _e4m3_grid_values(rng, shape, scale_pow):
    """Values of the form e4m3 value * 2^scale_pow (exact in bf16 and fp8)."""
    codes = rng.integers(0, 256, size=shape).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30     # no NaN codes
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64) * (2.0 ** scale_pow)
    return codes, v


def test_packed_equals_fp8_per_tile_when_representable():
    """A packed-640 problem with bf16 q, whose rope values and q values are
    e4m3 values times powers of two, is rebuilt as an fp8 problem with
    per-tile KV descales (tile 0 = rope with descale 2^k, tiles 1..7 = nope
    with descale 2^(E - 127)) and per-head q descales 2^j: the two oracle
    paths decode the same numbers, so their outputs agree bit for bit."""
    rng = np.random.default_rng(7)
    q_lens, ori, cmp = [3, 2], [200, 90], [50, 22]
    idx = rng.integers(-1, 55, size=(5, 24))
    base = make_custom(seed=77, q_lens=q_lens, ori_lens=ori, cmp_lens=cmp, cmp_ratio=4, residual=[0, 2],
                       indices=idx, kv_scale_mode=1, return_lse=True, n1=8)
    T1, n1 = base.t1, base.n1
    # q: fp8 codes with descale 2^j per (token, head)  <->  bf16 values
    qj = rng.integers(-8, 3, size=(T1, n1))
    q_codes, _ = _e4m3_grid_values(rng, (T1, n1, 512), 0)
    fp8 = replace(base, q=torch.from_numpy(q_codes), q_descale=torch.from_numpy((2.0 ** qj).astype(np.float32)))
    qv = torch.from_numpy(q_codes).view(torch.float8_e4m3fn).to(torch.float64) * torch.from_numpy(2.0 ** qj)[..., None]
    packed = replace(base, q=qv.to(torch.bfloat16), q_descale=None, q_format="bf16", kv_format="packed640",
                     kv_scale_mode=0)
    assert torch.equal(packed.q.to(torch.float64), qv)
    for which in ("ori", "cmp"):
        kv = getattr(base, f"{which}_kv")            # fp8 codes [blocks, bs, 1, 512]
        nb, bs = kv.shape[0], kv.shape[1]
        n = nb * bs
        codes = kv.reshape(n, 512).numpy().copy()
        codes[(codes & 0x7F) == 0x7F] = 0x30         # the spare (NaN) rows get finite codes here
        e = rng.integers(100, 140, size=(n, 8))      # tile t scale 2^(e - 127)
        ds = (2.0 ** (e - 127)).astype(np.float32)
        fp8_kv = torch.from_numpy(codes).view(nb, bs, 1, 512)
        setattr(fp8, f"{which}_kv", fp8_kv)
        setattr(fp8, f"{which}_kv_descale", torch.from_numpy(ds).view(nb, bs, 8))
        rows = np.zeros((n, 640), dtype=np.uint8)
        rope = torch.from_numpy(codes[:, :64]).view(torch.float8_e4m3fn).to(torch.float64) \
            * torch.from_numpy(2.0 ** (e[:, :1] - 127))
        rows[:, :128] = rope.to(torch.bfloat16).contiguous().view(torch.uint8).numpy().reshape(n, 128)
        assert torch.equal(rope.to(torch.bfloat16).to(torch.float64), rope)   # exact in bf16
        rows[:, 128:576] = codes[:, 64:]
        rows[:, 576:583] = e[:, 1:].astype(np.uint8)
        setattr(packed, f"{which}_kv", torch.from_numpy(rows).view(nb, bs, 1, 640))
        setattr(packed, f"{which}_kv_descale", None)
    a, b = oracle_forward(fp8), oracle_forward(packed)
    assert np.all(np.isfinite(a.out))
    assert np.array_equal(a.out, b.out) and np.array_equal(a.lse, b.lse)


def _torch_rows(inp, which, b, length):
    """Logical rows of batch b decoded with torch's own float types (paged)."""
    kv = getattr(inp, f"{which}_kv")
    tab = getattr(inp, f"{which}_block_table")
    bs = kv.shape[1]
    nb = (length + bs - 1) // bs
    rows = kv[tab[b, :nb].long()].reshape(nb * bs, kv.shape[-1])[:length]
    if inp.kv_format == "bf16":
        return rows.to(torch.float64)
    rope = rows[:, :128].contiguous().view(torch.bfloat16).to(torch.float64)
    nope = rows[:, 128:576].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
    sc = rows[:, 576:583].contiguous().view(torch.float8_e8m0fnu).to(torch.float64)
    return torch.cat([rope, nope * sc.repeat_interleave(64, dim=1)], dim=1)


def _brute(inp, ori, cmp, res):
    """Dense masked softmax over every logical row, masks cell by cell (the
    alignment rules of the fp8 brute force), bf16 q decoded by torch."""
    out = torch.zeros(inp.t1, inp.n1, 512, dtype=torch.float64)
    lse = torch.full((inp.t1, inp.n1), -math.inf, dtype=torch.float64)
    r = inp.cmp_ratio
    t = 0
    for b in range(inp.batch):
        span = int(inp.cu_seqlens_q[b + 1] - inp.cu_seqlens_q[b])
        s2, C, R = ori[b], cmp[b], res[b]
        L = C * r + R
        K_o, K_c = _torch_rows(inp, "ori", b, s2), _torch_rows(inp, "cmp", b, C)
        for i in range(span):
            dq = i - (span - 1)
            keys, ok = [], []
            for j in range(s2):
                dk = j - (s2 - 1)
                keys.append(K_o[j]); ok.append(0 <= dq - dk <= inp.ori_win_left)
            cand = range(C) if inp.cmp_sparse_indices is None else [int(x) for x in inp.cmp_sparse_indices[t, 0]]
            for c in cand:
                keys.append(K_c[c] if 0 <= c < C else torch.zeros(512, dtype=torch.float64))
                ok.append(0 <= c < C and (c * r + r - 1) - (L - 1) <= dq)
            Q = inp.q[t].to(torch.float64)
            K = torch.stack(keys)
            s = Q @ K.T * inp.softmax_scale
            s[:, ~torch.tensor(ok)] = -math.inf
            logits = torch.cat([s, inp.sinks.to(torch.float64)[:, None]], dim=1)
            w = torch.softmax(logits, dim=1)
            out[t] = w[:, :-1] @ K
            lse[t] = torch.logsumexp(logits, dim=1)
            t += 1
    return out, lse


@pytest.mark.parametrize("kv_format", ["bf16", "packed640"])
def test_variant_oracle_vs_brute_force(kv_format):
    rng = np.random.default_rng(11)
    q_lens, ori, r = [3, 4], [190, 77], 4
    cmp = [o // r for o in ori]
    res = [o % r for o in ori]
    idx = rng.integers(-2, max(cmp) + 3, size=(sum(q_lens), 30))
    idx[rng.random(idx.shape) < 0.2] = -1
    idx[0, :3] = idx[0, 0]                   # a duplicate entry
    inp = make_custom(seed=12, q_lens=q_lens, ori_lens=ori, cmp_lens=cmp, cmp_ratio=r, residual=res,
                      indices=idx, n1=4, block_size=16, q_format="bf16", kv_format=kv_format, return_lse=True)
    got = oracle_forward(inp)
    out, lse = _brute(inp, ori, cmp, res)
    _assert_close(got.out, out.numpy())
    _assert_close(got.lse, lse.numpy())


def test_bf16_oracle_vs_sdpa_float64():
    """No mask, no cmp, no sink, bf16 q and KV: plain softmax attention, as
    torch computes it in float64 (scaled_dot_product_attention)."""
    inp = make_custom(seed=33, q_lens=[5], ori_lens=[90], n1=8, block_size=16, ori_mask_mode=0,
                      win_left=-1, win_right=-1, with_sinks=False, cmp_mask_mode=0, softmax_scale=0.05,
                      q_format="bf16", kv_format="bf16")
    res = oracle_forward(inp)
    K = inp.ori_kv[inp.ori_block_table[0, :6].long()].reshape(96, 512)[:90].to(torch.float64)
    Q = inp.q.to(torch.float64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q.transpose(0, 1)[None], K[None, None], K[None, None], scale=0.05)[0].transpose(0, 1)
    _assert_close(res.out, ref.numpy(), 1e-12)


@pytest.mark.parametrize("kv_format", ["bf16", "packed640"])
def test_variant_empty_rows(kv_format):
    """Rows that see no key (more query rows than kv tokens): O = 0 and lse =
    the sink (QuantSparseFlashMla readings R8), in both formats."""
    inp = make_custom(seed=209, q_lens=[9, 4], ori_lens=[5, 300], cmp_lens=[1, 75], cmp_ratio=4, residual=[1, 0],
                      indices=None, n1=4, block_size=16, q_format="bf16", kv_format=kv_format, return_lse=True)
    res = oracle_forward(inp)
    assert np.all(res.out[0] == 0) and np.array_equal(res.lse[0], inp.sinks.double().numpy())
    out, lse = _brute(inp, [5, 300], [1, 75], [1, 0])
    _assert_close(res.out, out.numpy())
    _assert_close(res.lse, lse.numpy())
