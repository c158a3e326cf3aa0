"""GPU parity of the bf16-q paths against the CPU oracle, through the C ABI:
bf16 q with bf16 KV rows (SparseCompressedFlashAttention) and bf16 q with
packed 640-byte KV rows (KvQuantSparseAttnSharedkv: bf16 rope, e4m3 nope,
e8m0 tile scales).  Same bar as the fp8 paths: every bf16 output element
within 1e-2 + 1e-2 |ref|, lse within 1e-3, the resolved gather rows bit-exact;
unused cache slots hold NaN so that a stray read shows."""
import os

import numpy as np
import pytest
import torch

import sparse_compressed_mla_amd as m
from oracle import oracle_forward
from workloads import make_custom
from tests.test_gpu_parity import check, check_rows, say, DEV, _rand_idx

pytestmark = pytest.mark.gpu

FORMATS = ["bf16", "packed640"]


def _mk(fmt, **kw):
    return make_custom(q_format="bf16", kv_format=fmt, **kw)


@pytest.mark.parametrize("fmt", FORMATS)
def test_csa_decode_shape(fmt):
    """The CSA decode configuration's shape: 32 decode rows, ori 8192 (band
    128), 2048 compressed tokens, 512 top-k indices drawn without
    replacement."""
    rng = np.random.default_rng(201)
    B = 32
    idx = np.stack([rng.choice(2048, 512, replace=False) for _ in range(B)])
    inp = _mk(fmt, seed=202, q_lens=[1] * B, ori_lens=[8192] * B, layout_q="BSND", cmp_lens=[2048] * B,
              cmp_ratio=4, residual=[0] * B, indices=idx, spare_blocks=8, return_lse=True)
    stats, *_ = check(inp, name=f"{fmt} csa decode B=32")
    check_rows(inp, name=f"{fmt} csa decode")


@pytest.mark.parametrize("fmt", FORMATS)
def test_csa_prefill_shape(fmt):
    """Prefill rows as in the CSA prefill configuration (k = min(512, visible)
    indices per row, -1 padded, lse returned), two sequences of 700."""
    rng = np.random.default_rng(203)
    s, r = 700, 4
    rows = np.full((2 * s, 512), -1)
    for b in range(2):
        for p in range(s):
            vis = (p + 1) // r
            k = min(512, vis)
            rows[b * s + p, :k] = rng.choice(vis, k, replace=False) if k else []
    inp = _mk(fmt, seed=204, q_lens=[s, s], ori_lens=[s, s], cmp_lens=[s // r] * 2, cmp_ratio=r, residual=[0, 0],
              indices=rows, return_lse=True)
    check(inp, tokens=list(range(0, 2 * s, 3)) + [s - 1, s, 2 * s - 1], name=f"{fmt} csa prefill 2x700")
    check_rows(inp, name=f"{fmt} csa prefill")


@pytest.mark.parametrize("fmt", FORMATS)
def test_hca_and_swa(fmt):
    inp = _mk(fmt, seed=205, q_lens=[2, 3], ori_lens=[5000, 2600], cmp_lens=[39, 20], cmp_ratio=128,
              residual=[5000 % 128, 2600 % 128], indices=None, layout_q="TND", return_lse=True)
    check(inp, name=f"{fmt} hca")
    check_rows(inp, name=f"{fmt} hca")
    swa = _mk(fmt, seed=206, q_lens=[4, 4], ori_lens=[300, 200], return_lse=True)
    check(swa, name=f"{fmt} swa tiny")


@pytest.mark.parametrize("fmt", FORMATS)
def test_edges_invalid_duplicate_topk_length_padding(fmt):
    rng = np.random.default_rng(207)
    q_lens, ori = [3, 5, 1], [700, 260, 90]
    cmp = [o // 4 for o in ori]
    idx = _rand_idx(rng, sum(q_lens), 300, max(cmp))
    idx[0, 10:20] = idx[0, 0]
    inp = _mk(fmt, seed=208, q_lens=q_lens, ori_lens=ori, cmp_lens=cmp, cmp_ratio=4,
              residual=[o % 4 for o in ori], indices=idx, seqused_q=[3, 4, 1],
              topk_length=rng.integers(0, 300, size=sum(q_lens)), return_lse=True)
    check(inp, name=f"{fmt} invalid/dup/topk_length/padding")
    check(inp, name=f"{fmt} invalid/dup/topk_length/padding, 3 splits", splits=3)
    check_rows(inp, name=f"{fmt} invalid/dup")
    for sinks in (True, False):   # rows that see nothing
        e = _mk(fmt, seed=209, q_lens=[9, 4], ori_lens=[5, 300], cmp_lens=[1, 75], cmp_ratio=4, residual=[1, 0],
                indices=None, with_sinks=sinks, return_lse=True)
        check(e, name=f"{fmt} empty rows, sinks={sinks}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("case", [
    dict(ori_mask_mode=0, win_left=-1, win_right=-1, cmp_mask_mode=0, ori=[1500, 3000]),   # > 1024 keys a row
    dict(ori_mask_mode=3, win_left=-1, win_right=-1, ori=[2100, 40]),
    dict(ori_mask_mode=4, win_left=5, win_right=9, ori=[300, 31]),
])
def test_mask_modes(fmt, case):
    case = dict(case)
    ori = case.pop("ori")
    r = 7
    inp = _mk(fmt, seed=210, q_lens=[6, 6], ori_lens=ori, cmp_lens=[o // r for o in ori], cmp_ratio=r,
              residual=[o % r for o in ori], indices=None, layout_q="BSND", return_lse=True, **case)
    check(inp, name=f"{fmt} mask {case}")
    check_rows(inp, name=f"{fmt} mask {case}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("layout_kv", ["TND", "BSND"])
def test_contiguous_kv_layouts(fmt, layout_kv):
    rng = np.random.default_rng(211)
    ori = [333, 150, 700]
    cmp = [o // 4 for o in ori]
    lq = "TND" if layout_kv == "TND" else "BSND"
    q_lens = [3, 2, 4] if lq == "TND" else [3, 3, 3]
    idx = _rand_idx(rng, sum(q_lens), 128, max(cmp), 0.1)
    inp = _mk(fmt, seed=212, q_lens=q_lens, ori_lens=ori, cmp_lens=cmp, cmp_ratio=4, residual=[0, 0, 0],
              indices=idx, layout_q=lq, layout_kv=layout_kv, return_lse=True)
    check(inp, name=f"{fmt} kv layout {layout_kv}")
    check_rows(inp, name=f"{fmt} kv layout {layout_kv}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_block_sizes_and_128_heads(fmt):
    rng = np.random.default_rng(213)
    ori = [1100, 517]
    cmp = [o // 4 for o in ori]
    idx = _rand_idx(rng, 4, 64, max(cmp), 0.3)
    inp = _mk(fmt, seed=214, q_lens=[2, 2], ori_lens=ori, cmp_lens=cmp, cmp_ratio=4,
              residual=[o % 4 for o in ori], indices=idx, block_size=96, cmp_block_size=24, return_lse=True)
    check(inp, name=f"{fmt} blocks 96 / 24")
    inp = _mk(fmt, seed=215, q_lens=[3, 3], ori_lens=[900, 400], cmp_lens=[225, 100], cmp_ratio=4,
              residual=[0, 0], indices=_rand_idx(rng, 6, 80, 225, 0.2), n1=128, return_lse=True)
    check(inp, name=f"{fmt} n1 128")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("off", [-128, -127, 0])
@pytest.mark.parametrize("mixed", [False, True])
def test_dominant_band_key(fmt, off, mixed):
    """Row 0 of a 2-row batch over 400 ori tokens sits at p = 398 (band
    [271, 398]); its query is a scaled copy of the key at p + off, which
    scores ~40 above the rest: the output follows that key's value row iff
    the key is in the band.  Mixed: only the even heads get that query, so
    in the tile holding the key some heads' softmax maxima jump and the
    others' do not."""
    inp = _mk(fmt, seed=216, q_lens=[2], ori_lens=[400], cmp_lens=[100], cmp_ratio=4, residual=[0],
              indices=None, return_lse=True)
    p = 398
    j = p + off
    bs = inp.ori_kv.shape[1]
    blk = int(inp.ori_block_table[0, j // bs])
    row = inp.ori_kv[blk, j % bs, 0]
    if fmt == "bf16":
        kvec = row.double()
    else:
        from oracle.formats import decode_packed640
        kvec = torch.from_numpy(decode_packed640(row.numpy()[None])[0])
    scale = 40.0 / (512 ** -0.5 * float((kvec ** 2).sum()))
    heads = slice(0, inp.n1, 2) if mixed else slice(0, inp.n1)
    dom = (kvec * scale).to(torch.bfloat16)[None, :]
    inp.q[0, heads] = dom.expand(inp.q[0, heads].shape[0], -1)
    _, o, l, ref = check(inp, tokens=[0], name=f"{fmt} dominant band {off}{' mixed' if mixed else ''}")
    visible = -127 <= off <= 0
    val = kvec.numpy()
    assert (np.abs(ref.out[0][heads] - val[None, :]).max() < 1e-2) == visible
    assert (np.abs(o[0][heads] - val[None, :]).max() < 0.05) == visible
