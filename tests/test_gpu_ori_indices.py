"""GPU parity of listed ori keys (QuantSparseFlashMla, 参数说明:
ori_sparse_indices with -1 invalid, ori_topk_length): the ori part of K~ is the
listed positions, in slot order, that the ori mask and window admit
(duplicates kept), then the compressed part.  Through the C ABI, against the
oracle; the resolved rows bit-exact."""
import numpy as np
import pytest
import torch

from workloads import make_custom
from tests.test_gpu_parity import check, check_rows, _rand_idx

pytestmark = pytest.mark.gpu


def _ori_rows(rng, t1, k1, hi, p_invalid=0.15):
    idx = rng.integers(-3, hi + 4, size=(t1, k1))
    idx[rng.random(idx.shape) < p_invalid] = -1
    idx[:, 3:6] = idx[:, 2:3]                   # duplicates are separate keys
    return idx


@pytest.mark.parametrize("kv_scale_mode", [0, 1])
def test_decode_band_with_listed_ori_keys(kv_scale_mode):
    """Decode rows over 2000 ori tokens: 200 listed ori slots, some inside the
    127/0 band, with ori_topk_length; CSA compressed indices beside them."""
    rng = np.random.default_rng(301)
    B = 8
    ori, cmp = [2000] * B, [500] * B
    oidx = _ori_rows(rng, B, 200, 2000)
    oidx[:, 10:60] = 2000 - 1 - rng.integers(0, 128, size=(B, 50))   # band positions
    inp = make_custom(seed=302, q_lens=[1] * B, ori_lens=ori, layout_q="BSND", cmp_lens=cmp, cmp_ratio=4,
                      residual=[0] * B, indices=_rand_idx(rng, B, 300, 500, 0.1), kv_scale_mode=kv_scale_mode,
                      ori_indices=oidx, ori_topk_length=rng.integers(40, 210, size=B), return_lse=True)
    check(inp, name=f"listed ori keys, decode, scale mode {kv_scale_mode}")
    check(inp, name=f"listed ori keys, decode, 3 splits", splits=3)
    check_rows(inp, name="listed ori keys, decode")


@pytest.mark.parametrize("case", [
    dict(ori_mask_mode=0, win_left=-1, win_right=-1),
    dict(ori_mask_mode=3, win_left=-1, win_right=-1),
    dict(ori_mask_mode=4, win_left=40, win_right=3),
])
def test_mask_modes_with_listed_ori_keys(case):
    rng = np.random.default_rng(303)
    q_lens, ori = [5, 4], [900, 350]
    cmp = [o // 4 for o in ori]
    T1 = sum(q_lens)
    inp = make_custom(seed=304, q_lens=q_lens, ori_lens=ori, cmp_lens=cmp, cmp_ratio=4,
                      residual=[o % 4 for o in ori], indices=None, ori_indices=_ori_rows(rng, T1, 500, 900),
                      return_lse=True, **case)
    check(inp, name=f"listed ori keys, {case}")
    check_rows(inp, name=f"listed ori keys, {case}")


@pytest.mark.parametrize("fmt", ["bf16", "packed640"])
def test_listed_ori_keys_bf16_q(fmt):
    rng = np.random.default_rng(305)
    q_lens, ori = [3, 3], [700, 260]
    cmp = [o // 4 for o in ori]
    inp = make_custom(seed=306, q_lens=q_lens, ori_lens=ori, cmp_lens=cmp, cmp_ratio=4,
                      residual=[o % 4 for o in ori], indices=_rand_idx(rng, 6, 128, max(cmp), 0.2),
                      ori_indices=_ori_rows(rng, 6, 96, 700), ori_topk_length=[96, 50, 0, 96, 96, 20],
                      q_format="bf16", kv_format=fmt, return_lse=True)
    check(inp, name=f"listed ori keys, {fmt}")
    check_rows(inp, name=f"listed ori keys, {fmt}")


@pytest.mark.parametrize("listed", [True, False])
def test_dominant_ori_key_listed_or_not(listed):
    """A band key scoring ~40 above the rest decides the output when it is
    listed, and is no key at all when its slot holds -1."""
    s2 = 400
    j = s2 - 1 - 30                                   # inside row 0's band [271, 398] (row 0 of 2 at p = 398)
    rows = np.full((2, 64), -1)
    rows[:, 0:40] = np.arange(s2 - 1 - 39, s2)[None, :] - 1
    rows[:, 0:40][rows[:, 0:40] == j] = -1            # j appears only where placed below
    if listed:
        rows[:, 50] = j
    inp = make_custom(seed=307, q_lens=[2], ori_lens=[s2], cmp_lens=[100], cmp_ratio=4, residual=[0],
                      indices=None, ori_indices=rows, return_lse=True)
    q = inp.q[0].clone()
    q[:] = q[0]
    inp.q[0] = q
    inp.q_descale[0] = inp.q_descale[0, 0]
    qq = float((q[0].view(torch.float8_e4m3fn).float() ** 2).sum())
    kds = 40.0 / (float(inp.q_descale[0, 0]) * 512 ** -0.5 * qq)
    bs = inp.ori_kv.shape[1]
    blk = int(inp.ori_block_table[0, j // bs])
    inp.ori_kv[blk, j % bs, 0] = q[0]
    inp.ori_kv_descale[blk, j % bs] = kds
    value = q[0].view(torch.float8_e4m3fn).double().numpy() * kds
    _, o, l, ref = check(inp, tokens=[0], name=f"dominant ori key, listed={listed}")
    assert (np.abs(ref.out[0] - value[None, :]).max() < 1e-3) == listed
    assert (np.abs(o[0] - value[None, :]).max() < 0.05) == listed
