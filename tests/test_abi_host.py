"""Host-side tests of the C ABI (no GPU): exported symbols, the validation
matrix of the QuantSparseFlashMla page's constraints, the planner's
invariants, and the errors csmla_forward reports before any launch."""
import copy
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_compressed_mla_amd as m
from sparse_compressed_mla_amd.binding import CsmlaProblem, CsmlaHostLengths, CsmlaTensors

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, INVALID, UNSUPPORTED, WORKSPACE, MISMATCH = 0, 1, 2, 3, 4
WS_FIXED = 4096 + 256 * 33792   # sync words + exchange slots, at the start of every workspace


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            src = open(os.path.join(ROOT, "include", h)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(csmla_\w+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = m.load()
    names = declared_functions()
    assert len(names) >= 12 and "csmla_indexer_forward" in names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strings():
    assert m.csmla_abi_version() == 2
    assert m.csmla_metadata_words() == 1024
    for s in range(6):
        assert m.csmla_status_string(s)
    assert m.csmla_status_string(99) == "unknown status"


def base_problem(**kw):
    p = CsmlaProblem()
    vals = dict(batch=32, n1=64, n2=1, d=512, layout_q=0, layout_kv=2, q_s=1, t1=32,
                ori_block_size=128, cmp_block_size=128, ori_num_blocks=2056, cmp_num_blocks=520,
                ori_table_cols=64, cmp_table_cols=16, has_cmp=1, topk=512, softmax_scale=512 ** -0.5,
                cmp_ratio=4, ori_mask_mode=4, cmp_mask_mode=3, ori_win_left=127, ori_win_right=0,
                kv_scale_mode=0, q_descale_per_head=1, topk_value_mode=0, return_softmax_lse=0)
    vals.update(kw)
    for k, v in vals.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,status", [
    (dict(), OK),
    (dict(n2=2), INVALID),                      # N2 only 1
    (dict(d=576), INVALID),                     # D only 512
    (dict(n1=128), OK),                         # N1 = 128 (KvQuantSparseAttnSharedkv): two 64-head launches
    (dict(n1=96), UNSUPPORTED),                 # only 64 and 128 are built
    (dict(n1=32), UNSUPPORTED),
    (dict(batch=0, t1=0), INVALID),             # empty tensors
    (dict(cmp_ratio=0), INVALID),
    (dict(cmp_ratio=129), INVALID),             # 1..128
    (dict(has_cmp=0, topk=0, cmp_ratio=4), INVALID),   # SWA keeps cmp_ratio 1
    (dict(has_cmp=0, topk=0, cmp_ratio=1), OK),
    (dict(has_cmp=0, topk=16, cmp_ratio=1), INVALID),  # indices need cmp_kv
    (dict(ori_mask_mode=1), INVALID),           # 0/3/4
    (dict(cmp_mask_mode=4), INVALID),           # 0/3
    (dict(ori_mask_mode=3, ori_win_left=127, ori_win_right=0), INVALID),   # windows >= 0 only with band
    (dict(ori_mask_mode=3, ori_win_left=-1, ori_win_right=-1), OK),
    (dict(ori_win_left=-2), INVALID),
    (dict(ori_win_right=-1), OK),
    (dict(layout_q=1, layout_kv=0), INVALID),   # layout pairs
    (dict(layout_q=0, layout_kv=1), INVALID),
    (dict(layout_q=1, layout_kv=1, ori_s=100, cmp_s=25, t1=32), OK),
    (dict(ori_block_size=0), INVALID),          # block size 1..1024
    (dict(ori_block_size=1025), INVALID),
    (dict(cmp_block_size=2048), INVALID),
    (dict(ori_block_size=1024), OK),
    (dict(q_s=2, t1=32), INVALID),              # BSND: t1 = B * Q_S
    (dict(kv_scale_mode=2), INVALID),
    (dict(topk_value_mode=1), UNSUPPORTED),
    (dict(softmax_scale=float("inf")), INVALID),
    (dict(q_dtype=1, kv_dtype=1), OK),          # bf16 q and KV (SparseCompressedFlashAttention)
    (dict(q_dtype=1, kv_dtype=2), OK),          # bf16 q, packed 640-byte rows (KvQuantSparseAttnSharedkv)
    (dict(q_dtype=0, kv_dtype=1), INVALID),     # bf16 / packed rows pair with bf16 q
    (dict(q_dtype=0, kv_dtype=2), INVALID),
    (dict(q_dtype=1, kv_dtype=0), UNSUPPORTED), # bf16 q with fp8 rows and fp32 descales: not built
    (dict(q_dtype=2), INVALID),
    (dict(q_dtype=1, kv_dtype=3), INVALID),
    (dict(q_dtype=1, kv_dtype=2, kv_scale_mode=1), INVALID),   # scales live in the packed row
    (dict(q_dtype=1, kv_dtype=1, topk=2048), UNSUPPORTED),     # the bf16-q kernel keeps <= 1024 slots
    (dict(ori_topk=200), OK),                   # listed ori keys (QuantSparseFlashMla: ori_sparse_indices)
    (dict(ori_topk=513), UNSUPPORTED),          # ori_topk + topk <= 1024 (one index list per row)
    (dict(ori_topk=-1), INVALID),
    (dict(ori_topk=100, q_dtype=1, kv_dtype=2), OK),
])
def test_validation_matrix(kw, status):
    assert m.csmla_validate(base_problem(**kw)) == status, m.csmla_last_error()


def test_plan_head_split_for_small_decode_batches(monkeypatch):
    """A 32-token per-token-descale decode batch is planned as 8-head groups
    over whole key lists: 256 units, one split, no workspace; 33 tokens:
    16-head groups over whole key lists."""
    for k in ("CSMLA_KERNEL", "CSMLA_DK_PARTS", "CSMLA_DK_TEST"):
        monkeypatch.delenv(k, raising=False)
    _, md, ws = m.csmla_plan(base_problem())
    assert md[12] == 8 and md[14] == 1 and md[5] == 1 and md[6] == 32 * 8 and md[7] == 256 and ws == 0
    _, md, ws = m.csmla_plan(base_problem(batch=33, t1=33))
    assert md[12] == 16 and md[14] == 1 and md[6] == 33 * 4 and ws == 0
    _, md, _ = m.csmla_plan(base_problem(batch=48, t1=48))
    assert md[12] == 16 and md[6] == 48 * 4               # 8-head groups would need two rounds
    _, md, _ = m.csmla_plan(base_problem(batch=128, t1=128))
    assert md[12] == 16 and md[6] == 128 * 4
    _, md, _ = m.csmla_plan(base_problem(batch=160, t1=160))
    assert md[12] == 64 and md[6] == 160                  # whole tokens from 129 tokens
    _, md, _ = m.csmla_plan(base_problem(batch=160, t1=160, kv_scale_mode=1))
    assert md[12] == 0                                    # per-tile below 257 tokens: key split
    _, md, _ = m.csmla_plan(base_problem(batch=512, t1=512))
    assert md[12] == 64 and md[5] == 1 and md[6] == 512   # prefill-sized batches: whole tokens
    _, md, _ = m.csmla_plan(base_problem(batch=512, t1=512, kv_scale_mode=1))
    assert md[12] == 64 and md[6] == 512                  # also with per-tile descales
    _, md, _ = m.csmla_plan(base_problem(kv_scale_mode=1))
    assert md[12] == 0                                    # small per-tile batches: key split
    monkeypatch.setenv("CSMLA_KERNEL", "prefill")
    _, md, _ = m.csmla_plan(base_problem())
    assert md[12] == 64 and md[6] == 32 and md[7] == 32
    monkeypatch.setenv("CSMLA_KERNEL", "split")
    _, md, _ = m.csmla_plan(base_problem(batch=512, t1=512))
    assert md[12] == 0
    monkeypatch.setenv("CSMLA_KERNEL", "heads16")
    _, md, _ = m.csmla_plan(base_problem())
    assert md[12] == 16 and md[6] == 32 * 4 and md[14] == 1


def test_plan_key_parts(monkeypatch):
    """Up to 11 decode tokens: 8-head groups, each split into two key parts on
    one XCD (the grid a whole number of XCD rounds of groups, one unit per
    work-group, the fixed workspace of sync words and exchange slots); 12 to
    28 tokens: 16-head groups in two parts; CSMLA_DK_PARTS overrides the
    count within what fits 256 work-groups and the key list's tiles."""
    for k in ("CSMLA_KERNEL", "CSMLA_DK_PARTS", "CSMLA_DK_TEST"):
        monkeypatch.delenv(k, raising=False)
    for b, grid in ((11, 176), (8, 128), (4, 64), (3, 48), (1, 16)):
        _, md, ws = m.csmla_plan(base_problem(batch=b, t1=b))
        assert md[12] == 8 and md[14] == 2 and md[6] == b * 16 and md[7] == grid and ws == WS_FIXED, (b, md[:16])
        assert md[5] == 1 and md[15] == 0
    for b, grid in ((12, 96), (16, 128), (24, 192), (25, 208), (28, 224)):
        _, md, ws = m.csmla_plan(base_problem(batch=b, t1=b))
        assert md[12] == 16 and md[14] == 2 and md[6] == b * 8 and md[7] == grid and ws == WS_FIXED, (b, md[:16])
    for b in (29, 32):
        _, md, ws = m.csmla_plan(base_problem(batch=b, t1=b))
        assert md[12] == 8 and md[14] == 1 and md[6] == b * 8 and ws == 0, (b, md[:16])
    monkeypatch.setenv("CSMLA_DK_PARTS", "8")
    _, md, _ = m.csmla_plan(base_problem(batch=4, t1=4))
    assert md[14] == 4 and md[6] == 4 * 8 * 4 and md[7] == 128     # 640 keys = 5 tiles: at most 4 parts
    _, md, _ = m.csmla_plan(base_problem(batch=4, t1=4, topk=128))
    assert md[14] == 2                                             # 256 keys: 2 tiles
    monkeypatch.setenv("CSMLA_DK_PARTS", "1")
    _, md, ws = m.csmla_plan(base_problem(batch=4, t1=4))
    assert md[14] == 1 and md[6] == 32 and ws == 0
    monkeypatch.setenv("CSMLA_DK_PARTS", "2")
    monkeypatch.setenv("CSMLA_KERNEL", "heads16")
    _, md, _ = m.csmla_plan(base_problem())
    assert md[12] == 16 and md[14] == 2 and md[6] == 256 and md[7] == 256
    monkeypatch.setenv("CSMLA_DK_TEST", "1")
    _, md, _ = m.csmla_plan(base_problem())
    assert md[15] == 1


def test_forward_rejects_inconsistent_key_parts(monkeypatch):
    for k in ("CSMLA_KERNEL", "CSMLA_DK_PARTS", "CSMLA_DK_TEST"):
        monkeypatch.delenv(k, raising=False)
    p = base_problem(batch=4, t1=4)
    _, md, ws = m.csmla_plan(p)
    assert md[14] == 2
    for word, val in ((14, 3), (14, 4), (14, 1), (7, 48), (15, 3), (12, 64)):
        bad = md.copy(); bad[word] = val
        assert m.csmla_forward(p, fake_tensors(ws), bad, raise_on_error=False) == MISMATCH, (word, val)
    assert m.csmla_forward(p, fake_tensors(ws - 256), md, raise_on_error=False) == WORKSPACE


def test_binding_metadata_pointer_follows_the_array(monkeypatch):
    """The binding reuses the ctypes pointer of a metadata array passed again:
    in-place edits of that array must still reach the C side, and a converted
    copy (another dtype) must never be the one kept."""
    from sparse_compressed_mla_amd import binding as bd
    for k in ("CSMLA_KERNEL", "CSMLA_DK_PARTS", "CSMLA_DK_TEST"):
        monkeypatch.delenv(k, raising=False)
    p = base_problem(batch=4, t1=4)
    _, md, ws = m.csmla_plan(p)
    t = fake_tensors(ws)
    ok = m.csmla_forward(p, t, md, raise_on_error=False)
    assert ok not in (MISMATCH, INVALID, WORKSPACE)      # past every host check (no GPU here)
    assert bd._md_pointer(md) is bd._md_pointer(md)
    assert ctypes.addressof(bd._md_pointer(md).contents) == md.ctypes.data
    md[14] = 3                                           # same object, edited in place
    assert m.csmla_forward(p, t, md, raise_on_error=False) == MISMATCH
    md[14] = 2
    assert m.csmla_forward(p, t, md, raise_on_error=False) == ok
    wide = md.astype(np.int64)
    assert m.csmla_forward(p, t, wide, raise_on_error=False) == ok
    assert bd._md_last[0][0] is md
    wide[14] = 3
    assert m.csmla_forward(p, t, wide, raise_on_error=False) == MISMATCH


def test_forward_rejects_bad_head_group(monkeypatch):
    monkeypatch.delenv("CSMLA_KERNEL", raising=False)
    p = base_problem()
    _, md, ws = m.csmla_plan(p)
    bad = md.copy(); bad[12] = 4
    assert m.csmla_forward(p, fake_tensors(ws), bad, raise_on_error=False) == MISMATCH
    bad = md.copy(); bad[12] = 16          # units no longer match the head group
    assert m.csmla_forward(p, fake_tensors(ws), bad, raise_on_error=False) == MISMATCH


def test_plan_invariants_and_determinism(monkeypatch):
    monkeypatch.setenv("CSMLA_KERNEL", "split")
    p = base_problem()
    _, md, ws = m.csmla_plan(p)
    assert md[0] == 0x4C4D5343 and md[1] == 2
    S, U, G = md[5], md[6], md[7]
    assert U == 32 * S and 1 <= G <= 256 and G <= U
    starts = md[16:16 + G + 1]
    assert starts[0] == 0 and starts[-1] == U and np.all(np.diff(starts) >= 1)
    a256 = lambda x: (x + 255) // 256 * 256
    # workspace: 4 KiB of sync words, 256 exchange slots of 33 KiB, per-unit XCD ids, the
    # partial outputs (bf16), their (max, sum)
    o = a256(WS_FIXED + 4 * U)
    assert ws == (0 if S == 1 else a256(o + U * 64 * 512 * 2) + U * 64 * 8)
    _, md2, ws2 = m.csmla_plan(p)
    assert np.array_equal(md, md2) and ws == ws2
    # a decode batch of 32 tokens is split so that the grid fills the chip
    assert S > 1 and G == 256


def test_plan_balances_prefill_ramp():
    """Prefill rows have fewer visible keys early on; the contiguous unit
    ranges are cut by estimated keys, not by count."""
    B, S1 = 4, 4096
    p = base_problem(batch=B, layout_q=1, q_s=0, t1=B * S1, ori_table_cols=32, cmp_table_cols=8,
                     kv_scale_mode=1, return_softmax_lse=1)
    cu = np.arange(0, B * S1 + 1, S1, dtype=np.int32)
    su = np.full(B, S1, dtype=np.int32)
    sc = np.full(B, S1 // 4, dtype=np.int32)
    res = np.zeros(B, dtype=np.int32)
    hl = CsmlaHostLengths()
    hl.cu_seqlens_q, hl.seqused_ori_kv, hl.seqused_cmp_kv, hl.cmp_residual_kv = (
        cu.ctypes.data, su.ctypes.data, sc.ctypes.data, res.ctypes.data)
    _, md, ws = m.csmla_plan(p, hl)
    assert md[5] == 1 and ws == 0
    G = md[7]
    starts = md[16:16 + G + 1]
    sizes = np.diff(starts)
    # the first range (cheap early tokens) holds more tokens than a late one
    assert sizes[0] > sizes[G // 8 - 1]
    assert md[3] != 0  # lengths hash recorded


def test_plan_rejects_bad_lengths_and_buffers():
    p = base_problem(layout_q=1, q_s=0)
    cu = np.array([0] + [1] * 31 + [31], dtype=np.int32)  # last element != t1
    hl = CsmlaHostLengths()
    hl.cu_seqlens_q = cu.ctypes.data
    st, _, _ = m.csmla_plan(p, hl, raise_on_error=False)
    assert st == INVALID
    cu2 = np.arange(33, dtype=np.int32)
    cu2[5] = 2  # decreasing
    hl.cu_seqlens_q = cu2.ctypes.data
    assert m.csmla_plan(p, hl, raise_on_error=False)[0] == INVALID
    lib = m.load()
    md = np.zeros(10, dtype=np.int32)
    ws = ctypes.c_size_t()
    assert lib.csmla_plan(ctypes.byref(base_problem()), None, md.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                          10, ctypes.byref(ws)) == INVALID
    assert lib.csmla_plan(ctypes.byref(base_problem()), None, None, 1024, ctypes.byref(ws)) == INVALID


def test_split_override_from_environment(monkeypatch):
    monkeypatch.setenv("CSMLA_KERNEL", "split")
    monkeypatch.setenv("CSMLA_SPLITS", "3")
    _, md, ws = m.csmla_plan(base_problem())
    assert md[5] == 3 and md[6] == 96 and ws > 0


def fake_tensors(ws_bytes=0):
    t = CsmlaTensors()
    for i, (name, _) in enumerate(CsmlaTensors._fields_[:-1]):
        setattr(t, name, 0x10000 * (i + 1))       # never dereferenced: every call below fails validation
    t.workspace_bytes = ws_bytes
    return t


def test_forward_rejects_before_launch(monkeypatch):
    monkeypatch.setenv("CSMLA_KERNEL", "split")   # a plan with a workspace
    p = base_problem()
    _, md, ws = m.csmla_plan(p)
    t = fake_tensors(ws)
    # metadata for another problem
    _, md_other, _ = m.csmla_plan(base_problem(topk=256))
    assert m.csmla_forward(p, t, md_other, raise_on_error=False) == MISMATCH
    # corrupted header / ranges
    bad = md.copy(); bad[0] = 0
    assert m.csmla_forward(p, t, bad, raise_on_error=False) == MISMATCH
    bad = md.copy(); bad[16 + 3] = bad[16 + 2] - 1
    assert m.csmla_forward(p, t, bad, raise_on_error=False) == MISMATCH
    # workspace
    t2 = fake_tensors(ws - 1)
    assert m.csmla_forward(p, t2, md, raise_on_error=False) == WORKSPACE
    t3 = fake_tensors(ws); t3.workspace = None
    assert m.csmla_forward(p, t3, md, raise_on_error=False) == WORKSPACE
    t4 = fake_tensors(ws); t4.workspace = 0x10008
    assert m.csmla_forward(p, t4, md, raise_on_error=False) == WORKSPACE   # alignment
    # required pointers (QuantSparseFlashMla 约束说明: PA needs seqused_ori_kv + block table)
    for name in ("q", "q_descale", "ori_kv", "ori_kv_descale", "cmp_kv", "cmp_sparse_indices",
                 "seqused_ori_kv", "ori_block_table", "cmp_block_table", "attn_out"):
        tt = fake_tensors(ws); setattr(tt, name, None)
        assert m.csmla_forward(p, tt, md, raise_on_error=False) == INVALID, name
    p_lse = base_problem(return_softmax_lse=1)
    _, md_lse, _ = m.csmla_plan(p_lse)
    tt = fake_tensors(ws); tt.softmax_lse = None
    assert m.csmla_forward(p_lse, tt, md_lse, raise_on_error=False) == INVALID
    # TND q needs cu_seqlens_q; TND kv needs cu_seqlens_ori_kv / cu_seqlens_cmp_kv
    pt = base_problem(layout_q=1, layout_kv=1, q_s=0, ori_s=1000, cmp_s=250)
    _, mdt, wst = m.csmla_plan(pt)
    for name in ("cu_seqlens_q", "cu_seqlens_ori_kv", "cu_seqlens_cmp_kv"):
        tt = fake_tensors(wst); setattr(tt, name, None)
        assert m.csmla_forward(pt, tt, mdt, raise_on_error=False) == INVALID, name
    # a NULL metadata pointer
    lib = m.load()
    assert lib.csmla_forward(ctypes.byref(p), ctypes.byref(t), None, None) == INVALID
    assert "metadata" in m.csmla_last_error()


def test_problem_struct_layout_matches_header():
    """Field order of the ctypes mirror equals the C struct's."""
    src = open(os.path.join(ROOT, "include", "csmla.h")).read()
    body = src[src.index("typedef struct {", src.index("Shapes and attributes")):src.index("} csmla_problem;")]
    names = re.findall(r"^\s*(?:int32_t|float)\s+([\w,\s]+);", body, flags=re.M)
    flat = [n.strip() for grp in names for n in grp.split(",")]
    assert flat == [f[0] for f in CsmlaProblem._fields_]
    body_t = src[src.index("typedef struct {", src.index("Device pointers")):src.index("} csmla_tensors;")]
    tnames = re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+);", body_t, flags=re.M)
    assert tnames == [f[0] for f in CsmlaTensors._fields_]


def test_noalloc_rejects_plans_beyond_the_static_scratch(monkeypatch):
    """csmla_forward_noalloc holds 64 MiB of static scratch per GPU; a plan
    whose split partials need more is refused on the host, before any HIP
    call (no GPU is needed to see the refusal)."""
    monkeypatch.setenv("CSMLA_KERNEL", "split")
    monkeypatch.setenv("CSMLA_SPLITS", "64")
    p = base_problem()
    _, md, ws = m.csmla_plan(p)
    assert ws > 64 << 20
    st = m.csmla_forward_noalloc(p, fake_tensors(0), md, raise_on_error=False)
    assert st == 3, (st, m.csmla_last_error())          # CSMLA_ERR_WORKSPACE
    assert "64" in m.csmla_last_error() or "67108864" in m.csmla_last_error()


def test_plan_split_key_decode(monkeypatch):
    """The split-key decode plan: token t's S splits on block ids equal mod 8
    (grid 8 S ceil(T1 / 8) <= 256, one resident round), at most 128 keys per
    unit, a workspace with the sync words, and forced S clamped to what fits."""
    monkeypatch.setenv("CSMLA_KERNEL", "splitkey")
    p = base_problem()                                  # 32 tokens, <= 128 band + 512 cmp keys
    _, md, ws = m.csmla_plan(p)
    S, U, G = md[5], md[6], md[7]
    assert md[13] == 1 and md[12] == 0
    assert S == 8 and U == 32 * 8 and G == 256 and ws > 4096
    monkeypatch.setenv("CSMLA_SPLITS", "2")             # 640 keys need >= 5 splits of 128
    _, md, _ = m.csmla_plan(p)
    assert md[5] == 5 and md[7] == 8 * 5 * 4
    monkeypatch.delenv("CSMLA_SPLITS")
    _, md, _ = m.csmla_plan(base_problem(batch=20, t1=20))
    assert md[13] == 1 and md[7] == 8 * md[5] * 3 and md[7] <= 256 and md[6] == 20 * md[5]
    _, md, _ = m.csmla_plan(base_problem(batch=64, t1=64))   # 5 splits x 8 rounds > 256: not taken
    assert md[13] == 0
    bad = m.csmla_plan(p)[1].copy()
    bad[7] = 128                                        # grid no longer 8 S ceil(T1 / 8)
    assert m.csmla_forward(p, fake_tensors(ws), bad, raise_on_error=False) == MISMATCH


def test_plan_bf16_q_kernels(monkeypatch):
    """bf16 q with bf16 or packed rows: key splits (the bf16-q kernel and the
    combine) whatever kernel override is set, at most 1024 keys per unit."""
    for env in (None, "heads8", "prefill", "splitkey"):
        if env is None:
            monkeypatch.delenv("CSMLA_KERNEL", raising=False)
        else:
            monkeypatch.setenv("CSMLA_KERNEL", env)
        for kv in (1, 2):
            _, md, ws = m.csmla_plan(base_problem(q_dtype=1, kv_dtype=kv))
            assert md[12] == 0 and md[13] == 0 and md[5] >= 1
            _, md, _ = m.csmla_plan(base_problem(q_dtype=1, kv_dtype=kv, batch=1, t1=1, ori_mask_mode=0,
                                                 ori_win_left=-1, ori_win_right=-1, topk=0,
                                                 ori_table_cols=40, cmp_table_cols=10))
            assert md[5] >= 3                       # up to 5120 + 1280 keys: >= 7 units of <= 1024 ... per token


def test_plan_listed_ori_keys_take_the_key_split(monkeypatch):
    """Listed ori keys run on the key-split kernels whatever the override."""
    for env in (None, "heads8", "prefill", "splitkey"):
        if env is None:
            monkeypatch.delenv("CSMLA_KERNEL", raising=False)
        else:
            monkeypatch.setenv("CSMLA_KERNEL", env)
        _, md, _ = m.csmla_plan(base_problem(ori_topk=64))
        assert md[12] == 0 and md[13] == 0
    monkeypatch.delenv("CSMLA_KERNEL", raising=False)
    p = base_problem(ori_topk=64)
    _, md, ws = m.csmla_plan(p)
    bad = md.copy(); bad[12] = 8; bad[6] = 32 * 8; bad[5] = 1   # a head-split header for this problem
    assert m.csmla_forward(p, fake_tensors(ws), bad, raise_on_error=False) == MISMATCH


def test_plan_check_sees_other_lengths():
    """csmla_plan_check: the plan's own problem and lengths pass; other host
    lengths, another problem, or a foreign buffer do not (csmla_forward cannot
    see lengths, so this is the check for a reused plan)."""
    p = base_problem()
    su = np.full(32, 8192, dtype=np.int32)
    hl = m.CsmlaHostLengths()
    hl.seqused_ori_kv = su.ctypes.data
    _, md, _ = m.csmla_plan(p, hl)
    assert m.csmla_plan_check(p, hl, md) == OK
    su2 = su.copy(); su2[3] = 4000
    hl2 = m.CsmlaHostLengths()
    hl2.seqused_ori_kv = su2.ctypes.data
    assert m.csmla_plan_check(p, hl2, md) == MISMATCH
    assert m.csmla_plan_check(p, None, md) == MISMATCH
    assert m.csmla_plan_check(base_problem(topk=256), hl, md) == MISMATCH
    assert m.csmla_plan_check(p, hl, np.zeros(1024, dtype=np.int32)) == MISMATCH
