"""Host-side tests of the indexer's C ABI (include/csmla_indexer.h), no GPU:
the validation matrix of the QuantLightningIndexerV2 page's constraints, the
work split's invariants, and the errors csmla_indexer_forward reports before
any launch."""
import ctypes

import numpy as np
import pytest

import sparse_compressed_mla_amd as m
from sparse_compressed_mla_amd.binding import (CsmlaIndexerHostLengths, CsmlaIndexerProblem,
                                               CsmlaIndexerTensors)

OK, INVALID, UNSUPPORTED, WORKSPACE, MISMATCH = 0, 1, 2, 3, 4


def problem(**kw):
    p = CsmlaIndexerProblem()
    vals = dict(batch=32, g=64, n2=1, d=128, layout_q=0, layout_k=2, q_s=1, t1=32, k_s=0, block_size=128,
                num_blocks=520, table_cols=16, topk=512, mask_mode=3, cmp_ratio=4, quant_mode=1)
    vals.update(kw)
    for k, v in vals.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,status", [
    (dict(), OK),
    (dict(g=0), INVALID), (dict(g=65), INVALID), (dict(g=1), OK),        # query N in [1, 64]
    (dict(n2=2), INVALID),                                               # key N only 1
    (dict(topk=0), INVALID), (dict(topk=8193), INVALID), (dict(topk=8192), OK),
    (dict(quant_mode=2), UNSUPPORTED), (dict(quant_mode=3), UNSUPPORTED), (dict(quant_mode=5), UNSUPPORTED),
    (dict(d=64), UNSUPPORTED), (dict(d=256), UNSUPPORTED),
    (dict(batch=0, t1=0), INVALID),
    (dict(layout_q=2), INVALID),                                         # query: BSND or TND
    (dict(layout_k=3), INVALID),
    (dict(q_s=2), INVALID),                                              # BSND: t1 = B * S1
    (dict(layout_q=1, q_s=0, t1=100), OK),
    (dict(block_size=0), INVALID), (dict(block_size=1025), INVALID), (dict(block_size=7), OK),
    (dict(table_cols=0), INVALID),
    (dict(layout_k=1, k_s=0), INVALID), (dict(layout_k=1, k_s=5000), OK), (dict(layout_k=0, k_s=300), OK),
    (dict(cmp_ratio=0), INVALID), (dict(cmp_ratio=129), INVALID), (dict(cmp_ratio=1), OK),
    (dict(mask_mode=1), INVALID), (dict(mask_mode=4), INVALID), (dict(mask_mode=0), OK),
])
def test_validation_matrix(kw, status):
    assert m.csmla_indexer_validate(problem(**kw)) == status, m.csmla_last_error()


def lengths(**arrays):
    hl = CsmlaIndexerHostLengths()
    keep = []
    for k, v in arrays.items():
        a = np.ascontiguousarray(np.asarray(v, dtype=np.int32))
        keep.append(a)
        setattr(hl, k, a.ctypes.data)
    return hl, keep


def test_plan_decode_prefill_and_mtp_shapes():
    # decode: one row per batch, the keys split over the 4 waves
    hl, _k = lengths(seqused_k=[2048] * 32, cmp_residual_k=[0] * 32)
    _, md, ws = m.csmla_indexer_plan(problem(), hl)
    assert md[0] == 0x58444943 and (md[4], md[5], md[6]) == (1, 1, 256)
    assert (md[7], md[8], md[9]) == (1, 8, 2048) and ws == 32 * 2048 * 4
    assert (md[10], md[11]) == (256, 4)
    # two rows per batch (MTP), long keys
    hl, _k = lengths(seqused_k=list(range(20000, 20064)))
    _, md, ws = m.csmla_indexer_plan(problem(batch=64, q_s=2, t1=128, table_cols=200), hl)
    assert (md[4], md[5], md[6]) == (2, 1, 4096) and md[9] == 20096 and md[8] == 5
    assert (md[10], md[11]) == (1024, 8)
    # prefill: 16 rows per work-group
    hl, _k = lengths(cu_seqlens_q=[0, 4096, 8192], seqused_k=[1024, 1024])
    _, md, ws = m.csmla_indexer_plan(problem(batch=2, layout_q=1, q_s=0, t1=8192, table_cols=8), hl)
    assert (md[4], md[5], md[6]) == (2, 4, 1024) and md[7] == 512 and md[8] == 1 and md[9] == 1024
    assert (md[10], md[11]) == (256, 1)
    # the same problem without host lengths plans from the shapes
    _, md2, ws2 = m.csmla_indexer_plan(problem(batch=2, layout_q=1, q_s=0, t1=8192, table_cols=8))
    assert md2[7] == 1024 and md2[9] == 1024 and md2[3] == 0 and md[3] != 0
    assert ws2 == 8192 * 1024 * 4


def test_plan_is_deterministic_and_hash_tracks_problem():
    _, a, _ = m.csmla_indexer_plan(problem())
    _, b, _ = m.csmla_indexer_plan(problem())
    _, c, _ = m.csmla_indexer_plan(problem(topk=256))
    assert np.array_equal(a, b) and a[2] != c[2]


@pytest.mark.parametrize("arrays,kw", [
    (dict(cu_seqlens_q=[0, 5, 3]), dict(batch=2, layout_q=1, q_s=0, t1=3)),       # decreasing
    (dict(cu_seqlens_q=[1, 2, 3]), dict(batch=2, layout_q=1, q_s=0, t1=3)),       # [0] != 0
    (dict(cu_seqlens_q=[0, 2, 4]), dict(batch=2, layout_q=1, q_s=0, t1=3)),       # [B] != t1
    (dict(cu_seqlens_q=[0, 1, 2]), dict(batch=2, t1=2)),                          # BSND query
    (dict(cu_seqlens_k=[0, 10, 20]), dict(batch=2, t1=2)),                        # not TND key
    (dict(cu_seqlens_k=[0, 10, 2000]), dict(batch=2, t1=2, layout_k=1, k_s=100)),  # past the key rows
    (dict(seqused_k=[3000, 1]), dict(batch=2, t1=2)),                             # past 16 x 128
    (dict(seqused_k=[-1, 1]), dict(batch=2, t1=2)),
    (dict(cmp_residual_k=[4, 0]), dict(batch=2, t1=2)),                           # >= cmp_ratio
    (dict(seqused_q=[-1, 0]), dict(batch=2, t1=2)),
])
def test_plan_rejects_bad_lengths(arrays, kw):
    hl, _k = lengths(**arrays)
    st, _, _ = m.csmla_indexer_plan(problem(**kw), hl, raise_on_error=False)
    assert st == INVALID, m.csmla_last_error()


def test_plan_needs_a_metadata_buffer():
    lib = m.load()
    m.csmla_indexer_metadata_words()
    md = np.zeros(8, dtype=np.int32)
    ws = ctypes.c_size_t()
    assert lib.csmla_indexer_plan(ctypes.byref(problem()), None, md.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                  8, ctypes.byref(ws)) == INVALID
    assert lib.csmla_indexer_plan(ctypes.byref(problem()), None, None, 32, ctypes.byref(ws)) == INVALID
    assert m.csmla_indexer_metadata_words() == 32


def fake_tensors(ws_bytes, **override):
    t = CsmlaIndexerTensors()
    for name in ("query", "key", "weights", "query_dequant_scale", "key_dequant_scale", "seqused_k",
                 "block_table", "sparse_indices"):
        setattr(t, name, 0x100000)          # never dereferenced: every call below fails before a launch
    t.workspace = 0x200000
    t.workspace_bytes = ws_bytes
    for k, v in override.items():
        setattr(t, k, v)
    return t


def test_forward_rejects_before_launch():
    p = problem()
    _, md, ws = m.csmla_indexer_plan(p)
    f = lambda t, meta=md, prob=p: m.csmla_indexer_forward(prob, t, meta, raise_on_error=False)
    _, other, _ = m.csmla_indexer_plan(problem(topk=100))
    assert f(fake_tensors(ws), other) == MISMATCH                 # planned for another problem
    bad = md.copy(); bad[0] = 0
    assert f(fake_tensors(ws), bad) == MISMATCH                   # not a plan
    bad = md.copy(); bad[4] = 3
    assert f(fake_tensors(ws), bad) == MISMATCH                   # no such tile
    bad = md.copy(); bad[9] = 100
    assert f(fake_tensors(ws), bad) == MISMATCH                   # stride not a multiple of 64
    bad = md.copy(); bad[10] = 512
    assert f(fake_tensors(ws), bad) == MISMATCH                   # no such top-k shape
    bad = md.copy(); bad[10], bad[11] = 256, 2
    assert f(fake_tensors(ws), bad) == MISMATCH
    assert f(fake_tensors(ws - 4)) == WORKSPACE
    assert f(fake_tensors(ws, workspace=0x200010)) == WORKSPACE   # misaligned
    assert f(fake_tensors(ws, query=None)) == INVALID
    assert f(fake_tensors(ws, sparse_indices=None)) == INVALID
    assert f(fake_tensors(ws, seqused_k=None)) == INVALID         # PA needs seqused_k
    assert f(fake_tensors(ws, block_table=None)) == INVALID
    assert f(fake_tensors(ws, cu_seqlens_q=0x100000)) == INVALID  # BSND query takes no cu_seqlens_q
    assert f(fake_tensors(ws, cu_seqlens_k=0x100000)) == INVALID  # PA key takes no cu_seqlens_k
    pt = problem(layout_q=1, q_s=0, layout_k=1, k_s=4096)
    _, mdt, wst = m.csmla_indexer_plan(pt)
    assert f(fake_tensors(wst), mdt, pt) == INVALID                # TND query needs cu_seqlens_q
    assert f(fake_tensors(wst, cu_seqlens_q=0x100000), mdt, pt) == INVALID   # TND key needs cu_seqlens_k
    lib = m.load()
    assert lib.csmla_indexer_forward(ctypes.byref(p), ctypes.byref(fake_tensors(ws)), None, None) == INVALID
    assert "metadata" in m.csmla_last_error()


def test_paged_tiny_blocks_shrink_the_key_chunk():
    """A wave reads its block-table entries with one load per lane: its keys
    may span at most 64 blocks, so tiny blocks shrink the chunk (and fall back
    to waves that split keys)."""
    for bs in (1, 2, 3, 7, 48, 128, 1024):
        hl, _k = lengths(cu_seqlens_q=[0, 40], seqused_k=[600])
        _, md, _ = m.csmla_indexer_plan(problem(batch=1, layout_q=1, q_s=0, t1=40, block_size=bs,
                                                table_cols=(600 + bs - 1) // bs), hl)
        part = md[6] // (4 // md[5])
        worst = max((k0 + part - 1) // bs - k0 // bs + 1 for k0 in range(0, 64 * bs, 64))
        assert worst <= 64 and part >= 64, (bs, md[4:7])


def test_tuning_overrides(monkeypatch):
    monkeypatch.setenv("CSMLA_IDX_TILE", "2,4")
    monkeypatch.setenv("CSMLA_IDX_KC", "512")
    monkeypatch.setenv("CSMLA_IDX_TOPK", "1024,2")
    _, md, _ = m.csmla_indexer_plan(problem())
    assert (md[4], md[5], md[6], md[10], md[11]) == (2, 4, 512, 1024, 2)
    monkeypatch.setenv("CSMLA_IDX_TILE", "3,3")      # not a built shape: ignored
    monkeypatch.setenv("CSMLA_IDX_TOPK", "128,1")
    _, md, _ = m.csmla_indexer_plan(problem())
    assert (md[4], md[5]) == (1, 1) and (md[10], md[11]) != (128, 1)
