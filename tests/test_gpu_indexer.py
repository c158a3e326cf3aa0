"""GPU parity of the lightning-indexer top-k (csmla_indexer_forward through the
C ABI) against the CPU oracle (oracle/indexer.py).

Bar:
* rows that see at most topk keys, padding rows and rows with no visible key:
  the index row is bit-exact (0..vis-1 then -1, or all -1);
* the float32 scores the kernel leaves in the workspace are within the
  tolerance of the oracle's, key by key;
* other rows: the index row equals, bit for bit, the selection the page's rule
  (topk largest, ties to the lower position, ascending) makes on the kernel's
  own scores; and against the oracle's scores no left-out key beats a chosen
  one by more than the two keys' tolerances, so where the oracle's ranking is
  decided by more than the tolerance the chosen set is exactly the oracle's.
Tolerance: the kernel accumulates the 128 fp8 products of a head and the 64
heads in float32 in another order than the oracle (whose dot products are
exact), so a score may differ by about (128 + 64) float32 roundings of the
absolute-value sum; the bound used is 2e-5 * A[s], with
A[s] = sum_h |W_h| scale_q_h scale_k_s sum_d |q_hd k_sd|.
"""
import numpy as np
import pytest
import torch

import sparse_compressed_mla_amd as m
from oracle.fp8 import decode_e4m3
from oracle.indexer import key_rows, oracle_scores, token_context, topk_positions
from workloads.indexer_gen import IndexerInputs, make_indexer, make_indexer_workload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REL_TOL = 2e-5


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


def abs_bound(inp, t, vis):
    """A[s] of the docstring for row t's visible keys (float64)."""
    b = token_context(inp, t)[0]
    kc, ks = key_rows(inp, b, vis)
    q = np.abs(decode_e4m3(inp.q[t].numpy()))
    k = np.abs(decode_e4m3(kc))
    wq = np.abs(inp.weights[t].numpy().astype(np.float64)) * inp.q_scale[t].numpy().astype(np.float64)
    return (wq @ (q @ k.T)) * ks.astype(np.float64)


def run(inp_cpu, plan_lengths=True):
    g = inp_cpu.to(DEV)
    plan = m.IndexerPlan(g if plan_lengths else g, lengths=plan_lengths)
    out, ws = m.indexer_forward(g, plan=plan)
    torch.cuda.synchronize()
    idx = out.cpu().numpy().reshape(inp_cpu.t1, inp_cpu.topk)
    scores = ws.view(torch.float32)[: inp_cpu.t1 * plan.stride].view(inp_cpu.t1, plan.stride).cpu().numpy()
    return idx, scores, plan


def check(inp, rows=None, name="", plan_lengths=True):
    say(f"case {name}: t1={inp.t1} g={inp.g} topk={inp.topk} layout_q={inp.layout_q} layout_k={inp.layout_k}")
    idx, scores, plan = run(inp, plan_lengths)
    rows = range(inp.t1) if rows is None else rows
    n_sel = n_amb = 0
    worst = 0.0
    for t in rows:
        vis = token_context(inp, t)[4]
        row = idx[t]
        if vis <= 0:
            assert (row == -1).all(), (name, t, vis, row[:8])
            continue
        if vis <= inp.topk:
            want = np.full(inp.topk, -1, np.int32)
            want[:vis] = np.arange(vis)
            assert np.array_equal(row, want), (name, t, vis, row[:8])
        sc = oracle_scores(inp, t).astype(np.float64)
        tol = REL_TOL * abs_bound(inp, t, vis)
        err = np.abs(scores[t, :vis].astype(np.float64) - sc)
        worst = max(worst, float((err / np.maximum(tol, 1e-300)).max()))
        assert (err <= tol).all(), (name, t, "score", np.argmax(err - tol), err.max())
        if vis <= inp.topk:
            continue
        n_sel += 1
        assert (row >= 0).all() and (row < vis).all(), (name, t, row.min(), row.max(), vis)
        assert (np.diff(row) > 0).all(), (name, t, "not strictly ascending")
        # the top-k step, bit for bit: the selection the page's rule makes on the
        # kernel's own float32 scores (ties to the lower position)
        assert np.array_equal(row, topk_positions(scores[t, :vis], inp.topk)), (name, t, "top-k of own scores")
        # end to end: no left-out key beats a chosen one by more than both tolerances
        chosen = np.zeros(vis, bool)
        chosen[row] = True
        lo_chosen = (sc - tol)[chosen].min()
        hi_left = (sc + tol)[~chosen].max()
        assert (sc + tol)[chosen].min() >= (sc - tol)[~chosen].max(), (name, t, "a left-out key clearly wins")
        n_amb += int(hi_left > lo_chosen)
    say(f"case {name}: ok; {n_sel} selected rows, {n_amb} with near-ties at the threshold, "
        f"worst score error {worst:.3f} of the bound")
    return idx, scores


def tie_exact(inp, name):
    """Rows whose scores repeat exactly: the chosen positions must be exactly
    the oracle's (ties to the lower position)."""
    from oracle.indexer import oracle_indexer
    idx, _ = check(inp, name=name)
    want = oracle_indexer(inp)
    assert np.array_equal(idx, want), name


# ------------------------------------------------------------------ small cases

def test_tiny_all_rows():
    check(make_indexer_workload("idx_tiny"), name="idx_tiny")


@pytest.mark.parametrize("layout_k,block_size", [("PA_BBND", 128), ("PA_BBND", 16), ("PA_BBND", 7),
                                                 ("TND", 0), ("BSND", 0)])
def test_decode_layouts(layout_k, block_size):
    inp = make_indexer(seed=21, q_lens=[1] * 5, k_lens=[2048, 1500, 700, 300, 513], layout_q="BSND",
                       layout_k=layout_k, block_size=max(block_size, 1), residual=[0, 1, 2, 3, 0], topk=512)
    check(inp, name=f"decode_{layout_k}_{block_size}")


def test_mtp_two_rows_long_keys():
    inp = make_indexer(seed=22, q_lens=[2] * 3, k_lens=[9000, 4097, 5000], layout_q="BSND",
                       residual=[3, 0, 1], topk=512)
    check(inp, name="mtp_9000")


def test_prefill_causal_rows():
    inp = make_indexer(seed=23, q_lens=[70, 37, 9], k_lens=[300, 150, 40], layout_q="TND",
                       residual=[1, 2, 0], topk=64, cmp_ratio=4)
    check(inp, name="prefill_causal")


def test_prefill_mask_mode_zero_and_partial_heads():
    inp = make_indexer(seed=24, q_lens=[20, 13], k_lens=[333, 97], layout_q="TND", g=17,
                       residual=[0, 0], topk=50, mask_mode=0, block_size=32)
    check(inp, name="mask0_g17")


@pytest.mark.parametrize("g", [1, 8, 63, 64])
def test_head_counts(g):
    inp = make_indexer(seed=25 + g, q_lens=[3, 5], k_lens=[600, 260], layout_q="TND", g=g,
                       residual=[2, 0], topk=100)
    check(inp, name=f"g{g}")


def test_padding_rows_tnd_and_bsnd():
    inp = make_indexer(seed=30, q_lens=[6, 4, 5], k_lens=[100, 200, 90], layout_q="TND", topk=40,
                       residual=[0, 1, 3], seqused_q=[3, 0, 5])
    check(inp, name="pad_tnd")
    inp = make_indexer(seed=31, q_lens=[4] * 3, k_lens=[100, 200, 90], layout_q="BSND", topk=40,
                       residual=[0, 1, 3], seqused_q=[4, 1, 2])
    check(inp, name="pad_bsnd")


def test_rows_with_no_key_and_topk_extremes():
    # early prefill rows see no compressed key; topk 1 and 8192
    inp = make_indexer(seed=32, q_lens=[12], k_lens=[5], layout_q="TND", topk=1, residual=[0], cmp_ratio=4,
                       block_size=4)
    check(inp, name="topk1")
    inp = make_indexer(seed=33, q_lens=[2, 3], k_lens=[3000, 9000], layout_q="TND", topk=8192, residual=[0, 0])
    check(inp, name="topk8192")


def test_empty_batches_and_zero_keys():
    inp = make_indexer(seed=34, q_lens=[3, 0, 4, 0], k_lens=[80, 50, 0, 60], layout_q="TND", topk=16,
                       residual=[0, 0, 0, 0])
    check(inp, name="empty_batches")


def test_plan_without_host_lengths():
    inp = make_indexer(seed=35, q_lens=[5, 7], k_lens=[400, 123], layout_q="TND", topk=64, residual=[1, 2])
    check(inp, name="no_host_lengths", plan_lengths=False)


def test_rows_past_the_register_cache():
    # 40000 keys: the top-k streams chunks past the 32768 it keeps in registers
    inp = make_indexer(seed=36, q_lens=[1, 1], k_lens=[40000, 33000], layout_q="BSND", topk=512,
                       residual=[0, 0], g=16)
    check(inp, name="streamed_chunks")


def test_exact_ties_prefer_lower_positions():
    # every key row identical: all scores equal, the first topk positions win
    inp = make_indexer(seed=37, q_lens=[2, 1], k_lens=[700, 3000], layout_q="TND", topk=100, residual=[0, 0],
                       g=16, block_size=64)
    inp.key[:] = inp.key[inp.block_table[0, 0], 0]
    inp.key_scale[:] = 0.01
    tie_exact(inp, "all_equal")
    # scores repeating with period 5 (ties at the threshold between distinct positions)
    inp = make_indexer(seed=38, q_lens=[3], k_lens=[997], layout_q="TND", layout_k="TND", topk=301,
                       residual=[0], g=32)
    for s in range(5, 997):
        inp.key[s] = inp.key[s % 5]
        inp.key_scale[s] = inp.key_scale[s % 5]
    tie_exact(inp, "period5")


def test_repeat_calls_are_identical():
    inp = make_indexer(seed=39, q_lens=[1] * 8, k_lens=[3000] * 8, layout_q="BSND", topk=512, residual=[0] * 8)
    a, _, _ = run(inp)
    b, _, _ = run(inp)
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ full-size workloads

def _sample(inp, n, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(inp.t1, size=min(n, inp.t1), replace=False).tolist())
    rows |= {0, inp.t1 - 1}
    return sorted(rows)


def test_full_decode_all_rows():
    check(make_indexer_workload("idx_csa_decode"), name="idx_csa_decode")


def test_full_mtp_sampled_rows():
    inp = make_indexer_workload("idx_csa_mtp_long")
    check(inp, rows=_sample(inp, 12, 1), name="idx_csa_mtp_long")


def test_full_prefill_sampled_rows():
    inp = make_indexer_workload("idx_csa_prefill")
    rows = _sample(inp, 40, 2) + [2047, 2048, 2049, 4095, 4096]   # around the topk = visible boundary
    check(inp, rows=sorted(set(rows)), name="idx_csa_prefill")


@pytest.mark.parametrize("tile", ["1,1", "2,1", "2,4", "4,1", "4,4"])
def test_every_tile_shape(tile, monkeypatch):
    # the planner's tile choice forced: rows per wave x waves across rows
    monkeypatch.setenv("CSMLA_IDX_TILE", tile)
    inp = make_indexer(seed=40, q_lens=[37, 11, 2], k_lens=[700, 150, 1300], layout_q="TND",
                       residual=[1, 2, 0], topk=64, cmp_ratio=4, block_size=64)
    check(inp, name=f"tile_{tile}")


@pytest.mark.parametrize("bs", [1, 3, 48])
def test_small_and_odd_block_sizes(bs):
    # a wave's keys span at most 64 blocks: tiny blocks shrink the key chunk
    inp = make_indexer(seed=41, q_lens=[20, 1], k_lens=[600, 333], layout_q="TND", residual=[0, 3], topk=50,
                       block_size=bs, g=16)
    check(inp, name=f"block_size_{bs}")


def test_key_chunk_override(monkeypatch):
    monkeypatch.setenv("CSMLA_IDX_KC", "1024")
    inp = make_indexer(seed=42, q_lens=[1] * 4, k_lens=[5000, 3000, 64, 1], layout_q="BSND", residual=[0] * 4,
                       topk=512)
    check(inp, name="kc1024")


@pytest.mark.parametrize("shape", ["256,1", "256,4", "1024,2", "1024,4", "1024,8"])
def test_every_topk_shape(shape, monkeypatch):
    # rows of 700 to 40000 keys: most shapes also re-read chunks past the registers
    monkeypatch.setenv("CSMLA_IDX_TOPK", shape)
    inp = make_indexer(seed=43, q_lens=[1] * 5, k_lens=[700, 1100, 2100, 9000, 40000], layout_q="BSND",
                       residual=[0] * 5, topk=512, g=8)
    check(inp, name=f"topk_{shape}")
