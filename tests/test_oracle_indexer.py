"""Pins of the lightning-indexer oracle (oracle/indexer.py) against things
other than itself:

* a hand-worked example (tests/golden/indexer_worked.json): ReLU on each head,
  a negative weight, both dequant scales, ties, ordering, -1 padding and the
  causal visibility of compressed keys
* closed forms: scores that grow with the key position make the top-k the last
  visible keys, for many ratios, residuals and row counts
* library special cases: the selection equals a stable argsort; the scores
  equal a float64 matmul over torch's own e4m3 decoding
* invariants: layouts (paged with shuffled blocks, TND, BSND) agree; power-of-two
  rescaling of weights or scales leaves the indices unchanged
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle.indexer import index_scores, oracle_indexer, oracle_scores, token_context, topk_positions
from workloads.indexer_gen import IndexerInputs, make_indexer

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _worked():
    with open(os.path.join(GOLD, "indexer_worked.json")) as f:
        return json.load(f)


def _worked_inputs(w, s1, topk, mask_mode, ratio=1, residual=0, layout_k="TND"):
    d = w["d"]
    q1 = np.zeros((2, d), np.uint8)
    for h, j, c in w["query"]["nonzero"]:
        q1[h, j] = int(c, 16)
    n = len(w["keys"]["a"])
    k = np.zeros((n, d), np.uint8)
    k[:, 0] = [int(c, 16) for c in w["keys"]["a"]]
    k[:, 1] = [int(c, 16) for c in w["keys"]["b"]]
    q = np.repeat(q1[None], s1, axis=0)
    kw = dict(layout_q="TND", layout_k=layout_k, batch=1, q_s=0, q=torch.from_numpy(q),
              q_scale=torch.tensor([w["scale_q"]] * s1, dtype=torch.float32),
              weights=torch.tensor([w["weights"]] * s1, dtype=torch.float32),
              cu_seqlens_q=torch.tensor([0, s1], dtype=torch.int32),
              cmp_residual_k=torch.tensor([residual], dtype=torch.int32),
              topk=topk, mask_mode=mask_mode, cmp_ratio=ratio)
    ks = torch.tensor(w["scale_k"], dtype=torch.float32)
    if layout_k == "TND":
        kw.update(key=torch.from_numpy(k).view(n, 1, d), key_scale=ks,
                  cu_seqlens_k=torch.tensor([0, n], dtype=torch.int32))
    else:  # paged, one key per block, blocks stored in reverse order
        kw.update(key=torch.from_numpy(k[::-1].copy()).view(n, 1, 1, d), key_scale=ks.flip(0).view(n, 1),
                  block_table=torch.arange(n - 1, -1, -1, dtype=torch.int32).view(1, n),
                  seqused_k=torch.tensor([n], dtype=torch.int32))
    return IndexerInputs(**kw)


def test_worked_scores():
    w = _worked()
    inp = _worked_inputs(w, 1, 1, 0)
    assert oracle_scores(inp, 0).tolist() == w["scores"]["value"]


@pytest.mark.parametrize("layout_k", ["TND", "PA_BBND"])
def test_worked_cases(layout_k):
    w = _worked()
    for c in w["cases"]:
        s1 = c.get("s1", 1)
        inp = _worked_inputs(w, s1, c["topk"], c["mask_mode"], c.get("cmp_ratio", 1),
                             c.get("cmp_residual_k", 0), layout_k)
        assert oracle_indexer(inp).tolist() == c["rows"], c


def test_dropped_head_changes_result():
    """The worked example needs both heads: without head 1, key 1 outranks key 0."""
    w = _worked()
    inp = _worked_inputs(w, 1, 3, 0)
    inp.weights[:, 1] = 0.0
    assert oracle_indexer(inp).tolist() == [[1, 3, 4]]


def _ramp_inputs(k_lens, q_lens, ratio, residual, topk, mask_mode, layout_q="TND"):
    """Keys whose score is exactly their position + 1 (key_scale = s + 1, one
    head with q = k = 1 at d = 0, weight 1, query scale 1)."""
    inp = make_indexer(seed=3, q_lens=q_lens, k_lens=k_lens, layout_q=layout_q, layout_k="TND",
                       g=1, cmp_ratio=ratio, residual=residual, topk=topk, mask_mode=mask_mode)
    inp.q.zero_()
    inp.q[:, 0, 0] = 0x38
    inp.key.zero_()
    inp.key[:, 0, 0] = 0x38
    inp.q_scale.fill_(1.0)
    inp.weights.fill_(1.0)
    cu = inp.cu_seqlens_k.numpy()
    ks = np.zeros(int(cu[-1]), np.float32)
    for b in range(len(k_lens)):
        ks[cu[b]:cu[b + 1]] = np.arange(1, k_lens[b] + 1)
    inp.key_scale = torch.from_numpy(ks)
    return inp


@pytest.mark.parametrize("ratio,residual", [(1, 0), (4, 0), (4, 3), (2, 1), (128, 77)])
def test_causal_ramp_closed_form(ratio, residual):
    k_lens, q_lens, topk = [40, 9, 0], [13, 5, 3], 6
    inp = _ramp_inputs(k_lens, q_lens, ratio, [residual] * 3, topk, 3)
    got = oracle_indexer(inp)
    t = 0
    for b in range(3):
        L = k_lens[b] * ratio + residual
        for i in range(q_lens[b]):
            p = L - q_lens[b] + i
            vis = min(max((p + 1) // ratio, 0), k_lens[b])
            lo = max(vis - topk, 0)
            want = list(range(lo, vis)) + [-1] * (topk - (vis - lo))
            assert got[t].tolist() == want, (b, i, vis)
            t += 1


def test_mask_mode_zero_sees_every_key():
    inp = _ramp_inputs([30], [7], 4, [0], 5, 0)
    assert all(r == list(range(25, 30)) for r in oracle_indexer(inp).tolist())


def test_padding_rows_are_minus_one():
    inp = make_indexer(seed=4, q_lens=[5, 3], k_lens=[20, 30], layout_q="TND", topk=4, seqused_q=[2, 3],
                       residual=[1, 2], g=4)
    got = oracle_indexer(inp)
    assert (got[2:5] == -1).all()
    assert (got[:2] >= 0).all() and (got[5:] >= 0).all()


def test_topk_matches_stable_argsort():
    rng = np.random.default_rng(0)
    for n, k in [(1, 1), (7, 3), (50, 50), (50, 64), (300, 17)]:
        s = rng.integers(-4, 5, size=n).astype(np.float32)   # many exact ties
        order = np.argsort(-s, kind="stable")[:k]
        want = np.full(k, -1, np.int32)
        want[:len(order)] = np.sort(order)
        assert topk_positions(s, k).tolist() == want.tolist(), (n, k)


def test_scores_match_float64_matmul_with_torch_decode():
    inp = make_indexer(seed=5, q_lens=[3], k_lens=[70], layout_q="TND", layout_k="TND", g=8)
    q = inp.q.view(torch.float8_e4m3fn).double()          # torch's own e4m3 decoding
    k = inp.key.view(torch.float8_e4m3fn).double()[:, 0]
    for t in range(3):
        vis = token_context(inp, t)[4]
        dots = q[t] @ k[:vis].T                            # [g, vis]
        rel = (inp.q_scale[t].double()[:, None] * inp.key_scale[:vis].double()[None, :] * dots).clamp_min(0)
        want = (inp.weights[t].double()[:, None] * rel).sum(0).numpy()
        got = oracle_scores(inp, t)
        assert np.allclose(got, want, rtol=1e-5, atol=1e-5 * np.abs(want).max())


def _relayout(inp, layout_k, seed=11):
    """The keys of a TND input in another layout (paged blocks shuffled, TND, BSND)."""
    B = inp.batch
    cu = inp.cu_seqlens_k.numpy()
    n = [int(cu[b + 1] - cu[b]) for b in range(B)]
    d = inp.key.shape[-1]
    rows = [(inp.key.numpy()[cu[b]:cu[b + 1], 0], inp.key_scale.numpy()[cu[b]:cu[b + 1]]) for b in range(B)]
    kw = {k: v for k, v in inp.__dict__.items()}
    kw.update(layout_k=layout_k, block_table=None, seqused_k=None, cu_seqlens_k=None)
    if layout_k == "TND":
        kw["key"] = torch.from_numpy(np.concatenate([r[0] for r in rows])).view(-1, 1, d)
        kw["key_scale"] = torch.from_numpy(np.concatenate([r[1] for r in rows]))
        kw["cu_seqlens_k"] = torch.tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int32)
    elif layout_k == "BSND":
        S = max(n) + 3
        key = np.full((B, S, 1, d), 0x7F, np.uint8)
        ks = np.full((B, S), np.nan, np.float32)
        for b in range(B):
            key[b, :n[b], 0] = rows[b][0]
            ks[b, :n[b]] = rows[b][1]
        kw.update(key=torch.from_numpy(key), key_scale=torch.from_numpy(ks),
                  seqused_k=torch.tensor(n, dtype=torch.int32))
    else:  # paged with block size 8, blocks placed at random
        bs = 8
        nb = [(x + bs - 1) // bs for x in n]
        perm = np.random.default_rng(seed).permutation(sum(nb) + 2)
        key = np.full((sum(nb) + 2, bs, 1, d), 0x7F, np.uint8)
        ks = np.full((sum(nb) + 2, bs), np.nan, np.float32)
        tab = np.full((B, max(nb) + 1), perm[-1], np.int32)
        o = 0
        for b in range(B):
            for j in range(nb[b]):
                blk = perm[o]
                o += 1
                tab[b, j] = blk
                m = min(bs, n[b] - j * bs)
                key[blk, :m, 0] = rows[b][0][j * bs:j * bs + m]
                ks[blk, :m] = rows[b][1][j * bs:j * bs + m]
        kw.update(key=torch.from_numpy(key), key_scale=torch.from_numpy(ks), block_table=torch.from_numpy(tab),
                  seqused_k=torch.tensor(n, dtype=torch.int32))
    return IndexerInputs(**kw)


def test_layouts_agree():
    inp = make_indexer(seed=6, q_lens=[4, 2, 3], k_lens=[45, 17, 60], layout_q="TND", layout_k="TND", topk=12,
                       residual=[1, 0, 3], g=16)
    want = oracle_indexer(inp)
    for lay in ("TND", "BSND", "PA_BBND"):
        assert np.array_equal(oracle_indexer(_relayout(inp, lay)), want), lay


def test_bsnd_query_layout_matches_tnd():
    a = make_indexer(seed=8, q_lens=[3, 3], k_lens=[33, 41], layout_q="TND", topk=9, residual=[2, 1], g=8)
    b = IndexerInputs(**{**a.__dict__, "layout_q": "BSND", "q_s": 3, "cu_seqlens_q": None})
    assert np.array_equal(oracle_indexer(a), oracle_indexer(b))


def test_power_of_two_rescaling_keeps_indices():
    inp = make_indexer(seed=9, q_lens=[6], k_lens=[90], layout_q="TND", topk=20, residual=[0], g=32)
    want = oracle_indexer(inp)
    for field, f in (("weights", 4.0), ("q_scale", 0.25), ("key_scale", 2.0)):
        x = IndexerInputs(**inp.__dict__)
        setattr(x, field, getattr(inp, field) * f)
        assert np.array_equal(oracle_indexer(x), want), field
