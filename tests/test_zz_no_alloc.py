"""csmla_forward_noalloc (the entry point for callers that cannot allocate)
against csmla_forward with a caller workspace: the same kernels, so the
outputs must be bit-identical, and both meet the oracle.  Two calls in a row,
the second with a smaller input, with key splits forced so that the split
partials really live in the library's static scratch; the scratch keeps the
first call's contents when the second runs."""
import os

import numpy as np
import pytest
import torch

import sparse_compressed_mla_amd as m
from oracle import oracle_forward
from workloads import make_custom
from tests.parity_util import compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _case(seed, q_lens, ori):
    rng = np.random.default_rng(seed)
    cmp = [o // 4 for o in ori]
    idx = rng.integers(-2, max(cmp) + 3, size=(sum(q_lens), 200))
    idx[rng.random(idx.shape) < 0.2] = -1
    return make_custom(seed=seed, q_lens=q_lens, ori_lens=ori, cmp_lens=cmp, cmp_ratio=4,
                       residual=[o % 4 for o in ori], indices=idx, return_lse=True)


def _plan(g, splits):
    os.environ["CSMLA_KERNEL"] = "split"
    os.environ["CSMLA_SPLITS"] = str(splits)
    try:
        return m.Plan(g)
    finally:
        os.environ.pop("CSMLA_KERNEL", None)
        os.environ.pop("CSMLA_SPLITS", None)


def test_noalloc_matches_forward_two_calls():
    stream = torch.cuda.current_stream(DEV).cuda_stream
    for seed, q_lens, ori, splits in ((301, [3, 5, 4], [900, 1300, 700], 5), (302, [2, 1], [400, 260], 3)):
        inp = _case(seed, q_lens, ori)
        g = inp.to(DEV)
        plan = _plan(g, splits)
        print(f"[no-alloc] seed {seed}: t1={inp.t1} splits={plan.splits} workspace={plan.workspace_bytes}",
              flush=True)
        assert plan.splits == splits and plan.workspace_bytes > 0
        out_ws = torch.empty(g.q.shape, dtype=torch.bfloat16, device=DEV)
        lse_ws = torch.empty(g.q.shape[:2], dtype=torch.float32, device=DEV)
        ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=DEV)
        m.csmla_forward(plan.problem, m.tensors_from(g, out_ws, lse_ws, ws), plan.metadata, stream)
        out_na = torch.full(g.q.shape, 7.0, dtype=torch.bfloat16, device=DEV)
        lse_na = torch.full(g.q.shape[:2], 7.0, dtype=torch.float32, device=DEV)
        m.csmla_forward_noalloc(plan.problem, m.tensors_from(g, out_na, lse_na, None), plan.metadata, stream)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws), "no-alloc output differs from the workspace forward"
        assert torch.equal(lse_na, lse_ws), "no-alloc lse differs from the workspace forward"
        ref = oracle_forward(inp)
        compare(out_na.float().cpu().numpy(), ref.out, list(range(inp.t1)), lse_na.cpu().numpy(), ref.lse,
                name=f"no-alloc seed {seed}")
