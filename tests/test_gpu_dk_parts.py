"""GPU parity of the head-split decode kernel's key parts: each (token, head
group) split into parts of whole 128-key tiles, the last part merging the
others' partial outputs inside the kernel through tagged exchange words.

One workspace is reused across calls and across plans with other part counts
(the slots' epochs and presence words carry over from call to call), and the
bounded waits' take-over paths are forced from the host: writing parts that
arrive only after the merging part has given up on them, and a merging part
that gives up at once.  Every forced call is followed by ordinary calls on the
same workspace.  Bar as in test_gpu_parity (oracle, 1e-2 + 1e-2|r|, lse 1e-3),
and a repeated call must reproduce its output bit for bit.
"""
import os

import numpy as np
import pytest
import torch

import sparse_compressed_mla_amd as m
from oracle import oracle_forward
from workloads import make_config
from tests.parity_util import compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ENV_KEYS = ("CSMLA_KERNEL", "CSMLA_DK_PARTS", "CSMLA_DK_TEST")
WS_BYTES = 4096 + 256 * 33792   # sync words + exchange slots: what a key-part plan asks for


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(autouse=True)
def clean_env():
    saved = {k: os.environ.pop(k, None) for k in ENV_KEYS}
    yield
    for k, v in saved.items():
        os.environ.pop(k, None)
        if v is not None:
            os.environ[k] = v


def plan_with(inp_g, kernel, parts, test=None):
    os.environ["CSMLA_KERNEL"] = kernel
    os.environ["CSMLA_DK_PARTS"] = str(parts)
    if test is not None:
        os.environ["CSMLA_DK_TEST"] = str(test)
    try:
        return m.Plan(inp_g)
    finally:
        for k in ENV_KEYS:
            os.environ.pop(k, None)


def run(inp_g, plan, ws):
    out, lse = m.forward(inp_g, plan=plan, workspace=ws)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), (lse.cpu().numpy() if lse is not None else None)


def check_case(name, inp, plan, ws, ref, repeats=2):
    g = inp.to(DEV)
    first = None
    for r in range(repeats):
        say(f"case {name} call {r}: t1={inp.t1} head_group={plan.head_group} parts={plan.dk_parts} grid={plan.grid}")
        o, l = run(g, plan, ws)
        compare(o, ref.out, range(inp.t1), l, ref.lse, name=f"{name} call {r}")
        if first is None:
            first = o
        else:
            assert np.array_equal(o, first), f"{name}: call {r} differs from call 0"


def test_parts_workspace_reused_across_plans():
    """Plans with 2 and 4 parts, in 16- and 8-head groups, one after another on
    one workspace (a slot is a writer's in one plan and unused or another
    group's in the next), each called twice."""
    ws = torch.zeros(WS_BYTES, dtype=torch.uint8, device=DEV)
    cases = [("B32 16-head", dict(batch=32), "heads16", 2), ("B4 16-head", dict(batch=4), "heads16", 4),
             ("B16 8-head", dict(batch=16), "heads8", 2), ("B8 16-head", dict(batch=8), "heads16", 4),
             ("B32 16-head again", dict(batch=32), "heads16", 2)]
    for name, kw, kernel, want in cases:
        inp = make_config(2, **kw)
        inp.return_lse = kw["batch"] == 8
        plan = plan_with(inp.to(DEV), kernel, 8)
        assert plan.dk_parts == want and plan.head_group == int(kernel[5:]), (name, plan.dk_parts, plan.head_group)
        assert plan.workspace_bytes == WS_BYTES
        check_case(name, inp, plan, ws, oracle_forward(inp))


@pytest.mark.parametrize("hook", [1, 2])
def test_parts_take_over_then_ordinary_calls(hook):
    """hook 1: every writing part announces itself only after the merging part
    has given up on it, so the merger computes all parts itself and the late
    writers store nothing; hook 2: the merger gives up at once and, finding
    the writers arrived, takes their parts over after one more poll (their
    words land afterwards).  Both leave the workspace ready for ordinary
    calls, which follow on the same buffer."""
    ws = torch.zeros(WS_BYTES, dtype=torch.uint8, device=DEV)
    inp = make_config(2, batch=8)
    inp.return_lse = True
    ref = oracle_forward(inp)
    g = inp.to(DEV)
    forced = plan_with(g, "heads16", 8, test=hook)
    assert forced.dk_parts == 4
    check_case(f"hook {hook}", inp, forced, ws, ref, repeats=1)
    plain = plan_with(g, "heads16", 8)
    check_case(f"after hook {hook}", inp, plain, ws, ref, repeats=3)
    check_case(f"hook {hook} again", inp, forced, ws, ref, repeats=1)
    check_case(f"after hook {hook} again", inp, plain, ws, ref, repeats=2)


def test_parts_lengths_leave_some_parts_empty():
    """Tokens whose key lists span fewer tiles than there are parts (cmp
    top-k lengths of 0..600 next to the 128 band keys): the empty parts write
    nothing and the merger skips them (or has no keys of its own)."""
    ws = torch.zeros(WS_BYTES, dtype=torch.uint8, device=DEV)
    inp = make_config(2, batch=8)
    inp.return_lse = True
    rng = np.random.default_rng(5)
    tkl = np.array([0, 1, 100, 127, 128, 129, 384, 600], dtype=np.int32)
    inp.cmp_topk_length = torch.from_numpy(tkl[rng.permutation(8)])
    ref = oracle_forward(inp)
    plan = plan_with(inp.to(DEV), "heads16", 8)
    assert plan.dk_parts == 4
    check_case("topk lengths", inp, plan, ws, ref, repeats=2)


@pytest.mark.parametrize("batch", [12, 20, 28])
def test_default_plan_16_head_parts(batch, monkeypatch):
    """12 to 28 decode tokens: the planner's own choice is 16-head groups in
    two key parts (no override); parity on two calls of one workspace."""
    for k in ("CSMLA_KERNEL", "CSMLA_DK_PARTS", "CSMLA_DK_TEST"):
        monkeypatch.delenv(k, raising=False)
    inp = make_config(2, batch=batch)
    inp.return_lse = True
    plan = m.Plan(inp.to(DEV))
    assert plan.head_group == 16 and plan.dk_parts == 2, (plan.head_group, plan.dk_parts)
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=DEV)
    check_case(f"default plan B={batch}", inp, plan, ws, oracle_forward(inp))
