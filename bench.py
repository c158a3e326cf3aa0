#!/usr/bin/env python3
"""Throughput of quantized sparse shared-KV MLA attention on one MI355X.

Workload (default): CSA decode — B=32 query tokens (S_q=1), 64 heads, D=512,
fp8 e4m3 q / KV with per-token fp32 descales, paged KV (block 128), ori
length 8192 with a 128-token band (left 127, right 0), cmp_ratio 4 (2048
compressed tokens) and 512 top-k indices per token drawn uniformly without
replacement, sinks ~ N(0,1).  Synthetic, seeded data.

A step is one csmla_forward over one batch (the whole path: key resolution,
gather, QK^T, masks and sink, softmax, P V, epilogue, and the split-KV combine
when the plan splits keys).  The decode-shaped workloads run as consecutive
model layers would: --layers copies of the KV pools, each layer with its own
q, q descales, top-k index rows and output (block tables, lengths and sinks
shared); step k runs layer k % layers, so every step's rows come from HBM,
not from the 256 MB Infinity Cache.  Exactly --steps forwards are timed
after --warmup untimed ones, with HIP events on the stream the kernels run
on: launched one after another behind a short spin kernel that keeps the
GPU busy while the host submits them (--timing eager, the default), or as
replays of HIP graphs over the layers (--timing graph).  Either way the
graphs are captured and each replay is checked equal to the eager forwards.
The plan is made once per pass over the layers.

Prints one JSON line.  --gpus above 1 is refused: this build runs on one GPU.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0   # dense fp8 MFMA, MI355X
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X
# bytes of one KV row the method reads: fp8 codes + a 4-byte descale; a bf16
# row; a packed row's rope, nope and scale bytes (its 57 pad bytes are not read)
ROW_BYTES = {"fp8": 512 + 4, "bf16": 1024, "packed640": 128 + 448 + 7}
METRIC = "CSA decode query-tokens/s + effective KV HBM GB/s (% roofline), 1 MI355X"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("csmla_kernels.hip", "csmla_host.cpp", "csmla_internal.h"):
        with open(os.path.join(ROOT, "sparse_compressed_mla_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"attn_{workload}_pmc_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--layers", type=int, default=48,
                    help="model layers rotated through (each its own KV pool copy, q, indices and output)")
    ap.add_argument("--copy-budget-gb", type=float, default=96.0,
                    help="device memory the KV pool copies may take (caps --layers for large caches)")
    ap.add_argument("--batch", type=int, default=0, help="batch of the decode workloads (0: the config's)")
    ap.add_argument("--timing", choices=["eager", "graph"], default="eager",
                    help="timed forwards as launches one after another, or as replays of captured graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of each oracle timing sample (one thread, then all threads)")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--kv-format", choices=["fp8", "bf16", "packed640"], default="fp8",
                    help="KV rows of the attention workloads: fp8 with descales (q fp8), or bf16 / packed "
                         "640-byte rows (q bf16)")
    ap.add_argument("--workload", choices=["csa_decode", "csa_prefill", "swa_tiny", "hca_decode", "csa_mtp",
                                           "idx_csa_decode", "idx_csa_mtp_long", "idx_csa_prefill"],
                    default="csa_decode",
                    help="csa_decode (default, the headline line), csa_prefill (fp8 MFMA utilisation), one of "
                         "the other attention configurations (forward time and effective KV bytes), or an "
                         "indexer top-k workload (idx_*)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain device-to-device copies of 512 MiB (the reference kernel that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters to bytes) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the path would shard by batch across GPUs; that is not built.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = 512 << 20
        src = torch.full((n,), 7, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)
        return

    import sparse_compressed_mla_amd as m
    from workloads import make_config

    if args.workload.startswith("idx_"):
        indexer(args, m, torch, np)
        return
    if args.workload == "csa_prefill":
        prefill(args, m, make_config, torch, np)
        return

    rotated(args, m, make_config, torch, np)


# ---------------------------------------------------------------------------
# helpers shared by the workloads
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(run_one, n_items, seconds, unit, what):
    """The oracle as it stands, timed on the host on a bounded sample: items
    (query tokens or rows) run one at a time in a fixed shuffled order until
    `seconds` have passed, once with BLAS on one thread and once on all the
    threads the BLAS pool holds.  The all-threads figure is `value`."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    order = np.random.default_rng(0).permutation(n_items)

    def timed():
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < seconds or done == 0:
            run_one(int(order[done % n_items]))
            done += 1
        return done, time.perf_counter() - t0

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    with threadpool_limits(limits=1):
        d1, s1 = timed()
    dn, sn = timed()
    return {"value": round(dn / sn, 3), "unit": unit, "cores": int(threads), "kind": "oracle",
            "sample": f"{dn} {what} in {sn:.1f} s on {threads} BLAS threads (float64 NumPy oracle, "
                      f"{cpu_model()})",
            "cpu_model": cpu_model(),
            "single_thread": {"value": round(d1 / s1, 3), "unit": unit, "cores": 1,
                              "sample": f"{d1} {what} in {s1:.1f} s on one thread"}}


def unique_rows(m, inp, np, torch):
    """(token, key) pairs and rows unique per batch of the resolved key lists
    (csmla_debug_resolve; bit-exact against the oracle in the GPU tests)."""
    keys, counts = m.debug_resolve(inp, 1024 if inp.topk <= 1024 else 4096)
    torch.cuda.synchronize()
    keys, counts = keys.cpu().numpy(), counts.cpu().numpy()
    from oracle.attention import token_table
    tt = token_table(inp)
    per_batch = {}
    for t in range(inp.t1):
        n_o, n_c = counts[t]
        s = per_batch.setdefault(tt[t][0], set())
        s.update(("o", int(x)) for x in keys[t, :n_o])
        s.update(("c", int(x)) for x in keys[t, n_o:n_o + n_c])
    return int(counts.sum()), sum(len(v) for v in per_batch.values())


def cover_submission(torch, stream):
    """Queue a short spin kernel (well under a millisecond of GPU time) on
    `stream` ahead of the start event, so that the host's submission of the
    timed work (a graph launch takes some tens of microseconds) happens while
    the GPU is still busy: the events then bracket the forwards running back
    to back, as a model's layer loop runs them, and not the host's launch
    latency.  Untimed."""
    with torch.cuda.stream(stream):
        torch.cuda._sleep(1_000_000)


def timed_graph_steps(m, torch, plan, tens, dev, steps, warmup, timing="eager"):
    """Forward i of a pass uses layer i's tensors.  Graphs of forwards over
    the layers are captured once (a full pass, and the partial passes the
    step counts need); each is replayed once and checked equal to the eager
    forwards before the warm-up.
    Warm-up runs `warmup` untimed forwards on the last layers; the timed
    region runs exactly `steps` forwards from layer 0 on, with HIP events
    on the stream the kernels run on, as launches one after another
    (timing "eager") or as graph replays ("graph": full passes, then the
    partial one; each replay adds a fixed ~25 us on this stack, which a model
    pays once per graph of all its layers).  The host planner runs once per
    full pass (its host time is reported apart).  Returns (ms for the steps,
    host planner seconds, passes, host seconds spent submitting the timed
    steps)."""
    L = len(tens)
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))

    def fwd(l):
        m.csmla_forward(plan.problem, tens[l][0], plan.metadata, cap.cuda_stream)

    with torch.cuda.stream(cap):
        for l in range(L):
            fwd(l)
    torch.cuda.synchronize()
    eager = [t[1].clone() for t in tens]

    def capture(layers):
        if not layers:
            return None
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for l in layers:
                fwd(l)
        torch.cuda.synchronize()
        return g

    full = capture(list(range(L)))
    part_k = capture(list(range(steps % L)))
    part_w = capture(list(range(L - warmup % L, L)) if warmup % L else [])
    # every graph is replayed once here and checked (this first replay also
    # uploads the graph, which otherwise costs ~30 us inside the first timed
    # replay)
    for g, layers in ((full, range(L)), (part_k, range(steps % L)), (part_w, range(L - warmup % L, L))):
        if g is None:
            continue
        for t in tens:
            t[1].zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(cap):
            g.replay()
        torch.cuda.synchronize()
        for l in layers:
            assert torch.equal(tens[l][1], eager[l]), f"graph replay differs from the eager forward (layer {l})"
    with torch.cuda.stream(cap):
        if timing == "eager":
            for i in range(warmup):
                fwd((L - warmup % L + i) % L)
        else:
            if part_w is not None:
                part_w.replay()
            for _ in range(warmup // L):
                full.replay()
    torch.cuda.synchronize()
    hl, keep = m.host_lengths_from(tens[0][2])
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_plan = 0.0
    cover_submission(torch, cap)
    with torch.cuda.stream(cap):
        start.record(cap)
        t_sub = time.perf_counter()
        if timing == "eager":
            for i in range(steps):
                if i % L == L - 1:
                    t0 = time.perf_counter()
                    m.csmla_plan(plan.problem, hl)
                    t_plan += time.perf_counter() - t0
                fwd(i % L)
        else:
            for _ in range(steps // L):
                t0 = time.perf_counter()
                m.csmla_plan(plan.problem, hl)
                t_plan += time.perf_counter() - t0
                full.replay()
            if part_k is not None:
                part_k.replay()
        stop.record(cap)
        t_sub = time.perf_counter() - t_sub
    torch.cuda.synchronize()
    return start.elapsed_time(stop), t_plan, max(1, steps // L), t_sub


def kernel_name(plan, fmt="fp8"):
    if fmt != "fp8":
        return f"bk_kernel<{fmt}> (bf16 q, {plan.splits} key splits)" + (" + combine_kernel" if plan.splits > 1
                                                                          else "")
    if plan.split_key:
        return f"sk_kernel (split-key decode: 64 heads, {plan.splits} key splits per token, in-kernel merge)"
    if plan.head_group == 64:
        return "pf_kernel (whole-token)"
    if plan.head_group > 0 and plan.dk_parts > 1:
        return (f"dk_kernel (head-split, groups of {plan.head_group} heads, keys in {plan.dk_parts} parts "
                "merged in-kernel)")
    if plan.head_group > 0:
        return f"dk_kernel (head-split, groups of {plan.head_group} heads over whole key lists)"
    return f"attn_kernel<0> (split attention, {plan.splits} key splits)" + (" + combine_kernel" if plan.splits > 1
                                                                           else "")


ROTATED = {"csa_decode": 2, "hca_decode": 3, "csa_mtp": 4, "swa_tiny": 1}
CONFIG_TEXT = {
    2: dict(q_tokens_per_batch=1, ori_len=8192, band=128, cmp_ratio=4, topk=512),
    3: dict(q_tokens_per_batch=1, ori_len="U[32768, 65536]", band=128, cmp_ratio=128, topk=0),
    4: dict(q_tokens_per_batch=2, ori_len="U[65536, 131072]", band=128, cmp_ratio=4, topk=512),
    1: dict(q_tokens_per_batch=4, ori_len="300 / 200", band=128, cmp_ratio=1, topk=0),
}


def rotated(args, m, make_config, torch, np):
    """A decode-shaped workload as consecutive model layers would run it:
    `layers` copies of the KV pools, each layer with its own q, q descales
    and (CSA) top-k index rows, drawn by the config's recipe, and its own
    output; block tables, lengths and sinks are shared, as the layers of
    one sequence share them.  Step k runs layer k % layers, so each step's
    KV rows, queries and indices come from HBM and not from the 256 MB
    Infinity Cache."""
    from workloads import redraw_query_side
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    k = ROTATED[args.workload]
    kw = {"batch": args.batch} if k in (2, 3, 4) and args.batch else {}
    fmt = args.kv_format
    if fmt != "fp8":
        kw.update(q_format="bf16", kv_format=fmt)
    print(f"[bench] building inputs: {args.workload} {kw}", file=sys.stderr, flush=True)
    inp = make_config(k, device=dev, **kw)
    T1 = inp.t1
    if not args.no_parity:
        from oracle import oracle_forward
        from tests.parity_util import compare
        toks = sorted({0, T1 // 2, T1 - 1})
        cpu = inp.to("cpu")
        ref = oracle_forward(cpu, toks)
        o, _ = m.forward(inp)
        torch.cuda.synchronize()
        compare(o.float().cpu().numpy(), ref.out, toks, name="bench precheck", verbose=False)
        print("[bench] parity precheck ok", file=sys.stderr, flush=True)
    pairs, uniq = unique_rows(m, inp, np, torch)
    kv_bytes = uniq * ROW_BYTES[fmt]
    out_bytes = T1 * 64 * 512 * 2
    q_bytes = T1 * 64 * (512 + 4) if fmt == "fp8" else T1 * 64 * 512 * 2
    other_bytes = q_bytes + out_bytes + 4 * inp.topk * T1
    pool = sum(x.numel() * x.element_size() for x in (inp.ori_kv, inp.ori_kv_descale, inp.cmp_kv, inp.cmp_kv_descale)
               if x is not None)
    L = max(2, min(args.layers, int(args.copy_budget_gb * 1e9 // pool)))
    layers = [inp]
    for l in range(1, L):
        c = redraw_query_side(inp, k, l)
        cl = lambda x: None if x is None else x.clone()
        c.ori_kv, c.ori_kv_descale = cl(inp.ori_kv), cl(inp.ori_kv_descale)
        if inp.cmp_kv is not None:
            c.cmp_kv, c.cmp_kv_descale = cl(inp.cmp_kv), cl(inp.cmp_kv_descale)
        layers.append(c)
    print(f"[bench] {L} layers resident: KV pools {L * pool / 1e9:.1f} GB, {kv_bytes / 1e6:.2f} MB of KV rows "
          f"touched per step", file=sys.stderr, flush=True)
    plan = m.Plan(inp)
    tens = []
    for x in layers:
        out = torch.empty(x.q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(x.q.shape[:2], dtype=torch.float32, device=dev) if x.return_lse else None
        ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
        tens.append((m.tensors_from(x, out, lse, ws if plan.workspace_bytes else None), out, x, lse, ws))
    K, W = args.steps, args.warmup
    total_ms, t_plan, passes, t_sub = timed_graph_steps(m, torch, plan, tens, dev, K, W, args.timing)
    timing = args.timing
    if timing == "eager" and t_sub * 1e3 > 0.8 * total_ms:
        # The host submitted the forwards about as fast as the GPU ran them, so
        # the queue may have drained and the events timed the host: time graph
        # replays instead (each replay adds a fixed ~25 us) and say so.
        print(f"[bench] eager forwards host-bound ({1e6 * t_sub / K:.1f} us host per forward against "
              f"{1e3 * total_ms / K:.1f} us on the GPU): timing graph replays", file=sys.stderr, flush=True)
        total_ms, t_plan, passes, t_sub = timed_graph_steps(m, torch, plan, tens, dev, K, W, "graph")
        timing = "graph (eager host-bound)"
    fwd_ms = total_ms / K
    value = T1 * K / (total_ms / 1e3)
    achieved = kv_bytes / (fwd_ms / 1e3) / 1e9
    kern = kernel_name(plan, fmt)
    print(f"[bench] {args.workload}: forward {fwd_ms * 1e3:.2f} us per step over {K} steps ({timing}, {L} "
          f"layers); {kern}, grid {plan.grid}; plan {1e6 * t_plan / passes:.0f} us host per pass",
          file=sys.stderr, flush=True)
    headline = args.workload == "csa_decode" and fmt == "fp8"
    wname = args.workload if fmt == "fp8" else f"{args.workload}_{fmt}"
    res = {
        "metric": METRIC if headline else f"{wname} query-tokens/s + effective KV HBM GB/s, 1 MI355X",
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(fwd_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 (fp32 accumulate)" if fmt == "fp8" else
                 ("bf16 q and KV (fp32 accumulate)" if fmt == "bf16" else
                  "bf16 q, packed rows: bf16 rope + e4m3 nope x e8m0 scales, as bf16 (fp32 accumulate)"),
        "data": f"synthetic, seeded (workloads.make_config({k}); layers 1.. redraw q and indices)",
        "config": dict({"workload": wname, "batch": inp.batch, "n1": 64, "d": 512, "block_size": 128,
                        "kv_format": fmt,
                        "layers_rotated": L, "timing": timing, "host_submit_us": round(1e6 * t_sub / K, 2),
                        "splits": plan.splits, "grid": plan.grid,
                        "head_group": plan.head_group}, **CONFIG_TEXT[k]),
        "effective_kv_gbs": round(achieved, 1),
        "kv_bytes_per_step": kv_bytes,
        "total_bytes_per_step": kv_bytes + other_bytes,
        "pairs_per_step": pairs,
        "forward_us": round(fwd_ms * 1e3, 3),
        "plan_host_us": round(1e6 * t_plan / passes, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(wname), "kernel": kern},
    }
    if not args.no_cpu_baseline:
        from oracle import oracle_forward
        cpu = inp.to("cpu")
        res["cpu_baseline"] = cpu_baseline(lambda t: oracle_forward(cpu, [t]), T1, args.cpu_seconds,
                                           "query-tokens/s", f"{wname} query tokens")
    print(json.dumps(res), flush=True)


def prefill(args, m, make_config, torch, np):
    """CSA prefill (TND, B=4 x 4096 query tokens, per-tile-64 descales,
    return_softmax_lse): fp8 MFMA utilisation on the algorithmic flops
    4 * 64 * 512 per (query token, key) pair (S = Q K^T and O = P V over the
    64 heads).  The KV of one batch (4 x 4096 rows) is reused by every query
    token of the batch, so no layer rotation: the bound is the matrix cores."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fmt = args.kv_format
    kw = {} if fmt == "fp8" else dict(q_format="bf16", kv_format=fmt)
    print(f"[bench] building inputs: csa_prefill {kw}", file=sys.stderr, flush=True)
    inp = make_config(5, device=dev, **kw)
    T1 = inp.t1
    if not args.no_parity:
        from oracle import oracle_forward
        from tests.parity_util import compare
        toks = [0, 1500, T1 // 2 + 7, T1 - 1]
        cpu = inp.to("cpu")
        ref = oracle_forward(cpu, toks)
        o, _ = m.forward(inp)
        torch.cuda.synchronize()
        compare(o.float().cpu().numpy(), ref.out, toks, name="bench precheck", verbose=False)
        print("[bench] parity precheck ok", file=sys.stderr, flush=True)
    _, counts = m.debug_resolve(inp, 1024)
    torch.cuda.synchronize()
    pairs = int(counts.sum().item())
    flops = 4.0 * 64 * 512 * pairs
    plan = m.Plan(inp)
    out = torch.empty(inp.q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T1, 64), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    tens = m.tensors_from(inp, out, lse, ws if plan.workspace_bytes else None)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    steps = max(1, min(args.steps, 50))
    warm = max(1, min(args.warmup, 10))
    for _ in range(warm):
        m.csmla_forward(plan.problem, tens, plan.metadata, sp)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cover_submission(torch, stream)
    start.record(stream)
    for _ in range(steps):
        m.csmla_forward(plan.problem, tens, plan.metadata, sp)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    tflops = flops / (ms / 1e3) / 1e12
    peak = FP8_PEAK_TFLOPS if fmt == "fp8" else BF16_PEAK_TFLOPS
    print(f"[bench] prefill forward {ms * 1e3:.1f} us, {pairs} pairs, {tflops:.1f} TFLOP/s; "
          f"splits {plan.splits} grid {plan.grid} head_group {plan.head_group}", file=sys.stderr, flush=True)
    res = {
        "metric": ("CSA prefill query-tokens/s + fp8 MFMA TFLOP/s (% dense peak), 1 MI355X" if fmt == "fp8" else
                   f"CSA prefill ({fmt} KV, bf16 q) query-tokens/s + bf16 MFMA TFLOP/s (% dense peak), 1 MI355X"),
        "value": round(T1 / (ms / 1e3), 1), "unit": "query-tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8e4m3 S^T, f16 P V (fp32 accumulate)" if plan.head_group == 64 and fmt == "fp8"
                  else "fp8e4m3 (fp32 accumulate)" if fmt == "fp8" else "bf16 (fp32 accumulate)"),
        "data": "synthetic, seeded (workloads.make_config(5))",
        "config": {"workload": "csa_prefill" if fmt == "fp8" else f"csa_prefill_{fmt}", "batch": 4,
                   "q_tokens_per_batch": 4096, "n1": 64, "d": 512, "band": 128, "cmp_ratio": 4, "topk": 512,
                   "kv_scale": "per-tile-64" if fmt == "fp8" else fmt, "lse": True,
                   "splits": plan.splits, "grid": plan.grid},
        "pairs_per_step": pairs,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": None,
                     "kernel": (kernel_name(plan, fmt) if fmt != "fp8" else
                                "pf_kernel<1> (whole-token prefill: fp8 S^T, f16 P V, per-tile descales)"
                                if plan.head_group == 64 else
                                "attn_kernel<1> (split attention, per-tile descales)")},
    }
    if not args.no_cpu_baseline:
        from oracle import oracle_forward
        cpu = inp.to("cpu")
        res["cpu_baseline"] = cpu_baseline(lambda t: oracle_forward(cpu, [t]), T1, args.cpu_seconds,
                                           "query-tokens/s", "csa_prefill query tokens")
    print(json.dumps(res), flush=True)


def indexer(args, m, torch, np):
    """Lightning-indexer top-k (csmla_indexer_forward: score kernel + top-k
    kernel) on one of the indexer workloads.  Decode-shaped workloads are
    bound by HBM: algorithmic bytes = every batch's keys once (128 fp8 bytes
    + a 4-byte scale each) + the query rows (g x 128 bytes + 8 bytes of
    weight and scale per head) + the int32 index rows written.  The key pools
    are replicated over copies (read round-robin) so that no step finds them
    in the Infinity Cache.  Prefill is bound by the matrix cores: algorithmic
    flops = 2 x g x 128 per (query row, visible key) pair."""
    from workloads.indexer_gen import make_indexer_workload
    from oracle.indexer import token_context
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    name = args.workload
    print(f"[bench] building inputs: {name}", file=sys.stderr, flush=True)
    cpu = make_indexer_workload(name)
    inp = cpu.to(dev)
    T1, g = inp.t1, inp.g
    vis = np.array([max(token_context(cpu, t)[4], 0) for t in range(T1)], dtype=np.int64)
    nkeys = np.array([token_context(cpu, t)[3] for t in range(T1)], dtype=np.int64)
    plan = m.IndexerPlan(inp)
    out = torch.empty((T1, 1, inp.topk), dtype=torch.int32, device=dev)
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    if not args.no_parity:
        from oracle.indexer import oracle_scores, topk_positions
        rows = sorted({0, T1 // 2, T1 // 2 + 1, T1 - 1})
        m.indexer_forward(inp, out=out, workspace=ws, plan=plan)
        torch.cuda.synchronize()
        got = out.cpu().numpy().reshape(T1, -1)
        sc = ws.view(torch.float32)[: T1 * plan.stride].view(T1, plan.stride).cpu().numpy()
        for t in rows:
            v = int(vis[t])
            if v == 0:
                assert (got[t] == -1).all(), f"row {t} sees no key"
                continue
            ref = oracle_scores(cpu, t)
            assert np.allclose(sc[t, :v], ref, rtol=1e-3, atol=1e-3 * np.abs(ref).max()), f"row {t} scores"
            assert np.array_equal(got[t], topk_positions(sc[t, :v], inp.topk)), f"row {t} selection"
        print("[bench] parity precheck ok", file=sys.stderr, flush=True)
    decode_like = name != "idx_csa_prefill"
    copies = 1
    if decode_like:
        key_bytes = int(inp.key.numel()) + 4 * int(inp.key_scale.numel())
        copies = max(1, min(48, (1 << 30) // max(key_bytes, 1)))
    keys = [inp.key] + [inp.key.clone() for _ in range(copies - 1)]
    scales = [inp.key_scale] + [inp.key_scale.clone() for _ in range(copies - 1)]
    tens = []
    for c in range(copies):
        t = m.indexer_tensors_from(inp, out, ws)
        t.key, t.key_dequant_scale = keys[c].data_ptr(), scales[c].data_ptr()
        tens.append(t)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    steps = max(1, min(args.steps, 200))
    warm = max(1, min(args.warmup, 20))
    for i in range(warm):
        m.csmla_indexer_forward(plan.problem, tens[i % copies], plan.metadata, sp)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cover_submission(torch, stream)
    start.record(stream)
    for i in range(steps):
        m.csmla_indexer_forward(plan.problem, tens[i % copies], plan.metadata, sp)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    # keys each batch holds (every key of a batch is read once per call)
    per_batch = {}
    for t in range(T1):
        b = token_context(cpu, t)[0]
        per_batch[b] = int(nkeys[t]) if vis[t] > 0 else per_batch.get(b, 0)
    key_bytes = sum(per_batch.values()) * (128 + 4)
    alg_bytes = key_bytes + T1 * g * (128 + 8) + T1 * inp.topk * 4
    flops = 2.0 * g * 128 * float(vis.sum())
    gbs = alg_bytes / (ms / 1e3) / 1e9
    tflops = flops / (ms / 1e3) / 1e12
    kern = "idx_score_kernel + idx_topk_kernel (one csmla_indexer_forward)"
    if decode_like:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": kern}
    else:
        roof = {"bound": "mfma", "achieved": round(tflops, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / FP8_PEAK_TFLOPS, 4), "traffic": None, "kernel": kern}
    print(f"[bench] {name}: {ms * 1e3:.2f} us per call, {T1} rows, {gbs:.1f} GB/s algorithmic, "
          f"{tflops:.1f} TFLOP/s; tile tw={plan.metadata[4]} wt={plan.metadata[5]} kc={plan.metadata[6]}, "
          f"stride {plan.stride}, key copies {copies}", file=sys.stderr, flush=True)
    res = {
        "metric": f"{name} indexer query-rows/s, 1 MI355X", "value": round(T1 / (ms / 1e3), 1),
        "unit": "query-rows/s", "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3 (fp32 accumulate)",
        "data": f"synthetic, seeded (workloads.indexer_gen, {name})",
        "config": {"workload": name, "t1": T1, "g": g, "d": 128, "topk": int(inp.topk),
                   "layout_q": cpu.layout_q, "layout_k": cpu.layout_k, "visible_pairs": int(vis.sum())},
        "alg_bytes_per_step": alg_bytes, "flops_per_step": flops, "roofline": roof,
    }
    if not args.no_cpu_baseline:
        from oracle.indexer import oracle_indexer
        res["cpu_baseline"] = cpu_baseline(lambda t: oracle_indexer(cpu, [t]), T1, args.cpu_seconds,
                                           "query-rows/s", f"{name} rows")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
