#!/usr/bin/env python3
"""Throughput of quantized sparse shared-KV MLA attention on one MI355X.

Workload (default): CSA decode — B=32 query tokens (S_q=1), 64 heads, D=512,
fp8 e4m3 q / KV with per-token fp32 descales, paged KV (block 128), ori
length 8192 with a 128-token band (left 127, right 0), cmp_ratio 4 (2048
compressed tokens) and 512 top-k indices per token drawn uniformly without
replacement, sinks ~ N(0,1).  Synthetic, seeded data.

A step is one csmla_forward over one batch: as planned for this shape, the
head-split kernel alone (groups of 8 heads over whole key lists), or split
attention followed by the split-KV combine.  The KV pools are replicated over --layers distinct copies
and step k reads copy k % layers, as consecutive layers of a model would:
every step's KV rows come from HBM, not from the 256 MB Infinity Cache.
Block tables, indices and q are shared by the copies.  The plan is made
once per pass over the layers, as a model plans once per decode step.

Prints one JSON line (rank 0).  --gpus above 1 is refused: this build runs
on one GPU.
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
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--batch", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle timing sample")
    ap.add_argument("--no-parity", action="store_true")
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
    if args.workload != "csa_decode":
        other(args, m, make_config, torch, np)
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] building inputs: csa_decode batch={args.batch} layers={args.layers}", file=sys.stderr, flush=True)
    inp = make_config(2, device=dev, batch=args.batch)
    T1 = inp.t1

    # ---- parity precheck on a few rows (the oracle is the CPU reference) ----
    if not args.no_parity:
        from oracle import oracle_forward
        from tests.parity_util import compare
        toks = [0, T1 // 2, T1 - 1]
        cpu = inp.to("cpu")
        ref = oracle_forward(cpu, toks)
        o, _ = m.forward(inp)
        torch.cuda.synchronize()
        compare(o.float().cpu().numpy(), ref.out, toks, name="bench precheck", verbose=False)
        print("[bench] parity precheck ok", file=sys.stderr, flush=True)
        del cpu

    # ---- algorithmic bytes: unique KV rows per batch x (512 B + 4 B descale) ----
    nmax = 1024
    keys, counts = m.debug_resolve(inp, nmax)
    torch.cuda.synchronize()
    keys, counts = keys.cpu().numpy(), counts.cpu().numpy()
    uniq = 0
    tt = np.repeat(np.arange(args.batch), T1 // args.batch)
    for b in range(args.batch):
        ts = np.nonzero(tt == b)[0]
        ori = set(); cmp = set()
        for t in ts:
            n_o, n_c = counts[t]
            ori.update(keys[t, :n_o].tolist())
            cmp.update(keys[t, n_o:n_o + n_c].tolist())
        uniq += len(ori) + len(cmp)
    kv_bytes = uniq * (512 + 4)
    pairs = int(counts.sum())
    other_bytes = T1 * 64 * 512 + T1 * 64 * 4 + T1 * 64 * 512 * 2 + int(inp.cmp_sparse_indices.numel()) * 4

    # ---- layer copies of the KV pools ----
    layers = []
    for l in range(args.layers):
        if l == 0:
            layers.append(inp)
            continue
        c = type(inp)(**{k: v for k, v in inp.__dict__.items()})
        c.ori_kv = inp.ori_kv.clone(); c.ori_kv_descale = inp.ori_kv_descale.clone()
        c.cmp_kv = inp.cmp_kv.clone(); c.cmp_kv_descale = inp.cmp_kv_descale.clone()
        layers.append(c)
    pool_gb = sum(x.ori_kv.numel() + x.cmp_kv.numel() for x in layers) / 1e9
    print(f"[bench] KV pools resident: {pool_gb:.1f} GB over {args.layers} layers", file=sys.stderr, flush=True)

    plan = m.Plan(inp)
    out = torch.empty(inp.q.shape, dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    tens = [m.tensors_from(x, out, None, ws if plan.workspace_bytes else None) for x in layers]
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    hl, keep = m.host_lengths_from(inp)

    # ---- one HIP graph holding a forward per layer (no host work per step) ----
    L = args.layers
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        for l in range(L):                       # eager warm-up on the capture stream
            m.csmla_forward(plan.problem, tens[l], plan.metadata, cap.cuda_stream)
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for l in range(L):
            m.csmla_forward(plan.problem, tens[l], plan.metadata, cap.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(2):                          # replays must equal the eager result
        out.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(cap):
            graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "graph replay differs from the eager forward"

    reps_w = max(1, -(-args.warmup // L))
    reps = max(1, -(-args.steps // L))
    K = reps * L
    with torch.cuda.stream(cap):
        for _ in range(reps_w):
            graph.replay()
    torch.cuda.synchronize()

    # ---- timed region: K steps (reps x L layers), events on the kernels' stream ----
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_plan = 0.0
    with torch.cuda.stream(cap):                  # replay() launches on the current stream
        start.record(cap)
        for r in range(reps):
            t0 = time.perf_counter()
            m.csmla_plan(plan.problem, hl)       # the planner runs once per pass over the layers
            t_plan += time.perf_counter() - t0
            graph.replay()
        stop.record(cap)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    fwd_ms = total_ms / K
    ms_per_step = fwd_ms
    value = T1 * K / (total_ms / 1e3)
    achieved = kv_bytes / (fwd_ms / 1e3) / 1e9
    print(f"[bench] forward {fwd_ms * 1e3:.2f} us per step over {K} steps (graph of {L} layers); "
          f"splits {plan.splits} grid {plan.grid}; plan {1e6 * t_plan / reps:.0f} us host per pass",
          file=sys.stderr, flush=True)

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": reps_w * L,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 (fp32 accumulate)",
        "data": "synthetic, seeded (workloads.make_config(2))",
        "config": {"workload": "csa_decode", "batch": args.batch, "q_tokens_per_batch": 1, "n1": 64, "d": 512,
                   "ori_len": 8192, "band": 128, "cmp_ratio": 4, "topk": 512, "block_size": 128,
                   "layers_rotated": args.layers, "splits": plan.splits, "grid": plan.grid},
        "effective_kv_gbs": round(achieved, 1),
        "kv_bytes_per_step": kv_bytes,
        "total_bytes_per_step": kv_bytes + other_bytes,
        "pairs_per_step": pairs,
        "forward_us": round(fwd_ms * 1e3, 3),
        "plan_host_us": round(1e6 * t_plan / reps, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("csa_decode"),
                     "kernel": ("dk_kernel (head-split attention, whole key lists)" if plan.head_group > 0
                                else "attn_kernel<0> + combine_kernel (split attention, split-KV combine)")},
    }

    # ---- CPU baseline: the oracle as it stands, on a bounded sample ----
    if not args.no_cpu_baseline:
        from oracle import oracle_forward
        cpu = inp.to("cpu")
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:
            cores = len(os.sched_getaffinity(0))
        done = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds or done == 0:
            oracle_forward(cpu, [done % T1])
            done += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(done / dt, 2), "unit": "query-tokens/s", "cores": int(cores),
                               "kind": "oracle",
                               "sample": f"{done} csa_decode query tokens (640 keys each) in {dt:.1f} s, "
                                         f"float64 NumPy oracle on the host"}
    print(json.dumps(res), flush=True)


OTHER = {"swa_tiny": 1, "hca_decode": 3, "csa_mtp": 4}


def other(args, m, make_config, torch, np):
    """Forward time of another configuration (inputs resident, one KV pool,
    eager launches timed with HIP events on the kernels' stream), effective
    KV bytes = unique (row) keys of each batch x 516 B."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    k = OTHER[args.workload]
    print(f"[bench] building inputs: {args.workload}", file=sys.stderr, flush=True)
    inp = make_config(k, device=dev)
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
    keys, counts = m.debug_resolve(inp, 1024)
    torch.cuda.synchronize()
    keys, counts = keys.cpu().numpy(), counts.cpu().numpy()
    pairs = int(counts.sum())
    rows = set()
    for t in range(T1):
        n_o, n_c = counts[t]
        rows.update(("o", int(x)) for x in keys[t, :n_o])
        rows.update(("c", int(x)) for x in keys[t, n_o:n_o + n_c])
    kv_bytes = len(rows) * 516
    plan = m.Plan(inp)
    out = torch.empty(inp.q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T1, 64), dtype=torch.float32, device=dev) if getattr(inp, "return_lse", False) else None
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    tens = m.tensors_from(inp, out, lse, ws if plan.workspace_bytes else None)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    steps = max(1, min(args.steps, 200))
    for _ in range(max(1, min(args.warmup, 20))):
        m.csmla_forward(plan.problem, tens, plan.metadata, sp)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        m.csmla_forward(plan.problem, tens, plan.metadata, sp)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    gbs = kv_bytes / (ms / 1e3) / 1e9
    kernel = ("pf_kernel (whole-token prefill)" if plan.head_group == 64
              else f"dk_kernel (head groups of {plan.head_group})" if plan.head_group > 0
              else f"attn_kernel (splits {plan.splits})" + (" + combine_kernel" if plan.splits > 1 else ""))
    print(f"[bench] {args.workload} forward {ms * 1e3:.2f} us, {T1} query tokens, {pairs} pairs, "
          f"{gbs:.1f} GB/s effective KV; {kernel}, grid {plan.grid}", file=sys.stderr, flush=True)
    print(json.dumps({
        "metric": f"{args.workload} query-tokens/s + effective KV HBM GB/s, 1 MI355X",
        "value": round(T1 / (ms / 1e3), 1), "unit": "query-tokens/s", "n_gpus": 1, "steps": steps,
        "ms_per_step": round(ms, 6), "higher_is_better": True, "data": f"synthetic, seeded (workloads.make_config({k}))",
        "config": {"workload": args.workload, "t1": T1, "splits": plan.splits, "grid": plan.grid,
                   "head_group": plan.head_group},
        "pairs_per_step": pairs, "kv_bytes_per_step": kv_bytes,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": kernel}}), flush=True)


def prefill(args, m, make_config, torch, np):
    """CSA prefill (TND, B=4 x 4096 query tokens, per-tile-64 descales,
    return_softmax_lse): fp8 MFMA utilisation on the algorithmic flops
    4 * 64 * 512 per (query token, key) pair (S = Q K^T and O = P V over the
    64 heads).  The KV of one batch (4 x 4096 rows) is reused by every query
    token of the batch, so no layer rotation: the bound is the matrix cores."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] building inputs: csa_prefill", file=sys.stderr, flush=True)
    inp = make_config(5, device=dev)
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
    start.record(stream)
    for _ in range(steps):
        m.csmla_forward(plan.problem, tens, plan.metadata, sp)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    tflops = flops / (ms / 1e3) / 1e12
    print(f"[bench] prefill forward {ms * 1e3:.1f} us, {pairs} pairs, {tflops:.1f} TFLOP/s; "
          f"splits {plan.splits} grid {plan.grid} head_group {plan.head_group}", file=sys.stderr, flush=True)
    res = {
        "metric": "CSA prefill query-tokens/s + fp8 MFMA TFLOP/s (% dense peak), 1 MI355X",
        "value": round(T1 / (ms / 1e3), 1), "unit": "query-tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8e4m3 S^T, f16 P V (fp32 accumulate)" if plan.head_group == 64
                  else "fp8e4m3 (fp32 accumulate)"),
        "data": "synthetic, seeded (workloads.make_config(5))",
        "config": {"workload": "csa_prefill", "batch": 4, "q_tokens_per_batch": 4096, "n1": 64, "d": 512,
                   "band": 128, "cmp_ratio": 4, "topk": 512, "kv_scale": "per-tile-64", "lse": True,
                   "splits": plan.splits, "grid": plan.grid},
        "pairs_per_step": pairs,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / FP8_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": ("pf_kernel<1> (whole-token prefill: fp8 S^T, f16 P V, per-tile descales)"
                                if plan.head_group == 64 else
                                "attn_kernel<1> (split attention, per-tile descales)")},
    }
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
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:
            cores = len(os.sched_getaffinity(0))
        order = np.random.default_rng(0).permutation(T1)
        t0 = time.time()
        done = 0
        for t in order:
            oracle_indexer(cpu, [int(t)])
            done += 1
            if time.time() - t0 > args.cpu_seconds:
                break
        dt = time.time() - t0
        res["cpu_baseline"] = {"value": round(done / dt, 3), "unit": "query-rows/s",
                               "cores": int(cores), "kind": "oracle",
                               "sample": f"{done} random rows of {name} in {dt:.1f} s, NumPy oracle on the host"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
