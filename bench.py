#!/usr/bin/env python3
"""Benchmark of MLA decode over a paged latent KV cache on one MI355X.

Default workload (the batch-decode configuration C1): batch 64, one query token per
sequence, 128 heads, head width 576 (512 latent + 64 rope), V = the 512 latent columns,
cache lengths drawn uniformly from [1024, 4096] (seed 355001), page size 64 with a
shuffled page table, bf16 q and cache ~ N(0, 1), scale 1/sqrt(192), causal mask, split-KV
partitions chosen by the library.  A step is one call of the whole decode path (attention
kernel + log-sum-exp combine) over the batch.

The timed steps rotate over several independent copies of the inputs (more bytes than the
256 MB last-level cache holds), so every step reads its cache rows from HBM.  `value` is
algorithmic bytes (every visible cache row once plus q) per step divided by the step time.
Prints one JSON line.

Other workloads (--workload): C0 tiny decode, C2 long-context decode, C4 sparse fp8
decode (GB/s, HBM roofline), C3 ragged prefill (TFLOP/s, bf16 MFMA roofline), M2 / M4
multi-token decode (the C1 batch with 2 / 4 causal query tokens per sequence; the
algorithmic bytes count each cache row once per sequence, the read-once standard), D8
dense decode of the C1 batch over a paged fp8 cache, X4 the fp8 top-k indexer in front of C4.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C1]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode GB/s (% of HBM peak) + tokens/s, B=64 H=128 ctx≤4K, 1 GPU"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
# fp8 workloads whose 128-head batches run the balanced fp8 kernel: the logits of these
# many columns per key take fp8 MFMA, the rest of the logit (bf16 rope) and the 512 value
# columns bf16 MFMA
FP8_SCORE_COLS = {"C4": 576, "D8": 576, "S2": 576, "R8": 512}


def mfma_peak(wl):
    """Dense MFMA peak (TFLOP/s) of the workload's contraction mix: bf16, or for the fp8
    workloads the time-weighted peak of fp8 scores and bf16 rope and values (576 + 512
    flop columns per key and head, each at its own dtype's peak)."""
    if wl not in FP8_SCORE_COLS:
        return BF16_PEAK_TFLOPS
    f8 = FP8_SCORE_COLS[wl]
    bf = 576 - f8 + 512
    return (f8 + bf) / (f8 / FP8_PEAK_TFLOPS + bf / BF16_PEAK_TFLOPS)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_c1_traffic.txt")
CSRC = os.path.join(ROOT, "mla_decode_paged_02_amd", "csrc")

DESCRIPTIONS = {
    "C0": "C0: B=2 H=16 lens {37,100} PS=16, 1 query token per sequence, head 576 / V 512, causal, bf16",
    "C1": "C1: B=64 H=128 lens U[1024,4096] PS=64, 1 query token per sequence, head 576 / V 512, causal, bf16",
    "C2": "C2: B=8 H=128 lens {32768x4,65536x4} PS=64, 1 query token per sequence, head 576 / V 512, causal, bf16",
    "C3": "C3: ragged causal prefill, new {512,1024,2048,3968} after {0,256,0,1024}, H=128, q 192 / v 128, bf16",
    "C4": "C4: sparse decode, B=32 H=128, 16384 rows/seq PS=64, top-k U[1024,2048] of 2048 indices, fp8 e4m3 q and cache",
    "M2": "M2: multi-token decode, the C1 batch (B=64 H=128 lens U[1024,4096] PS=64) with 2 query tokens per sequence, causal within the new tokens, bf16",
    "M4": "M4: multi-token decode, the C1 batch (B=64 H=128 lens U[1024,4096] PS=64) with 4 query tokens per sequence, causal within the new tokens, bf16",
    "D8": "D8: dense decode over a paged fp8 e4m3 cache, the C1 batch (B=64 H=128 lens U[1024,4096] PS=64), one float32 scale per cache row and per q token",
    "R8": "R8: dense decode in the rope-aware layout (640-byte rows: 512 e4m3 latent codes + 64 bf16 rope values, one float32 scale per cache row and q token on the codes), the C1 batch (B=64 H=128 lens U[1024,4096] PS=64)",
    "S2": "S2: sparse decode with shared lists, the C4 batch (B=32 H=128, 16384 rows/seq PS=64, top-k U[1024,2048] of 2048 indices, fp8 e4m3) with 2 query tokens per sequence sharing its list",
    "X4": "X4: fp8 top-k indexer in front of C4, 32 sequences x 16384 cache rows PS=64, 1 query token each, 64 heads of width 128, top 2048, causal",
}
# multi-token workloads: (configuration they extend, query tokens per sequence)
MULTI_TOKEN = {"M2": (1, 2), "M4": (1, 4)}
KERNELS = {"C0": "mla_decode_kernel", "C1": "mla_decode2_kernel", "C2": "mla_decode2_kernel",
           "C3": "mla_prefill_kernel", "C4": "mla_fp8mma_kernel", "M2": "mla_decode_kernel",
           "M4": "mla_decode_kernel", "D8": "mla_fp8mma_kernel", "R8": "mla_fp8mma_kernel", "S2": "mla_fp8mma_kernel",
           "X4": "mla_indexer_score_kernel + mla_indexer_select_kernel"}


# sources the dense decode and combine kernels are built from
DECODE_SOURCES = ("mla_decode.hip", "mla_decode2.hip", "mla_device.h", "mla_kernels.h", "mla_plan.h", "mla_rows.h",
                  "mla_stage.h")


def kernel_digest():
    """Digest of the dense decode kernel's sources (the traffic summary is only used for the
    same code)."""
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload):
    """HBM bytes per launch of the decode kernel from the committed counter summary, if it
    was taken on the current kernel sources and this workload; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_digest") != kernel_digest() or vals.get("workload") != workload:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def hbm_read_ceiling(dev, gib=2, reps=20):
    """Context, not a roofline peak: the read bandwidth of a plain device reduction
    (row sums of a 2 GiB float32 tensor viewed as 16384 rows, every byte read once; the
    fastest of the torch reductions tried on MI355X, ~6.2 TB/s), best of `reps` timed
    passes, in GB/s."""
    import torch
    x = torch.ones((gib << 30) // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps + 2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        x.view(16384, -1).sum(dim=1)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    nbytes = x.numel() * 4
    del x
    torch.cuda.empty_cache()
    return round(nbytes / (best * 1e-3) / 1e9, 1)


def pct(values, q):
    """q-th percentile (linear interpolation) of a list of numbers."""
    v = sorted(values)
    if not v:
        return float("nan")
    x = (len(v) - 1) * q / 100.0
    lo = int(x)
    hi = min(lo + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (x - lo)


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([int(p.get("num_threads", 1)) for p in threadpool_info()
                    if p.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001 - report the affinity size if the BLAS is not visible
        return len(os.sched_getaffinity(0))


def cpu_baseline(case, alg_bytes, budget_s=12.0):
    """Time the float64 oracle (as it stands) on this host: whole passes over the dense
    decode workload until about `budget_s` seconds are spent (at least one pass)."""
    import oracle.mla_oracle as O
    passes, spent = 0, 0.0
    while passes == 0 or (spent < budget_s and passes < 50):
        t0 = time.perf_counter()
        O.decode_paged(case.q, case.input_row_offsets, case.page_table, case.cache_lens,
                       case.latent_cache, case.page_size, case.scale, case.mask, case.window)
        spent += time.perf_counter() - t0
        passes += 1
    return {"value": round(alg_bytes * passes / spent / 1e9, 4), "unit": "GB/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"{passes} full pass(es) of the {case.name} workload "
                      f"({case.total_q} query rows), {spent:.1f} s"}


def setup(workload, copies, num_partitions, dev):
    """Device inputs (rotated copies) and a step function for one workload."""
    import numpy as np
    import torch

    import mla_decode_paged_02_amd as m
    from synth import config_case

    if workload in MULTI_TOKEN:
        k, n_tok = MULTI_TOKEN[workload]
        case = config_case(k, q_per_seq=n_tok)
    elif workload == "D8":
        case = config_case(1, fp8=True)
    elif workload == "R8":
        from synth import rope_aware
        case = rope_aware(config_case(1, fp8=True), 355008)
    elif workload == "X4":
        from synth import indexer_config
        case = indexer_config()
    elif workload == "S2":
        from synth import make_shared_sparse_case
        case = make_shared_sparse_case(355004, [2] * 32, 128, 16384, 64, (1024, 2048), 2048, name="S2")
    else:
        case = config_case(int(workload[1]))

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(x):
        return torch.from_numpy(np.ascontiguousarray(x).astype(np.int32)).to(dev)

    def u8(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(dev)

    def f32(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)

    n = max(1, copies)
    if workload in ("C0", "C1", "C2") or workload in MULTI_TOKEN:
        q0, c0 = bf16(case.q), bf16(case.latent_cache)
        sets = [(q0, c0)] + [(q0.clone(), c0.clone()) for _ in range(n - 1)]
        off, pt, lens = i32(case.input_row_offsets), i32(case.page_table), i32(case.cache_lens)
        out = torch.empty((case.total_q, case.num_heads, 512), dtype=torch.bfloat16, device=dev)

        def step(i):
            q, c = sets[i % len(sets)]
            m.decode_paged(q, off, pt, lens, c, case.scale, mask=case.mask,
                           local_window_size=case.window, num_partitions=num_partitions, out=out)
        return case, step, case.total_q
    if workload == "X4":
        q0, k0 = u8(case.q8), u8(case.k8)
        sets = [(q0, k0)] + [(q0.clone(), k0.clone()) for _ in range(n - 1)]
        qs, ks = f32(case.q_s), f32(case.k_scale)
        off, pt, lens = i32(case.input_row_offsets), i32(case.page_table), i32(case.cache_lens)
        out = torch.empty((case.total_q, case.top_k), dtype=torch.int32, device=dev)

        def step(i):
            q, k = sets[i % len(sets)]
            m.indexer_paged_fp8(q, qs, off, pt, lens, k, ks, case.top_k, mask=case.mask, out=out)
        return case, step, case.total_q
    if workload in ("D8", "R8"):
        q0, c0 = u8(case.q8), u8(case.cache8)
        sets = [(q0, c0)] + [(q0.clone(), c0.clone()) for _ in range(n - 1)]
        qs, cs = f32(case.q_scale), f32(case.cache_scale)
        off, pt, lens = i32(case.input_row_offsets), i32(case.page_table), i32(case.cache_lens)
        out = torch.empty((case.total_q, case.num_heads, 512), dtype=torch.bfloat16, device=dev)

        def step(i):
            q, c = sets[i % len(sets)]
            m.decode_paged_fp8(q, qs, off, pt, lens, c, cs, case.scale, mask=case.mask,
                               num_partitions=num_partitions, out=out)
        return case, step, case.total_q
    if workload == "C4":
        q0, c0 = u8(case.q8), u8(case.cache8)
        sets = [(q0, c0)] + [(q0.clone(), c0.clone()) for _ in range(n - 1)]
        qs, cs = f32(case.q_scale), f32(case.cache_scale)
        off, idx, topk = i32(case.input_row_offsets), i32(case.d_indices), i32(case.topk_lengths)
        out = torch.empty((case.total_q, case.q8.shape[1], 512), dtype=torch.bfloat16, device=dev)

        def step(i):
            q, c = sets[i % len(sets)]
            m.decode_paged_sparse(q, qs, off, c, cs, idx, topk, case.scale,
                                  num_partitions=num_partitions, out=out)
        return case, step, case.total_q
    if workload == "S2":
        q0, c0 = u8(case.q8), u8(case.cache8)
        sets = [(q0, c0)] + [(q0.clone(), c0.clone()) for _ in range(n - 1)]
        qs, cs = f32(case.q_scale), f32(case.cache_scale)
        off, idx, topk = i32(case.input_row_offsets), i32(case.d_indices), i32(case.topk_lengths)
        out = torch.empty((case.total_q, case.q8.shape[1], 512), dtype=torch.bfloat16, device=dev)

        def step(i):
            q, c = sets[i % len(sets)]
            m.decode_paged_sparse_shared(q, qs, off, c, cs, idx, topk, case.scale,
                                         num_partitions=num_partitions, out=out)
        return case, step, case.total_q
    if workload == "C3":
        q0, k0, v0 = bf16(case.q), bf16(case.k), bf16(case.v)
        sets = [(q0, k0, v0)] + [(q0.clone(), k0.clone(), v0.clone()) for _ in range(min(n, 2) - 1)]
        bro, co, off = i32(case.buffer_row_offsets), i32(case.cache_offsets), i32(case.input_row_offsets)
        pt, lens, cache = i32(case.page_table), i32(case.cache_lens), bf16(case.latent_cache)
        out = torch.empty((case.q.shape[0], case.q.shape[1], 128), dtype=torch.bfloat16, device=dev)

        def step(i):
            q, k, v = sets[i % len(sets)]
            m.prefill_paged(q, k, v, bro, co, off, pt, lens, cache, case.scale, mask=case.mask, out=out)
        return case, step, int(case.q.shape[0])
    raise SystemExit(f"unknown workload {workload}")


def graph_workspace_bytes(m, wl, case, num_partitions):
    """Workspace a captured step needs: reserved on the capture stream before capturing."""
    if wl == "X4":
        return m.indexer_workspace_bytes(case.total_q, case.page_table.shape[1], case.page_size)
    if wl == "C3":
        return 1 << 20
    heads = case.num_heads if hasattr(case, "num_heads") else int(case.q8.shape[1])
    return m.decode_workspace_bytes(case.total_q, heads, num_partitions)


def graph_step_ms(m, torch, step, copies, warmup, steps, ws_bytes):
    """The same steps replayed from HIP graphs, one per rotated input copy, captured on a
    side stream whose workspace is reserved first; milliseconds per replayed step."""
    s = torch.cuda.Stream()
    m.reserve_workspace(ws_bytes, stream=s)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(copies):
            step(i)
    torch.cuda.synchronize()
    graphs = []
    for i in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % copies].replay()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(steps):
        graphs[i % copies].replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4, help="rotated input copies")
    ap.add_argument("--workload", default="C1", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--num-partitions", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the graph-replay context figure")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to calibrate HBM byte counters)")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_launch": n,
                          "copy_calibration_bytes_written_per_launch": n, "launches": 3}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "this decode path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch

    import mla_decode_paged_02_amd as m
    from synth import algorithmic_bytes, algorithmic_flops

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = args.workload
    case, step, tokens = setup(wl, args.copies, args.num_partitions, dev)
    alg_bytes = algorithmic_bytes(case)
    alg_flops = algorithmic_flops(case)
    prefill = wl == "C3"

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps, synchronised on both sides; an event
    # between consecutive steps gives each step's own duration as well
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3
    ms_step = evs[0].elapsed_time(evs[-1]) / args.steps
    step_each = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]

    # ---- warm-cache figure (same buffers every step), for context only
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step(0)
    ev1.record()
    torch.cuda.synchronize()
    warm_ms = ev0.elapsed_time(ev1) / args.steps

    # ---- the main kernel alone: the library brackets each launch with a pair of HIP
    # events (created once, before these steps) on the launch stream; at least 50 calls
    kernel_calls = max(args.steps, 50)
    m.profile_enable(True)
    for i in range(kernel_calls):
        step(i)
    torch.cuda.synchronize()
    k_each = m.profile_read_each()
    m.profile_enable(False)
    launches = len(k_each)
    k_avg_ms = pct(k_each, 50)
    step_ms_median = pct(step_each, 50)
    if k_avg_ms > step_ms_median:
        print(f"warning: median kernel time {k_avg_ms * 1e3:.2f} us exceeds the median step time "
              f"{step_ms_median * 1e3:.2f} us", file=sys.stderr)

    # ---- context: the same steps replayed from HIP graphs (no host work per step)
    graph_ms = None
    if not args.no_graph:
        graph_ms = graph_step_ms(m, torch, step, max(1, args.copies), args.warmup, args.steps,
                                 graph_workspace_bytes(m, wl, case, args.num_partitions))

    gbs = alg_bytes / (ms_step * 1e-3) / 1e9
    tflops = alg_flops / (ms_step * 1e-3) / 1e12
    # the roofline that bounds the kernel: MFMA (bf16, or the fp8 / bf16 mix) when its
    # arithmetic intensity is past the ridge (peak FLOP/s over peak bytes/s), else HBM
    peak_mfma = mfma_peak(wl)
    mfma_bound = alg_flops / alg_bytes > peak_mfma * 1e12 / (HBM_PEAK_GBS * 1e9)
    if mfma_bound and not prefill:
        achieved = alg_flops / (k_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak_mfma, 1), "unit": "TFLOP/s",
                "frac": round(achieved / peak_mfma, 4), "traffic": None,
                "hbm_achieved_gbs": round(alg_bytes / (k_avg_ms * 1e-3) / 1e9, 2)}
        if wl in FP8_SCORE_COLS:
            roof["peak_mix"] = f"fp8 scores over {FP8_SCORE_COLS[wl]} columns, bf16 for the rest and the values"
        metric = METRIC if wl == "C1" else f"MLA {'sparse ' if wl in ('C4', 'S2') else 'fp8 ' if wl == 'D8' else 'fp8 rope-aware ' if wl == 'R8' else ''}decode GB/s, {wl}, 1 GPU"
        if wl == "X4":
            metric = "MLA fp8 top-k indexer GB/s (cache rows once per token), X4, 1 GPU"
        if wl in MULTI_TOKEN:
            metric = f"MLA multi-token decode GB/s (cache rows once per sequence), {wl}, 1 GPU"
        value, unit = gbs, "GB/s"
    elif prefill:
        achieved = alg_flops / (k_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None}
        metric, value, unit = "MLA prefill TFLOP/s (causal pairs x 2H(192+128)), 1 GPU", tflops, "TFLOP/s"
    else:
        achieved = alg_bytes / (k_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(wl)}
        metric = METRIC if wl == "C1" else f"MLA {'sparse ' if wl in ('C4', 'S2') else 'fp8 ' if wl == 'D8' else 'fp8 rope-aware ' if wl == 'R8' else ''}decode GB/s, {wl}, 1 GPU"
        if wl == "X4":
            metric = "MLA fp8 top-k indexer GB/s (cache rows once per token), X4, 1 GPU"
        if wl in MULTI_TOKEN:
            metric = f"MLA multi-token decode GB/s (cache rows once per sequence), {wl}, 1 GPU"
        value, unit = gbs, "GB/s"
    roof.update({"kernel": KERNELS[wl],
                 "kernel_us": {"median": round(k_avg_ms * 1e3, 3), "p10": round(pct(k_each, 10) * 1e3, 3),
                               "p90": round(pct(k_each, 90) * 1e3, 3), "mean": round(sum(k_each) / max(1, launches) * 1e3, 3)},
                 "kernel_launches_timed": launches,
                 "kernel_median_le_step_median": bool(k_avg_ms <= step_ms_median)})
    res = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "step_us": {"median": round(step_ms_median * 1e3, 3), "p10": round(pct(step_each, 10) * 1e3, 3),
                    "p90": round(pct(step_each, 90) * 1e3, 3)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 in, bf16 MFMA" if wl in ("C4", "D8", "S2") else "fp8-e4m3 + bf16 rope in, bf16 MFMA" if wl == "R8" else "fp8-e4m3 in, f32 scores" if wl == "X4" else "bf16",
        "data": "synthetic",
        "config": {
            "workload": DESCRIPTIONS[wl],
            "num_partitions": args.num_partitions if args.num_partitions > 0 else "library",
            "rotated_input_copies": args.copies,
            "seed": 355000 + (MULTI_TOKEN[wl][0] if wl in MULTI_TOKEN else 1 if wl in ("D8", "R8") else 5 if wl == "X4" else 4 if wl == "S2" else int(wl[1])),
        },
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        "algorithmic_bytes_per_step": int(alg_bytes),
        "algorithmic_flops_per_step": int(alg_flops),
        "tflops": round(tflops, 2),
        "warm_cache_value": round((alg_flops / 1e12 if prefill else alg_bytes / 1e9) / (warm_ms * 1e-3), 2),
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "graph_value": None if graph_ms is None else
        round((alg_flops / 1e12 if prefill else alg_bytes / 1e9) / (graph_ms * 1e-3), 2),
        "wall_ms_timed_region": round(wall_ms, 3),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not prefill:
        ceiling = hbm_read_ceiling(dev)
        res["hbm_read_ceiling_gbs"] = ceiling
        res["kernel_frac_of_read_ceiling"] = round(alg_bytes / (k_avg_ms * 1e-3) / 1e9 / ceiling, 4)
    if wl == "C1" and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case, alg_bytes)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
