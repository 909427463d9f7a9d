#!/usr/bin/env python3
"""Benchmark of the W4A16 fused MoE layer on one MI355X.

One step = one pass of the whole layer over one batch of synthetic input: one
call of w4a16_moe_routed_forward, i.e. the alignment, gate_up + SiLU-and-mul,
down and the top-k combine (with per-expert tile sizes on skewed prefill).
Inputs and repacked weights are resident in HBM before timing starts; weight
repack is load time and is not timed. A staged replica of the same path gives
the per-kernel breakdown.

Timing follows the pages' kernel-benchmark method (Humming announcement,
"Humming: vLLM과 Ant Group, 양자화 추론을 위한 범용 커널 라이브러리 오픈소스 공개",
section "결과: 커널 마이크로벤치마크": warmed up, cold L2, each sample timed on
its own): before every timed step a 1 GiB buffer is *read* (a sum), outside
the timed interval, which pushes the layer's data out of L2 and the 256 MB
Infinity Cache and leaves them clean. (A write-based flush would leave up to
256 MB of dirty lines whose write-back then lands inside the timed kernel and
halves its read bandwidth.) Each step is timed with HIP events on the stream
the kernels run on, with events between the stages for the per-kernel
breakdown.

Prints one JSON line. --gpus above 1 is refused: the layer here is one GPU's share and runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
DEFAULT_WORKLOAD = "decode_ep48"


# the sources of the GEMM kernels and of the packed weight layout they read: the
# stored HBM byte counts stay valid while these are unchanged
GEMM_SOURCES = ("internal.h", "moe_gemm.hip", "moe_gemm_stream.hip", "moe_gemm_tiled.hip", "repack.hip")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4a16_grouped_gemm_amd", "csrc")
    for f in GEMM_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def algorithmic_work(c):
    """Bytes the method must move and flops it must do (padding and the h / y
    round trips through HBM excluded)."""
    ids = c.topk_ids
    local = (ids >= 0) & (ids < c.E)
    S = int(local.sum())
    U = int(local.any(axis=1).sum())
    active = int(np.unique(ids[local]).size)
    H, I = c.H, c.I
    w13 = H * 2 * I // 2 + (H // 32) * 2 * I * 2   # nibbles + bf16 scales per expert
    w2 = I * H // 2 + (I // 32) * H * 2
    gate_up_bytes = active * w13 + U * H * 2
    down_bytes = active * w2
    layer_bytes = gate_up_bytes + down_bytes + c.T * H * 2 + c.T * c.topk * 8
    return dict(S=S, U=U, active=active, w13_per_expert=w13, w2_per_expert=w2, gate_up_bytes=gate_up_bytes,
                down_bytes=down_bytes, layer_bytes=layer_bytes, gate_up_flops=2 * S * H * 2 * I,
                down_flops=2 * S * I * H, layer_flops=2 * S * (H * 2 * I + I * H))


def cpu_baseline(c, target_slots: int):
    """The oracle on a bounded sample of tokens, scaled to the whole layer by slots."""
    import oracle

    local = ((c.topk_ids >= 0) & (c.topk_ids < c.E)).sum(axis=1)
    order = np.random.default_rng(0).permutation(c.T)
    picked, slots = [], 0
    for t in order:
        if local[t] == 0:
            continue
        picked.append(int(t))
        slots += int(local[t])
        if slots >= target_slots:
            break
    tokens = np.array(sorted(picked), np.int32)
    S = int(local.sum())
    cores = oracle.num_threads()

    def timed(sample):
        t0 = time.perf_counter()
        oracle.moe_layer(c.x, c.topk_ids, c.topk_weights, c.w13_q, c.w13_s, c.w2_q, c.w2_s, E=c.E, I=c.I,
                         tokens=sample)
        return time.perf_counter() - t0

    runs = sorted(timed(tokens) for _ in range(3))
    dt = runs[1]  # median of 3
    # one core on an eighth of the sample (the same tokens' first eighth), scaled the same way
    few = tokens[:max(1, len(tokens) // 8)]
    few_slots = int(local[few].sum())
    oracle.set_num_threads(1)
    try:
        runs1 = sorted(timed(few) for _ in range(3))
    finally:
        oracle.set_num_threads(cores)
    dt1 = runs1[1]
    return {"value": round(dt / slots * S * 1e6, 1), "unit": "us", "cores": cores, "kind": "oracle",
            "sample": f"{len(tokens)} tokens / {slots} resident slots of {c.name} ({S} slots), median of 3 runs "
                      f"({', '.join(f'{r:.2f}' for r in runs)} s wall), scaled by slots to the whole layer",
            "one_core": {"value": round(dt1 / few_slots * S * 1e6, 1), "unit": "us", "cores": 1,
                         "sample": f"{len(few)} tokens / {few_slots} resident slots, median of 3 runs "
                                   f"({', '.join(f'{r:.2f}' for r in runs1)} s wall), scaled by slots to the "
                                   f"whole layer"}}


def gemm_dtype(kernel: str) -> str:
    """The MFMA operand type of a GEMM kernel: the tiled kernel multiplies exact fp16
    images of the bf16 activations and int4 * scale weights, the streaming kernels
    bf16 activations and exact bf16 integer weights; both accumulate in fp32."""
    return "fp16" if kernel == "moe_gemm_tiled_kernel" else "bf16"


def gemm_kernel_name(block_m: int, N: int, K: int) -> str:
    """The GEMM kernel the library dispatches to for this block_m and shape."""
    if block_m == 128 and N % 256 == 0 and (K // 32) % 2 == 0:
        return "moe_gemm_tiled_kernel"
    if block_m in (16, 32, 64) and N % 256 == 0 and (K // 32) % 4 == 0:
        return "moe_gemm_stream_lds_kernel"
    return "moe_gemm_stream_kernel"


def stored_traffic(workload: str, kernel: str, launches_per_step: int = 1):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def route_align_timing(w, synthetic, dev, c, bm, reps: int = 50):
    """Median µs of moe_route_align (top-k routing of fp32 logits over the global experts, then the
    alignment over the local slice) for one token and for the workload's T tokens, logits warm in L2.
    Not part of the layer step: the layer takes routed ids as input."""
    import torch

    Eg = c.meta.get("E_global", c.E)
    lg = dev(synthetic.router_logits(c.T, Eg, 7))
    ids = torch.empty((c.T, c.topk), dtype=torch.int32, device="cuda")
    wts = torch.empty((c.T, c.topk), dtype=torch.float32, device="cuda")
    buf = w.align_buffers(c.T, c.topk, c.E, bm)
    out = {}
    for n in sorted({1, c.T}):
        def call():
            w.moe_route_align(lg[:n], c.topk, c.E, bm, ids[:n], wts[:n], buf["sorted_token_ids"], buf["expert_ids"],
                              buf["num_tokens_post_padded"], workspace=buf["workspace"])
        for _ in range(5):
            call()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for i in range(reps):
            # a spin kernel keeps the GPU busy while the host queues the call, so the
            # events bracket GPU time and not the host's launch latency
            torch.cuda._sleep(200000)
            ev[2 * i].record()
            call()
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        out[f"T{n}"] = round(float(np.median([ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(reps)])), 2)
    out["experts_routed"] = Eg
    return out


def bench_grouped(args, layout: str):
    """The layer on an expert-grouped layout over the 48-expert Kimi-K2 slice (H 7168, I 2048):
    contiguous: the prefill_contig48 batch permuted into 48 x 128 rows (no padding);
    masked: a 32-row budget per expert, all 32 rows live (the grouped decode case of
    32 tokens per expert). One step = one entry-point call, cold caches."""
    import torch

    import synthetic
    import w4a16_grouped_gemm_amd as w

    c = synthetic.workload("prefill_contig48")
    E, H, I = c.E, c.H, c.I
    shape = w.make_shape(E, H, I)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).cuda()

    n13, n2 = w.w4a16_packed_bytes(shape)
    w13p = torch.empty(n13, dtype=torch.uint8, device="cuda")
    w2p = torch.empty(n2, dtype=torch.uint8, device="cuda")
    w.w4a16_repack(shape, dev(c.w13_q), dev(c.w13_s), dev(c.w2_q), dev(c.w2_s), w13p, w2p)
    torch.cuda.synchronize()
    if layout == "contiguous":
        slots = np.argsort(c.topk_ids.reshape(-1), kind="stable")
        m = c.topk_ids.reshape(-1)[slots].astype(np.int32)
        x = dev(c.x[slots // c.topk])
        M = len(m)
        mi = dev(m)
        ws = torch.empty(w.w4a16_moe_contiguous_workspace_bytes(shape, M), dtype=torch.uint8, device="cuda")
        out = torch.empty((M, H), dtype=torch.int16, device="cuda")
        bm, rows, name = 128, M, f"grouped_contiguous{E} ({E} experts x {M // E} rows, H {H}, I {I})"

        def step():
            w.w4a16_moe_contiguous_forward(shape, x, mi, w13p, w2p, out, ws)
    else:
        max_m = 32
        x = dev(synthetic.make_x(E * max_m, H, seed=41).reshape(E, max_m, H))
        mm = dev(np.full(E, max_m, np.int32))
        bm = w.w4a16_moe_masked_block_m(max_m, max_m)
        ws = torch.empty(w.w4a16_moe_masked_workspace_bytes(shape, max_m, bm), dtype=torch.uint8, device="cuda")
        out = torch.empty((E, max_m, H), dtype=torch.int16, device="cuda")
        rows, name = E * max_m, f"grouped_masked{E} ({E} experts x {max_m} live rows, H {H}, I {I})"

        def step():
            w.w4a16_moe_masked_forward(shape, x, mm, bm, w13p, w2p, out, ws)

    flush_buf = torch.ones(1 << 27, dtype=torch.int64, device="cuda")
    for _ in range(args.warmup):
        flush_buf.sum()
        step()
    torch.cuda.synchronize()
    evs = []
    for _ in range(args.steps):
        flush_buf.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    med = float(np.median(us))
    w13 = H * 2 * I // 2 + (H // 32) * 2 * I * 2
    w2 = I * H // 2 + (I // 32) * H * 2
    layer_bytes = E * (w13 + w2) + rows * H * 2 * 2
    layer_flops = 2 * rows * (H * 2 * I + I * H)
    gbps, tflops = layer_bytes / (med * 1e-6) / 1e9, layer_flops / (med * 1e-6) / 1e12
    print(json.dumps({
        "metric": f"W4A16 MoE layer µs, {layout} grouped layout", "value": round(med, 2), "unit": "us",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(med / 1e3, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": gemm_dtype(gemm_kernel_name(bm, 2 * I, H)), "data": "synthetic",
        "config": {"workload": name, "rows": rows, "block_m": bm, "cache": "cold (1 GiB read before each step)"},
        "layer_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "layer_TFLOPs": round(tflops, 2),
        "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4), "alg_bytes": layer_bytes, "alg_flops": layer_flops,
        "layer_us_p10_p90": [round(float(np.percentile(us, 10)), 2), round(float(np.percentile(us, 90)), 2)],
    }), flush=True)


def bench_sweep(args):
    """Tokens-per-expert sweep on the 48-expert Kimi-K2 slice (H 7168, I 2048; the decode workload's
    weights): for T = 1, 2, 4, ..., 8192 tokens routed top-8 over 384 experts from N(0,1) logits
    (experts 0-47 resident), the layer timed at every block_m through moe_align + w4a16_moe_forward,
    and the one-call routed layer with its own choice. The pages measure kernels at every power of two
    of M from 1 to 8192 tokens (Humming announcement, "결과: 커널 마이크로벤치마크") and pick the tile by
    routed tokens per expert (Chord page, "인덱스 커널 기법"). One JSON line per T."""
    import torch

    import synthetic
    import w4a16_grouped_gemm_amd as w

    E, H, I, topk, Eg = 48, synthetic.KIMI_H, synthetic.KIMI_I, synthetic.KIMI_TOPK, synthetic.KIMI_E
    shape = w.make_shape(E, H, I)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).cuda()

    print("[bench] sweep: building the 48-expert slice", file=sys.stderr, flush=True)
    w13_q, w13_s, w2_q, w2_s = synthetic.make_weights(E, H, I, 202)
    n13, n2 = w.w4a16_packed_bytes(shape)
    w13p = torch.empty(n13, dtype=torch.uint8, device="cuda")
    w2p = torch.empty(n2, dtype=torch.uint8, device="cuda")
    w.w4a16_repack(shape, dev(w13_q), dev(w13_s), dev(w2_q), dev(w2_s), w13p, w2p)
    torch.cuda.synchronize()
    del w13_q, w13_s, w2_q, w2_s
    flush_buf = torch.ones(1 << 27, dtype=torch.int64, device="cuda")
    mk = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    def timeit(step, steps):
        for _ in range(3):
            flush_buf.sum()
            step()
        torch.cuda.synchronize()
        evs = []
        for _ in range(steps):
            flush_buf.sum()
            a, b = mk()
            a.record()
            step()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))

    # clock settling before the first point
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.settle_ms / 1e3:
        flush_buf.sum()
        torch.cuda.synchronize()
    rows = []
    for lt in range(14):
        T = 1 << lt
        c = synthetic.random_case(f"sweep_T{T}", T=T, H=H, I=I, E=E, topk=topk, block_m=16, seed=500 + lt,
                                  E_global=Eg, weights=False)
        c.x = synthetic.make_x(T, H, 600 + lt)
        work = algorithmic_work(c)
        x, ids, wts = dev(c.x), dev(c.topk_ids.astype(np.int32)), dev(c.topk_weights.astype(np.float32))
        out = torch.empty((T, H), dtype=torch.int16, device="cuda")
        pt = {"T": T, "tok_e": round(T * topk / Eg, 3), "resident_slots": work["S"], "active_experts": work["active"]}
        us = {}
        for bm in (16, 32, 64, 128):
            buf = w.align_buffers(T, topk, E, bm)
            ws = torch.empty(w.w4a16_moe_workspace_bytes(shape, T, topk, bm), dtype=torch.uint8, device="cuda")

            def step(bm=bm, buf=buf, ws=ws):
                w.moe_align(ids, E, bm, buf["sorted_token_ids"], buf["expert_ids"], buf["num_tokens_post_padded"],
                            None, buf["workspace"])
                w.w4a16_moe_forward(shape, x, ids, wts, buf["sorted_token_ids"], buf["expert_ids"],
                                    buf["num_tokens_post_padded"], bm, w13p, w2p, out, ws)
            us[bm] = round(timeit(step, args.steps), 2)
            del ws, buf
        wsr = torch.empty(w.w4a16_moe_routed_workspace_bytes(shape, T, topk, Eg), dtype=torch.uint8, device="cuda")
        routed_us = round(timeit(lambda: w.w4a16_moe_routed_forward(shape, x, ids, wts, Eg, w13p, w2p, out, wsr),
                                 args.steps), 2)
        del wsr
        best = min(us, key=us.get)
        t_hbm = work["layer_bytes"] / (HBM_PEAK_GBPS * 1e9) * 1e6
        t_mfma = work["layer_flops"] / (BF16_PEAK_TFLOPS * 1e12) * 1e6
        pt.update({"layer_us_by_block_m": {str(k): v for k, v in us.items()}, "best_block_m": best,
                   "chosen_block_m": w.w4a16_choose_block_m(T, topk, E, Eg),
                   "routed_split": w.w4a16_moe_routed_split(shape, T, topk, Eg), "routed_us": routed_us,
                   "binding": "hbm" if t_hbm >= t_mfma else "mfma",
                   "routed_roofline_frac": round(max(t_hbm, t_mfma) / routed_us, 4),
                   "best_roofline_frac": round(max(t_hbm, t_mfma) / us[best], 4)})
        rows.append(pt)
        print(json.dumps(pt), flush=True)
    return rows


# Workloads the default run also times, after the headline one, each in this process with its own
# warm-up: the intermediate slice (HBM-bound) and the two prefill layers (MFMA-bound).
EXTRA_WORKLOADS = ("islice_tp8", "prefill_contig48", "prefill_skew48")


def bench_routed(args, workload: str, steps: int, warmup: int, settle_ms: float, with_cpu: bool,
                 with_router: bool, with_traffic: bool = True):
    """Time one routed workload: one call of the layer per step (alignment included), then a staged
    replica for the per-kernel breakdown. Returns the result dict of the JSON line."""
    import torch

    import synthetic
    import w4a16_grouped_gemm_amd as w

    print(f"[bench] building {workload}", file=sys.stderr, flush=True)
    c = synthetic.workload(workload)
    E, H, I, T, topk = c.E, c.H, c.I, c.T, c.topk
    Eg = c.meta.get("E_global", E)
    bm = args.block_m or w.w4a16_choose_block_m(T, topk, E, Eg)
    shape = w.make_shape(E, H, I)
    # the product path is the one-call routed layer (alignment included); --block-m forces
    # one alignment at that size through w4a16_moe_forward instead
    split = 0 if args.block_m else w.w4a16_moe_routed_split(shape, T, topk, Eg)

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).cuda()

    n13, n2 = w.w4a16_packed_bytes(shape)
    w13p = torch.empty(n13, dtype=torch.uint8, device="cuda")
    w2p = torch.empty(n2, dtype=torch.uint8, device="cuda")
    q13, s13, q2, s2 = dev(c.w13_q), dev(c.w13_s), dev(c.w2_q), dev(c.w2_s)
    w.w4a16_repack(shape, q13, s13, q2, s2, w13p, w2p)
    torch.cuda.synchronize()
    del q13, s13, q2, s2
    x, ids, wts = dev(c.x), dev(c.topk_ids.astype(np.int32)), dev(c.topk_weights.astype(np.float32))
    # staged replica of the path: one alignment set, or (split) the heavy set at block_m 128
    # and the light set at 16, each with its own h rows
    sets = [(128, split, 2**31 - 1), (16, 1, split - 1)] if split else [(bm, 0, 2**31 - 1)]
    bufs = [w.align_buffers(T, topk, E, b) for b, _, _ in sets]
    if split:  # one sorted array for both sets, heavy part first (rounded to 64 ids), as in the one-call layer
        hcap = -(-bufs[0]["sorted_token_ids"].numel() // 64) * 64
        joined = torch.empty(hcap + bufs[1]["sorted_token_ids"].numel(), dtype=torch.int32, device="cuda")
        bufs[0]["sorted_token_ids"], bufs[1]["sorted_token_ids"] = joined[:hcap], joined[hcap:]
        bufs[0]["expert_ids"] = torch.empty(-(-hcap // 128), dtype=torch.int32, device="cuda")
    hs = [torch.empty((b["sorted_token_ids"].numel(), I), dtype=torch.int16, device="cuda") for b in bufs]
    y = torch.empty((T * topk, H), dtype=torch.float32, device="cuda")
    scratch = torch.empty(max(256, w.w4a16_moe_stage_workspace_bytes(shape, T, topk, sets[0][0])), dtype=torch.uint8,
                          device="cuda")
    bm = sets[0][0]
    if args.block_m:
        ws = torch.empty(w.w4a16_moe_workspace_bytes(shape, T, topk, bm), dtype=torch.uint8, device="cuda")
    else:
        ws = torch.empty(w.w4a16_moe_routed_workspace_bytes(shape, T, topk, Eg), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    flush_buf = torch.ones(1 << 27, dtype=torch.int64, device="cuda")  # 1 GiB, read to evict caches

    def flush():
        flush_buf.sum()

    def align():
        if split:
            w.moe_align_split(ids, E, split, 128, hcap, bufs[0]["expert_ids"], bufs[0]["num_tokens_post_padded"], 16,
                              bufs[1]["expert_ids"], bufs[1]["num_tokens_post_padded"], joined, bufs[0]["workspace"])
        else:
            buf = bufs[0]
            w.moe_align(ids, E, bm, buf["sorted_token_ids"], buf["expert_ids"], buf["num_tokens_post_padded"], None,
                        buf["workspace"])

    def gemm(stage, k):
        b, buf = sets[k][0], bufs[k]
        srt, eid, ntpp = buf["sorted_token_ids"], buf["expert_ids"], buf["num_tokens_post_padded"]
        if stage == "gate_up":
            w.w4a16_moe_gate_up(shape, x, T, topk, srt, eid, ntpp, b, w13p, hs[k], scratch)
        else:
            w.w4a16_moe_down(shape, T, topk, hs[k], srt, eid, ntpp, b, w2p, y, scratch)

    # stage names, in order; one event between consecutive stages
    names = ["align", "prepare_x", "gate_up"] + (["gate_up_light"] if split else []) + ["prepare_h", "down"] + \
        (["down_light"] if split else []) + ["combine"]

    def stages(ev):
        marks = iter(ev)
        next(marks).record()
        align()
        next(marks).record()
        w.w4a16_moe_prepare_x(shape, x, ids, bm, scratch)
        for k in range(len(sets)):
            next(marks).record()
            gemm("gate_up", k)
        next(marks).record()
        w.w4a16_moe_prepare_h(shape, T, topk, hs[0], bufs[0]["sorted_token_ids"], bufs[0]["num_tokens_post_padded"],
                              bm, scratch)
        for k in range(len(sets)):
            next(marks).record()
            gemm("down", k)
        next(marks).record()
        w.w4a16_moe_combine(shape, ids, wts, y, out)
        next(marks).record()

    def forward_step(ev):
        ev[0].record()
        if args.block_m:
            align()
            buf = bufs[0]
            w.w4a16_moe_forward(shape, x, ids, wts, buf["sorted_token_ids"], buf["expert_ids"],
                                buf["num_tokens_post_padded"], bm, w13p, w2p, out, ws)
        else:
            w.w4a16_moe_routed_forward(shape, x, ids, wts, Eg, w13p, w2p, out, ws)
        ev[1].record()

    mk = lambda n: [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    # correctness of the stage split: the staged sequence equals forward bit for bit
    forward_step(mk(2))
    torch.cuda.synchronize()
    ref = out.clone()
    nev = len(names) + 1
    stages(mk(nev))
    torch.cuda.synchronize()
    assert torch.equal(ref, out), "staged sequence differs from the one-call layer"

    for _ in range(warmup):
        if not args.warm:
            flush()
        forward_step(mk(2))
        stages(mk(nev))
    torch.cuda.synchronize()
    # Clock and power settling: the MFMA-bound layers run ~20% slow for ~15 ms after the GPU
    # leaves idle (kernel traces), so untimed layers keep it busy for settle_ms of wall time
    # whatever the warm-up count, synchronising every few steps so the time is GPU time.
    settle_steps, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        for _ in range(4):
            if not args.warm:
                flush()
            forward_step(mk(2))
            settle_steps += 1
        torch.cuda.synchronize()
    settled_ms = (time.perf_counter() - t_settle) * 1e3

    print(f"[bench] timing {steps} steps of {workload}", file=sys.stderr, flush=True)
    layer_ev, stage_ev = [], []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if not args.warm:
            flush()
        ev = mk(2)
        forward_step(ev)
        layer_ev.append(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(steps):
        if not args.warm:
            flush()
        ev = mk(nev)
        stages(ev)
        stage_ev.append(ev)
    torch.cuda.synchronize()

    route_us = route_align_timing(w, synthetic, dev, c, bm) if with_router else None

    layer_us = np.array([a.elapsed_time(b) * 1e3 for a, b in layer_ev])
    st = np.array([[ev[k].elapsed_time(ev[k + 1]) * 1e3 for k in range(len(names))] for ev in stage_ev])
    med = float(np.median(layer_us))
    kmed = np.median(st, axis=0)
    work = algorithmic_work(c)
    decode = work["layer_flops"] / max(1, work["layer_bytes"]) < BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    layer_gbps = work["layer_bytes"] / (med * 1e-6) / 1e9
    layer_tflops = work["layer_flops"] / (med * 1e-6) / 1e12
    kus = {n: round(float(v), 2) for n, v in zip(names, kmed)}
    # the gate_up step: one kernel, or (split) the heavy-expert tiled kernel then the light-expert stream
    gate_us = kus["gate_up"] + kus.get("gate_up_light", 0.0)
    if decode:
        achieved = work["gate_up_bytes"] / (gate_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4)}
    else:
        achieved = work["gate_up_flops"] / (gate_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    roof["kernel"] = gemm_kernel_name(bm, 2 * I, H) + " (gate_up)"
    if split:
        roof["kernel"] = (gemm_kernel_name(128, 2 * I, H) + f" (gate_up, experts with >= {split} slots) + "
                          + gemm_kernel_name(16, 2 * I, H) + " (gate_up, lighter experts)")
    roof["traffic"] = stored_traffic(workload, "gate_up") if with_traffic else None
    # the whole layer against its binding roofline: the larger of the HBM time of its algorithmic
    # bytes and the MFMA time of its algorithmic flops, over the measured layer time
    t_hbm = work["layer_bytes"] / (HBM_PEAK_GBPS * 1e9) * 1e6
    t_mfma = work["layer_flops"] / (BF16_PEAK_TFLOPS * 1e12) * 1e6
    layer_roof = {"bound": "hbm" if t_hbm >= t_mfma else "mfma", "frac": round(max(t_hbm, t_mfma) / med, 4),
                  "t_hbm_us": round(t_hbm, 1), "t_mfma_us": round(t_mfma, 1)}

    result = {
        "metric": "W4A16 MoE layer µs; decode HBM GB/s, prefill TFLOPS as % of MI355X roofline",
        "value": round(med, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(med / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (gemm_dtype(gemm_kernel_name(128, 2 * I, H)) + "+" + gemm_dtype(gemm_kernel_name(16, 2 * I, H))
                  if split else gemm_dtype(gemm_kernel_name(bm, 2 * I, H))),
        "data": "synthetic",
        "config": {"workload": c.name, "T": T, "hidden": H, "intermediate": I, "experts_local": E,
                   "experts_global": Eg, "topk": topk, "block_m": bm if not split else f"128 / 16 split at {split} slots",
                   "resident_slots": work["S"],
                   "active_experts": work["active"], "cache": "warm" if args.warm else "cold (1 GiB read before each step)"},
        "layer_GBps": round(layer_gbps, 1),
        "hbm_frac": round(layer_gbps / HBM_PEAK_GBPS, 4),
        "layer_TFLOPs": round(layer_tflops, 2),
        "mfma_frac": round(layer_tflops / BF16_PEAK_TFLOPS, 4),
        "layer_roofline": layer_roof,
        "kernels_us": kus,
        "layer_us_p10_p90": [round(float(np.percentile(layer_us, 10)), 2), round(float(np.percentile(layer_us, 90)), 2)],
        "wall_ms_per_step_incl_flush": round(wall / steps * 1e3, 4),
        "settle": {"ms": round(settled_ms, 1), "steps": settle_steps},
        "alg_bytes": work["layer_bytes"],
        "alg_flops": work["layer_flops"],
        "roofline": roof,
        "route_align_us": route_us,
    }
    if with_cpu:
        print(f"[bench] cpu baseline (oracle) on {workload}", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(c, args.cpu_slots)
    del w13p, w2p, ws, hs, y, scratch, flush_buf
    torch.cuda.empty_cache()
    return result


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed layers for at least this much wall time after the warm-up steps (clock settling)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--only", action="store_true",
                    help="time only --workload (by default the decode line also carries the other workloads)")
    ap.add_argument("--block-m", type=int, default=0, help="0: the tokens-per-expert heuristic")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-router", action="store_true", help="skip the router + alignment timing")
    ap.add_argument("--layout", default="routed", choices=["routed", "contiguous", "masked"],
                    help="routed: the layer on top-k routed ids (the default line); contiguous / masked: "
                         "the grouped-layout entry points")
    ap.add_argument("--cpu-slots", type=int, default=3000,
                    help="resident slots the CPU baseline computes (all of them when the layer has fewer)")
    ap.add_argument("--warm", action="store_true", help="skip the cache flush between steps")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one 256 MiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--sweep", action="store_true",
                    help="tokens-per-expert sweep on the 48-expert slice: T = 1 .. 8192, every block_m")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the layer here is one GPU's expert or intermediate slice "
              "and no multi-GPU path is built; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import w4a16_grouped_gemm_amd as w

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w.load()  # fail loudly if the HIP library is not built
    if args.layout != "routed":
        return bench_grouped(args, args.layout)
    if args.sweep:
        return bench_sweep(args)
    result = bench_routed(args, args.workload, args.steps, args.warmup, args.settle_ms,
                          with_cpu=not args.no_cpu_baseline, with_router=not args.no_router)
    result["targets"] = {"decode_hbm_frac": 0.70, "prefill_mfma_frac": 0.50}
    result["context"] = ("pages' per-layer speedups of NVIDIA kernels (Chord vs Humming): 1.11-1.33x on H200, "
                         "1.81-2.15x on B300; context only, not a target on this GPU")
    result["source_hash"] = kernel_source_hash()
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = 1 << 28
    if args.workload == DEFAULT_WORKLOAD and not args.only and not args.block_m:
        # the other workloads of the metric, each timed the same way in this process: their
        # medians, spreads, rooflines and per-kernel breakdowns (the line's value stays decode's)
        keep = ("value", "layer_us_p10_p90", "roofline", "layer_roofline", "hbm_frac", "mfma_frac", "kernels_us",
                "settle", "config", "dtype", "alg_bytes", "alg_flops")
        result["workloads"] = {}
        for name in EXTRA_WORKLOADS:
            r = bench_routed(args, name, args.steps, args.warmup, args.settle_ms, with_cpu=False, with_router=False)
            result["workloads"][name] = {k: r[k] for k in keep}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
