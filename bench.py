#!/usr/bin/env python3
"""Benchmark of the quantized-matmul hot path on one MI355X.

Headline (`value`): the decode GEMV, 4-bit codes in groups of 64, W [4096, 4096] (uint32
[4096, 512] plus bf16 scales and biases [4096, 64]), bf16 x [1, 4096] -> bf16 y [1, 4096], as
effective GB/s of algorithmic bytes
    B = N*K*bits/8 + 4*N*K/G + M*K*2 + M*N*2 = 9,453,568 bytes per step,
against the 8 TB/s HBM peak. One step is one qmm call; consecutive steps use different copies of
the weights (about 1 GiB of copies, four times the 256 MB Infinity Cache), so every step reads its
weights from HBM. The K timed steps are one captured HIP graph (no Python between launches),
bracketed by synchronizations and timed with events on the stream the kernels run on.

Also measured, in the same JSON line: the prefill GEMM (4-bit g128, x bf16 [2048, 14336],
W [4096, 14336]) in TFLOP/s against the 2.5 PFLOP/s dense bf16 MFMA peak, and the CPU oracle on
the host cores (`cpu_baseline`).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-prefill]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
METRIC = "qmm effective weight GB/s (GEMV, % HBM peak); TFLOP/s (GEMM, % MFMA peak)"
ROTATE_BYTES = 1 << 30


def algorithmic_bytes(m, n, k, bits, group, xsize=2, ysize=2):
    return n * k * bits // 8 + 4 * n * k // group + m * k * xsize + m * n * ysize


def source_hash(*names):
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "quantized_matmul_mlx_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_key, sources):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when the
    kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(*sources):
        return None
    return rec.get("hbm_bytes_per_launch")


def device_inputs(torch, inp, copies):
    import numpy as np
    packed = torch.from_numpy(inp.packed.view(np.int32)).cuda()
    scales = torch.from_numpy(inp.scales.view(np.int16)).cuda().view(torch.bfloat16)
    biases = torch.from_numpy(inp.biases.view(np.int16)).cuda().view(torch.bfloat16)
    x = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
    sets = []
    for _ in range(copies):
        sets.append((x.clone(), packed.clone(), scales.clone(), biases.clone()))
    return sets


def time_graph(torch, q, sets, ys, group, bits, steps, warmup):
    """Runs `warmup` eager steps, then captures `steps` steps in one graph and times one replay."""
    nsets = len(sets)

    def step(i):
        x, p, s, b = sets[i % nsets]
        q.qmm(x, p, s, b, group, bits, out=ys[i % nsets])

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                step(i)
    torch.cuda.current_stream().wait_stream(side)
    g.replay()                      # untimed: first replay pays one-time graph upload costs
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps          # ms per step


def cpu_baseline_decode(inp, budget_s=10.0, max_runs=50):
    import oracle
    threads = oracle.default_threads()
    wl = inp.wl
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.qmm(inp.x, "bf16", inp.packed, inp.scales, inp.biases, wl.group_size, wl.bits,
                   threads=threads)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= max_runs:
            break
    b = algorithmic_bytes(inp.x.shape[0], wl.n, wl.k, wl.bits, wl.group_size)
    return {"value": round(b * runs / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"the full decode step (M=1, W 4096x4096 4-bit g64) run {runs} times in "
                      f"{el:.1f} s on {threads} host threads"}


def cpu_baseline_prefill(inp, rows):
    import oracle
    threads = oracle.default_threads()
    wl = inp.wl
    t0 = time.perf_counter()
    oracle.qmm(inp.x[:rows], "bf16", inp.packed, inp.scales, inp.biases, wl.group_size, wl.bits,
               threads=threads)
    el = time.perf_counter() - t0
    flop = 2.0 * rows * wl.n * wl.k
    return {"value": round(flop / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "sample": f"{rows} of the 2048 x rows against all of W, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the quantized matmul here runs on a single GPU's share and no multi-GPU figure is "
              "produced.", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_matmul_mlx_amd as q
    from quantized_matmul_mlx_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    q._lib.load()

    # ---- decode GEMV (headline) ----
    wl = W.WORKLOADS["decode_4bit_g64_4096x4096"]
    m = 1
    inp = W.make_inputs(wl, m=m)
    b_step = algorithmic_bytes(m, wl.n, wl.k, wl.bits, wl.group_size)
    copies = max(1, -(-ROTATE_BYTES // b_step))
    print(f"[bench] decode GEMV: {copies} weight copies, warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)
    sets = device_inputs(torch, inp, copies)
    ys = [torch.empty((m, wl.n), dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
    ms = time_graph(torch, q, sets, ys, wl.group_size, wl.bits, args.steps, args.warmup)
    gbs = b_step / (ms * 1e-3) / 1e9
    del sets, ys
    torch.cuda.empty_cache()

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "decode GEMV: 4-bit codes, group 64, W [4096, 4096] (uint32 [4096, 512]), "
                        "x bf16 [1, 4096] ~N(0,1), y bf16 [1, 4096]; seed 0",
            "m": m, "n": wl.n, "k": wl.k, "bits": wl.bits, "group_size": wl.group_size,
            "algorithmic_bytes_per_step": b_step,
            "weight_copies": copies,
            "timing": "one HIP graph of K qmm launches, events on the launch stream",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": read_traffic("gemv_4bit_g64_4096x4096_m1", ["gemv.hip", "qaff_device.h"]),
        },
    }

    # ---- prefill GEMM (second target) ----
    if not args.no_prefill:
        pwl = W.WORKLOADS["prefill_4bit_g128_4096x14336"]
        pm = 2048
        pinp = W.make_inputs(pwl, m=pm)
        pcopies = 4
        print(f"[bench] prefill GEMM: {pcopies} copies, steps {args.prefill_steps}", file=sys.stderr, flush=True)
        psets = device_inputs(torch, pinp, pcopies)
        pys = [torch.empty((pm, pwl.n), dtype=torch.bfloat16, device="cuda") for _ in range(pcopies)]
        pms = time_graph(torch, q, psets, pys, pwl.group_size, pwl.bits, args.prefill_steps, 3)
        flop = 2.0 * pm * pwl.n * pwl.k
        tflops = flop / (pms * 1e-3) / 1e12
        result["prefill_gemm"] = {
            "workload": "prefill GEMM: 4-bit codes, group 128, W [4096, 14336], x bf16 [2048, 14336], "
                        "y bf16 [2048, 4096]; seed 0",
            "ms_per_step": round(pms, 5),
            "tflops": round(tflops, 2),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                         "traffic": read_traffic("gemm_4bit_g128_prefill", ["gemm.hip", "qaff_device.h"])},
        }
        del psets, pys
        torch.cuda.empty_cache()
    else:
        pinp = None

    # ---- CPU oracle on the host cores ----
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline_decode(inp)
        if pinp is not None:
            result["prefill_gemm"]["cpu_baseline"] = cpu_baseline_prefill(pinp, rows=8)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
