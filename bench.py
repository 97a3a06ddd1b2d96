#!/usr/bin/env python3
"""Benchmark of the quantized-matmul hot path on one MI355X.

Headline (`value`): the decode GEMV, 4-bit codes in groups of 64, W [4096, 4096] (uint32
[4096, 512] plus bf16 scales and biases [4096, 64]), bf16 x [1, 4096] -> bf16 y [1, 4096], as
effective GB/s of algorithmic bytes
    B = N*K*bits/8 + 4*N*K/G + M*K*2 + M*N*2 = 9,453,568 bytes per step,
against the 8 TB/s HBM peak. One step is one qmm call; consecutive steps use different copies of
the operands (about 1 GiB of copies, four times the 256 MB Infinity Cache), so every step reads its
weights from HBM. The K timed steps are one captured HIP graph (no Python between launches),
bracketed by synchronizations and timed with events on the stream the kernels run on.

The same JSON line carries:
  * `prefill_gemm`: the 4-bit g128 prefill GEMM (x bf16 [2048, 14336], W [4096, 14336]) in TFLOP/s
    against the 2.5 PFLOP/s dense bf16 MFMA peak: GEMMs back to back for a few seconds, with the
    graphics clock and socket power sampled meanwhile (`sustained`; the chip is power-limited and
    settles after a transient dip), and a short graph of launches (`burst`);
  * `rows`: every other kernel of the path at its workload (the prefill GEMM at a small batch,
    M = 128, where K is split through a workspace; standalone dequantization, gathered
    rows, the 8-bit and the 3-/6-bit decode products at M = 1 and at their larger M, the decode
    product at M = 4, the fused decode FFN products gemv_gate_up and gemv_silu_gate with a
    residual, the product without the transpose at the decode shape, the decode product with
    float16 x, scales and biases, quantize of a bf16
    [4096, 4096] weight, and the mixture-of-experts gathered product
    gather_qmm at 1 and 64 tokens), each against its roofline;
  * `context`: what the GPU does on the same sizes without this library, timed the same way: an
    empty kernel launch, a device copy of the decode step's bytes, a dense bf16 matmul at the
    prefill shape;
  * `cpu_baseline`: the CPU oracle on the host cores, on a bounded sample of the same workload
    (also given per row).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-prefill] [--no-rows]
    python bench.py --eager ...           # plain launches, no graph (for profilers)
    python bench.py --copy-calibration    # a plain copy of known size (counter calibration)
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

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
METRIC = "qmm effective weight GB/s (GEMV, % HBM peak); TFLOP/s (GEMM, % MFMA peak)"
ROTATE_BYTES = 1 << 30


def qmm_bytes(m, n, k, bits, group, xsize=2, ysize=2):
    """Algorithmic bytes of one qmm: packed codes + bf16 scale and bias per group + x + y."""
    return n * k * bits // 8 + 4 * n * k // group + m * k * xsize + m * n * ysize


def dequant_bytes(rows, k, bits, group, osize, indices=False):
    """Reads the packed codes, scales and biases of `rows` rows (and the uint32 indices), writes
    rows * k outputs."""
    return rows * k * bits // 8 + 4 * rows * k // group + (4 * rows if indices else 0) + rows * k * osize


def source_hash(*names):
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "quantized_matmul_mlx_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_key, sources):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when the
    kernel's sources or the build flags (build.py) changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_key}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(*sources):
        return None
    return rec.get("hbm_bytes_per_launch")


class Aux:
    """The benchmark's measurement aids (libqaff_bench.so, include/qaff_bench.h): device timestamps
    and a plain streaming read. Not part of the product path."""

    def __init__(self):
        import ctypes
        path = os.path.join(ROOT, "quantized_matmul_mlx_amd", "libqaff_bench.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m quantized_matmul_mlx_amd.build` first")
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        lib.qaff_bench_read.argtypes = [vp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, vp, vp]
        lib.qaff_bench_read_store.argtypes = [vp, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, vp, ctypes.c_uint32, vp]
        lib.qaff_bench_stamp.argtypes = [vp, vp]
        lib.qaff_bench_read.restype = lib.qaff_bench_stamp.restype = ctypes.c_int
        lib.qaff_bench_read_store.restype = ctypes.c_int
        lib.qaff_bench_wall_clock_khz.restype = ctypes.c_int
        self.lib = lib

    def stamp(self, torch, slot):
        rc = self.lib.qaff_bench_stamp(slot.data_ptr(), torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"qaff_bench_stamp: hip error {rc}")

    def read(self, torch, src, per_thread, nt, sink, out=None):
        stream = torch.cuda.current_stream().cuda_stream
        if out is None:
            rc = self.lib.qaff_bench_read(src.data_ptr(), src.numel() * src.element_size(), per_thread, nt,
                                          0xFFFFFFFF, sink.data_ptr(), stream)
        else:
            rc = self.lib.qaff_bench_read_store(src.data_ptr(), src.numel() * src.element_size(), per_thread, nt,
                                                out.data_ptr(), out.numel(), stream)
        if rc != 0:
            raise RuntimeError(f"qaff_bench_read: hip error {rc}")


class Timer:
    """Times `steps` launches of `launch(i)` after `warmup` untimed ones.

    Graph mode (default): the K steps are one captured HIP graph, framed by two device-timestamp
    kernels inside the same graph. The time per step is (last stamp - first stamp - the same frame
    with nothing inside) / K: every kernel of the K steps and every gap between dependent kernels,
    without the graph's own submission. Events recorded on the launch stream around the replay
    give the second figure, submission included (`last["replay_ms"]`).
    Eager mode (for profilers): plain launches bracketed by events on the launch stream."""

    def __init__(self, torch, eager, aux):
        self.torch = torch
        self.eager = eager
        self.aux = aux
        self.last = {}
        self._frame = None
        if not eager:
            self.khz = aux.lib.qaff_bench_wall_clock_khz()
            if self.khz <= 0:
                raise RuntimeError("the device wall clock rate is unavailable")
            self.slots = torch.zeros(2, dtype=torch.int64, device="cuda")

    def _capture(self, body):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                self.aux.stamp(torch, self.slots[0:1])
                body()
                self.aux.stamp(torch, self.slots[1:2])
        torch.cuda.current_stream().wait_stream(side)
        return g

    def _stamped_ms(self):
        t = self.slots.cpu().tolist()
        return (t[1] - t[0]) / self.khz

    def frame_ms(self):
        """Two stamps with nothing between them: one gap and the stamp kernel itself."""
        if self._frame is None:
            g = self._capture(lambda: None)
            best = None
            for _ in range(20):
                g.replay()
                self.torch.cuda.synchronize()
                v = self._stamped_ms()
                best = v if best is None else min(best, v)
            self._frame = best
        return self._frame

    def __call__(self, launch, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            launch(i)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        if self.eager:
            start.record()
            for i in range(steps):
                launch(i)
            end.record()
            torch.cuda.synchronize()
            ms = start.elapsed_time(end) / steps
            self.last = {"replay_ms": ms}
            return ms
        frame = self.frame_ms()

        def body():
            for i in range(steps):
                launch(i)
        g = self._capture(body)
        g.replay()                      # untimed: the first replay pays one-time upload costs
        torch.cuda.synchronize()
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        replay_ms = start.elapsed_time(end) / steps
        ms = (self._stamped_ms() - frame) / steps
        self.last = {"replay_ms": replay_ms, "graph_ms": ms, "frame_ms": frame}
        return ms


def to_device(torch, inp):
    import numpy as np
    d = {
        "packed": torch.from_numpy(inp.packed.view(np.int32)).cuda(),
        "scales": torch.from_numpy(inp.scales.view(np.int16)).cuda().view(torch.bfloat16),
        "biases": torch.from_numpy(inp.biases.view(np.int16)).cuda().view(torch.bfloat16),
    }
    if inp.x is not None:
        d["x"] = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
    if inp.indices is not None:
        d["idx"] = torch.from_numpy(inp.indices.view(np.int32)).cuda()
    return d


def copies_for(nbytes, cap=256):
    return int(max(1, min(cap, -(-ROTATE_BYTES // max(1, nbytes)))))


def replicate(torch, d, copies):
    return [{k: v.clone() for k, v in d.items()} for _ in range(copies)]


def cpu_time(fn, budget_s, max_runs):
    """Runs fn until budget_s seconds or max_runs runs; returns (runs, seconds)."""
    runs, t0 = 0, time.perf_counter()
    while True:
        fn()
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= max_runs:
            return runs, el


def hbm_roofline(gbs, traffic=None):
    return {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}


# ---- the headline and the rows ------------------------------------------------------------------

def kernel_name(q, m, k):
    """The kernel the automatic dispatch picks for a bf16 x of m rows (the library's rule)."""
    if m > q.gemv_max_m():
        return "gemm"
    if m >= q.gemv_mfma_min_m(k) and k % 512 == 0 and k <= 32768:
        return "gemv_mfma"
    return "gemv"


def bench_qmm(torch, q, W, timer, name, m, steps, warmup, cpu, cpu_budget):
    """One qmm workload at M = m, rotated over ~1 GiB of operand copies."""
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, m=m)
    b = qmm_bytes(m, wl.n, wl.k, wl.bits, wl.group_size)
    copies = copies_for(b)
    sets = replicate(torch, to_device(torch, inp), copies)
    ys = [torch.empty((m, wl.n), dtype=torch.bfloat16, device="cuda") for _ in range(copies)]

    def launch(i):
        s = sets[i % copies]
        q.qmm(s["x"], s["packed"], s["scales"], s["biases"], wl.group_size, wl.bits, out=ys[i % copies])

    ms = timer(launch, steps, warmup)
    del sets, ys
    torch.cuda.empty_cache()
    gbs = b / (ms * 1e-3) / 1e9
    row = {"workload": f"{name} M={m}", "kernel": kernel_name(q, m, wl.k),
           "bytes_per_step": b, "ms_per_step": round(ms, 6), "weight_copies": copies,
           "roofline": hbm_roofline(gbs)}
    if cpu:
        import oracle
        threads = oracle.default_threads()
        runs, el = cpu_time(lambda: oracle.qmm(inp.x, "bf16", inp.packed, inp.scales, inp.biases,
                                               wl.group_size, wl.bits, threads=threads), cpu_budget, 100000)
        row["cpu_baseline"] = {"value": round(b * runs / el / 1e9, 4), "unit": "GB/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"the whole step, {runs} run(s) in {el:.1f} s"}
    return row, gbs, ms, inp


def bench_fused(torch, q, W, timer, kind, steps, warmup, cpu, cpu_budget):
    """The fused decode products at the FFN shapes (4-bit g64, M = 1): "gate_up" (both [14336, 4096]
    projections of one x) or "silu_gate" (down [4096, 14336] on silu(gate) * up plus the residual)."""
    import numpy as np
    if kind == "gate_up":
        wa, wb = W.WORKLOADS["ffn_gate_4bit_g64_14336x4096"], W.WORKLOADS["ffn_up_4bit_g64_14336x4096"]
        a, bb = W.make_inputs(wa, m=1), W.make_inputs(wb, m=1)
        wbytes = 2 * (qmm_bytes(1, wa.n, wa.k, wa.bits, wa.group_size) - wa.k * 2 - wa.n * 2)
        nbytes = wbytes + wa.k * 2 + 2 * wa.n * 2
        copies = copies_for(nbytes)
        sa = replicate(torch, to_device(torch, a), copies)
        sb = replicate(torch, to_device(torch, bb), copies)

        def launch(i):
            x, y = sa[i % copies], sb[i % copies]
            q.gemv_gate_up(x["x"], (x["packed"], x["scales"], x["biases"]),
                           (y["packed"], y["scales"], y["biases"]), wa.group_size, wa.bits)

        def cpu_step():
            oracle.qmm(a.x, "bf16", a.packed, a.scales, a.biases, wa.group_size, wa.bits, threads=threads)
            oracle.qmm(a.x, "bf16", bb.packed, bb.scales, bb.biases, wa.group_size, wa.bits, threads=threads)
        label = "gemv_gate_up 2 x [14336, 4096] 4-bit g64 M=1"
        sets = (sa, sb)
    else:
        wd = W.WORKLOADS["ffn_down_4bit_g64_4096x14336"]
        d = W.make_inputs(wd, m=1)
        rng = np.random.default_rng(34)
        gate = W.bf16_bits_from_f32(rng.standard_normal((1, wd.k), dtype=np.float32))
        up = W.bf16_bits_from_f32(rng.standard_normal((1, wd.k), dtype=np.float32))
        resid = W.bf16_bits_from_f32(rng.standard_normal((1, wd.n), dtype=np.float32))
        # weight + gate + up + residual + y
        nbytes = (qmm_bytes(1, wd.n, wd.k, wd.bits, wd.group_size) - wd.k * 2 - wd.n * 2) + 2 * wd.k * 2 + 2 * wd.n * 2
        copies = copies_for(nbytes)
        sd = replicate(torch, to_device(torch, d), copies)
        g_t = [torch.from_numpy(gate.view(np.int16)).cuda().view(torch.bfloat16) for _ in range(copies)]
        u_t = [torch.from_numpy(up.view(np.int16)).cuda().view(torch.bfloat16) for _ in range(copies)]
        r_t = torch.from_numpy(resid.view(np.int16)).cuda().view(torch.bfloat16)

        def launch(i):
            s = sd[i % copies]
            q.gemv_silu_gate(g_t[i % copies], u_t[i % copies], s["packed"], s["scales"], s["biases"],
                             wd.group_size, wd.bits, resid=r_t)

        def cpu_step():
            oracle.silu_gate_qmm(gate, up, resid, d.packed, d.scales, d.biases, wd.group_size, wd.bits,
                                 threads=threads)
        label = "gemv_silu_gate + residual [4096, 14336] 4-bit g64 M=1"
        sets = (sd, g_t, u_t)
    ms = timer(launch, steps, warmup)
    del sets
    torch.cuda.empty_cache()
    gbs = nbytes / (ms * 1e-3) / 1e9
    row = {"workload": label, "kernel": f"gemv_{kind} (fused)", "bytes_per_step": nbytes,
           "ms_per_step": round(ms, 6), "copies": copies, "roofline": hbm_roofline(gbs)}
    if cpu:
        import oracle
        threads = oracle.default_threads()
        runs, el = cpu_time(cpu_step, cpu_budget, 100000)
        row["cpu_baseline"] = {"value": round(nbytes * runs / el / 1e9, 4), "unit": "GB/s", "cores": threads,
                               "kind": "oracle", "sample": f"the whole step, {runs} run(s) in {el:.1f} s"}
    return row


def bench_gather(torch, q, W, timer, tokens, steps, warmup, cpu, cpu_budget, name="moe_4bit_g64_e128_768x2048",
                 f16=False):
    """A mixture-of-experts gathered product (gather_qmm): 128 experts of W [768, 2048] at 4-bit
    g64, 8 experts per token, the tokens' rows sorted by expert (rows = 8 * tokens, x [rows, 1, k]).
    Algorithmic bytes: the weights of the experts in use, x rows, y rows. At prefill size (experts
    averaging 32 rows or more: the grouped GEMM) the row is in TFLOP/s against the bf16 MFMA peak.
    f16: x, scales and biases as float16 (the workload's values converted; y float16): the float16
    forms of the same kernels."""
    import numpy as np
    wl = W.WORKLOADS[name]
    mi = W.moe_inputs(wl, tokens)
    rows = mi.expert.size
    used = int(np.unique(mi.expert).size)
    per_expert = wl.n * wl.k * wl.bits // 8 + 2 * wl.n * (wl.k // wl.group_size) * 2
    nbytes = used * per_expert + rows * wl.k * 2 + rows * wl.n * 2
    all_bytes = wl.experts * per_expert  # a copy holds every expert
    copies = copies_for(all_bytes)
    if f16:
        to16 = lambda a: W.f32_from_bf16_bits(a).astype(np.float16).view(np.uint16)
        hs, hb, hx = to16(mi.scales), to16(mi.biases), to16(mi.x_rows)
        tdt = torch.float16
    else:
        hs, hb, hx = mi.scales, mi.biases, mi.x_rows
        tdt = torch.bfloat16
    dev = [{"packed": torch.from_numpy(mi.packed.view(np.int32)).cuda(),
            "scales": torch.from_numpy(hs.view(np.int16)).cuda().view(tdt),
            "biases": torch.from_numpy(hb.view(np.int16)).cuda().view(tdt),
            "x": torch.from_numpy(hx.view(np.int16)).cuda().view(tdt)} for _ in range(copies)]
    rhs = torch.from_numpy(mi.expert.view(np.int32)).cuda()
    ys = [torch.empty((rows, 1, wl.n), dtype=tdt, device="cuda") for _ in range(copies)]

    def launch(i):
        s = dev[i % copies]
        q.gather_qmm(s["x"], s["packed"], s["scales"], s["biases"], wl.group_size, wl.bits, rhs_indices=rhs,
                     sorted_indices=True, out=ys[i % copies])

    ms = timer(launch, steps, warmup)
    del dev, ys
    torch.cuda.empty_cache()
    gbs = nbytes / (ms * 1e-3) / 1e9
    grouped = rows >= wl.experts
    gemm = rows >= 32 * wl.experts
    kernel = "gemm_grouped" if gemm else ("gemv_mfma_gather (grouped)" if grouped else "gemv_gather (batched)")
    if f16:
        kernel = kernel.replace("gemv_gather (batched)", "gemv_typed_kernel (gathered)") + (", float16" if grouped else "")
    row = {"workload": f"gather_qmm {wl.experts} experts [768, 2048] 4-bit g64, top-{wl.top_k}, {tokens} token(s), "
                       f"{rows} rows sorted by expert ({used} experts in use)" +
                       (", float16 x, scales and biases" if f16 else ""),
           "kernel": kernel,
           "bytes_per_step": nbytes, "ms_per_step": round(ms, 6), "weight_copies": copies,
           "roofline": hbm_roofline(gbs)}
    if gemm:
        flop = 2.0 * rows * wl.n * wl.k
        tflops = flop / (ms * 1e-3) / 1e12
        row["tflops"] = round(tflops, 2)
        row["roofline"] = {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None}
    if cpu and gemm:
        import oracle
        # a sample: the rows of the first expert through the oracle's product (the typed one on one
        # thread)
        threads = 1 if f16 else oracle.default_threads()
        sel = np.flatnonzero(mi.expert == mi.expert[0])
        xs = np.ascontiguousarray((hx if f16 else mi.x_rows)[sel, 0, :])
        e0 = int(mi.expert[0])
        t0 = time.perf_counter()
        if f16:
            oracle.qmm_typed(xs, "f16", mi.packed[e0], hs[e0], hb[e0], "f16", wl.group_size, wl.bits)
        else:
            oracle.qmm(xs, "bf16", mi.packed[e0], mi.scales[e0], mi.biases[e0], wl.group_size, wl.bits, threads=threads)
        el = time.perf_counter() - t0
        row["cpu_baseline"] = {"value": round(2.0 * sel.size * wl.n * wl.k / el / 1e12, 6), "unit": "TFLOP/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"the {sel.size} rows of one expert, {el:.2f} s"}
    elif cpu and f16:
        import oracle
        runs, el = cpu_time(lambda: oracle.gather_qmm_typed(hx, "f16", mi.packed, hs, hb, "f16", wl.group_size,
                                                            wl.bits, rhs=mi.expert), cpu_budget, 100000)
        row["cpu_baseline"] = {"value": round(nbytes * runs / el / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "sample": f"the whole step, {runs} run(s) in {el:.1f} s"}
    elif cpu:
        import oracle
        threads = oracle.default_threads()
        runs, el = cpu_time(lambda: oracle.gather_qmm(mi.x_rows, "bf16", mi.packed, mi.scales, mi.biases,
                                                      wl.group_size, wl.bits, rhs=mi.expert, threads=threads),
                            cpu_budget, 100000)
        row["cpu_baseline"] = {"value": round(nbytes * runs / el / 1e9, 4), "unit": "GB/s", "cores": threads,
                               "kind": "oracle", "sample": f"the whole step, {runs} run(s) in {el:.1f} s"}
    return row


def bench_qmm_nt(torch, q, W, timer, steps, warmup, cpu, cpu_budget, f16=False):
    """The product without the transpose at the decode shape: x bf16 [1, 4096] . dequantize(W) for
    W stored [4096 (k), 4096 (n)], 4-bit g64 (groups along n). Algorithmic bytes as for qmm. With
    f16, x, scales and biases are float16 (the same draws converted) and so is y."""
    import numpy as np
    wl = W.WORKLOADS["decode_4bit_g64_4096x4096"]
    inp = W.make_inputs(wl, m=1)          # the same draws, read as a [k, n] weight
    b = qmm_bytes(1, wl.n, wl.k, wl.bits, wl.group_size)
    copies = copies_for(b)
    if f16:
        s16 = W.f32_from_bf16_bits(inp.scales).astype(np.float16).view(np.uint16)
        b16 = W.f32_from_bf16_bits(inp.biases).astype(np.float16).view(np.uint16)
        x16 = W.f32_from_bf16_bits(inp.x).astype(np.float16).view(np.uint16)
        h = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.float16)
        sets = [{"packed": torch.from_numpy(inp.packed.view(np.int32)).cuda(), "scales": h(s16), "biases": h(b16),
                 "x": h(x16)} for _ in range(copies)]
    else:
        sets = replicate(torch, to_device(torch, inp), copies)
    ydt = torch.float16 if f16 else torch.bfloat16
    ys = [torch.empty((1, wl.n), dtype=ydt, device="cuda") for _ in range(copies)]

    def launch(i):
        s = sets[i % copies]
        q.qmm_nt(s["x"], s["packed"], s["scales"], s["biases"], wl.group_size, wl.bits, out=ys[i % copies])

    ms = timer(launch, steps, warmup)
    del sets, ys
    torch.cuda.empty_cache()
    gbs = b / (ms * 1e-3) / 1e9
    what = "x, scales and biases float16" if f16 else "x bf16"
    row = {"workload": f"qmm without the transpose, W [4096 (k), 4096 (n)] 4-bit g64, {what} [1, 4096]",
           "kernel": "qmm_nt_partial_kernel + qmm_nt_reduce_kernel" + (", typed form" if f16 else ""),
           "bytes_per_step": b, "ms_per_step": round(ms, 6), "weight_copies": copies, "roofline": hbm_roofline(gbs)}
    if cpu:
        import oracle
        if f16:
            fn = lambda: oracle.qmm_nt_typed(x16, "f16", inp.packed, s16, b16, "f16", wl.group_size, wl.bits)
        else:
            fn = lambda: oracle.qmm_nt(inp.x, "bf16", inp.packed, inp.scales, inp.biases, wl.group_size, wl.bits)
        runs, el = cpu_time(fn, cpu_budget, 100000)
        row["cpu_baseline"] = {"value": round(b * runs / el / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "sample": f"the whole step, {runs} run(s) in {el:.1f} s"}
    return row


def bench_typed(torch, q, W, timer, steps, warmup, cpu, cpu_budget, m=1):
    """qmm with float16 x, scales and biases (y float16) at the decode shape W [4096, 4096] 4-bit
    g64: at M = 1 the GEMV in float16, at M = 4 the matrix-core decode kernel in float16. The scales,
    biases and x are the decode workload's, as float16."""
    import numpy as np
    wl = W.WORKLOADS["decode_4bit_g64_4096x4096"]
    inp = W.make_inputs(wl, m=m)
    s16 = W.f32_from_bf16_bits(inp.scales).astype(np.float16).view(np.uint16)
    b16 = W.f32_from_bf16_bits(inp.biases).astype(np.float16).view(np.uint16)
    x16 = W.f32_from_bf16_bits(inp.x).astype(np.float16).view(np.uint16)
    b = qmm_bytes(m, wl.n, wl.k, wl.bits, wl.group_size)
    copies = copies_for(b)
    h = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.float16)
    sets = [{"packed": torch.from_numpy(inp.packed.view(np.int32)).cuda(), "scales": h(s16), "biases": h(b16),
             "x": h(x16)} for _ in range(copies)]
    ys = [torch.empty((m, wl.n), dtype=torch.float16, device="cuda") for _ in range(copies)]

    def launch(i):
        s = sets[i % copies]
        q.qmm(s["x"], s["packed"], s["scales"], s["biases"], wl.group_size, wl.bits, out=ys[i % copies])

    ms = timer(launch, steps, warmup)
    del sets, ys
    torch.cuda.empty_cache()
    gbs = b / (ms * 1e-3) / 1e9
    kernel = "gemv_mfma_kernel, float16" if m >= q.gemv_mfma_min_m(wl.k) else "gemv_bf16_kernel, float16 format"
    row = {"workload": f"qmm float16 x, scales and biases, W [4096, 4096] 4-bit g64, M={m}", "kernel": kernel,
           "bytes_per_step": b, "ms_per_step": round(ms, 6), "weight_copies": copies, "roofline": hbm_roofline(gbs)}
    if cpu:
        import oracle
        threads = oracle.default_threads()
        runs, el = cpu_time(lambda: oracle.qmm_typed(x16, "f16", inp.packed, s16, b16, "f16", wl.group_size, wl.bits),
                            cpu_budget, 100000)
        row["cpu_baseline"] = {"value": round(b * runs / el / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "sample": f"the whole step, {runs} run(s) in {el:.1f} s"}
    return row


def bench_quantize(torch, q, W, timer, steps, warmup, cpu, cpu_budget, dtype="bf16"):
    """quantize of a dense weight [4096, 4096] ~ N(0, 0.02^2) to 4-bit g64, bf16 (or, with dtype
    "f16", float16: the same draws converted), scales and biases in the weight's dtype. Algorithmic
    bytes: the weight read, the codes, scales and biases written."""
    import numpy as np
    wl = W.WORKLOADS["quantize_4bit_g64_4096x4096"]
    w = W.dense_weight(wl.n, wl.k, "bf16", seed=wl.seed)
    tdt = torch.bfloat16
    if dtype == "f16":
        w = W.f32_from_bf16_bits(w).astype(np.float16).view(np.uint16)
        tdt = torch.float16
    nbytes = wl.n * wl.k * 2 + wl.n * wl.k * wl.bits // 8 + 2 * wl.n * (wl.k // wl.group_size) * 2
    copies = copies_for(nbytes)
    ws = [torch.from_numpy(w.view(np.int16)).cuda().view(tdt) for _ in range(copies)]

    def launch(i):
        q.quantize(ws[i % copies], wl.group_size, wl.bits)

    ms = timer(launch, steps, warmup)
    del ws
    torch.cuda.empty_cache()
    gbs = nbytes / (ms * 1e-3) / 1e9
    name = {"bf16": "bf16", "f16": "float16"}[dtype]
    row = {"workload": f"quantize {name} [4096, 4096] -> 4-bit g64, {name} scales and biases",
           "kernel": "quantize_kernel", "bytes_per_step": nbytes, "ms_per_step": round(ms, 6), "copies": copies,
           "roofline": hbm_roofline(gbs)}
    if cpu:
        import oracle
        runs, el = cpu_time(lambda: oracle.quantize(w, dtype, wl.group_size, wl.bits, dtype), cpu_budget, 100000)
        row["cpu_baseline"] = {"value": round(nbytes * runs / el / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "sample": f"the whole step, {runs} run(s) in {el:.1f} s"}
    return row


def bench_dequant(torch, q, W, timer, name, out_dtype, steps, warmup, cpu, cpu_budget, gather):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl)
    rows_out = wl.n_indices if gather else wl.n
    osize = 4 if out_dtype == "f32" else 2
    tdt = torch.float32 if out_dtype == "f32" else torch.bfloat16
    b = dequant_bytes(rows_out, wl.k, wl.bits, wl.group_size, osize, indices=gather)
    d = to_device(torch, inp)
    if gather:
        # the table itself is large (75 MB); rotate the indices and outputs, and the table
        # copies as far as ~1 GiB allows
        table_bytes = inp.packed.nbytes + inp.scales.nbytes + inp.biases.nbytes
        copies = copies_for(table_bytes + rows_out * wl.k * osize, cap=16)
    else:
        copies = copies_for(b, cap=64)
    sets = replicate(torch, d, copies)
    outs = [torch.empty((rows_out, wl.k), dtype=tdt, device="cuda") for _ in range(copies)]

    def launch(i):
        s = sets[i % copies]
        if gather:
            q.dequant_rows(s["packed"], s["scales"], s["biases"], s["idx"], wl.group_size, wl.bits, tdt,
                           out=outs[i % copies])
        else:
            q.dequantize(s["packed"], s["scales"], s["biases"], wl.group_size, wl.bits, tdt,
                         out=outs[i % copies])

    ms = timer(launch, steps, warmup)
    del sets, outs
    torch.cuda.empty_cache()
    gbs = b / (ms * 1e-3) / 1e9
    kind = "dequant_rows" if gather else "dequantize"
    row = {"workload": f"{name} {kind} -> {out_dtype}", "kernel": kind, "bytes_per_step": b,
           "ms_per_step": round(ms, 6), "copies": copies, "roofline": hbm_roofline(gbs)}
    if cpu:
        import oracle
        threads = oracle.default_threads()
        sample = 512
        if gather:
            idx = inp.indices[:sample]
            fn = lambda: oracle.dequant_rows(inp.packed, inp.scales, inp.biases, idx, wl.group_size,
                                             wl.bits, out=out_dtype, threads=threads)
        else:
            fn = lambda: oracle.dequantize(inp.packed[:sample], inp.scales[:sample], inp.biases[:sample],
                                           wl.group_size, wl.bits, out=out_dtype, threads=threads)
        runs, el = cpu_time(fn, cpu_budget, 100000)
        bs = dequant_bytes(sample, wl.k, wl.bits, wl.group_size, osize, indices=gather)
        row["cpu_baseline"] = {"value": round(bs * runs / el / 1e9, 4), "unit": "GB/s", "cores": threads,
                               "kind": "oracle", "sample": f"{sample} of the {rows_out} rows, {runs} run(s) in {el:.1f} s"}
    return row


class GpuMetrics:
    """Graphics clock (MHz) and socket power (W) of the GPU from amdsmi's metrics table, or nothing
    where amdsmi is unavailable. The table refreshes on the order of a second, so only long
    windows of sustained work read anything meaningful from it."""

    def __init__(self):
        self.smi, self.h = None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.h = amdsmi.amdsmi_get_processor_handles()[0]
            self.smi = amdsmi
        except Exception:
            self.smi, self.h = None, None

    def read(self):
        if self.h is None:
            return None
        try:
            m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
        except Exception:
            return None
        clk, pw = m.get("current_gfxclk"), m.get("current_socket_power")
        if isinstance(clk, (int, float)) and isinstance(pw, (int, float)):
            return float(clk), float(pw)
        return None

    def close(self):
        if self.smi is not None:
            try:
                self.smi.amdsmi_shut_down()
            except Exception:
                pass


def sustained(torch, launch, seconds, metrics, flop):
    """Plain launches back to back for about `seconds`, never more than two batches queued ahead
    (the queue never runs dry), with the clock and power sampled every 50 ms after the first
    second. Time per launch over the whole window."""
    import statistics
    batch = 16
    pending = []
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    n, samples = 0, []
    t0 = last = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            launch(n)
            n += 1
        e = torch.cuda.Event()
        e.record()
        pending.append(e)
        if len(pending) > 2:
            pending.pop(0).synchronize()
        now = time.perf_counter()
        if metrics is not None and now - t0 >= 1.0 and now - last >= 0.05:
            r = metrics.read()
            if r is not None:
                samples.append(r)
            last = now
    end.record()
    end.synchronize()
    ms = start.elapsed_time(end) / n
    res = {"seconds": round(time.perf_counter() - t0, 2), "launches": n, "us_per_launch": round(ms * 1e3, 1),
           "tflops": round(flop / (ms * 1e-3) / 1e12, 1)}
    if samples:
        res["gfxclk_mhz_median"] = statistics.median(c for c, _ in samples)
        res["socket_power_w_median"] = statistics.median(p for _, p in samples)
        res["samples"] = len(samples)
    return res


def bench_prefill(torch, q, W, timer, steps, cpu, metrics=None, sustain_s=0.0):
    wl = W.WORKLOADS["prefill_4bit_g128_4096x14336"]
    m = 2048
    inp = W.make_inputs(wl, m=m)
    copies = 4
    sets = replicate(torch, to_device(torch, inp), copies)
    ys = [torch.empty((m, wl.n), dtype=torch.bfloat16, device="cuda") for _ in range(copies)]

    def launch(i):
        s = sets[i % copies]
        q.qmm(s["x"], s["packed"], s["scales"], s["biases"], wl.group_size, wl.bits, out=ys[i % copies])

    burst_ms = timer(launch, steps, 3)
    flop = 2.0 * m * wl.n * wl.k
    held = sustained(torch, launch, sustain_s, metrics, flop) if sustain_s > 0 else None
    del sets, ys
    torch.cuda.empty_cache()
    # The figure is the steady state of back-to-back GEMMs when measured (the power-limited chip
    # settles after a transient dip that a short burst right after idle falls into), else the burst.
    ms = held["us_per_launch"] * 1e-3 if held is not None else burst_ms
    tflops = flop / (ms * 1e-3) / 1e12
    res = {
        "workload": "prefill GEMM: 4-bit codes, group 128, W [4096, 14336], x bf16 [2048, 14336], "
                    "y bf16 [2048, 4096]; seed 0",
        "ms_per_step": round(ms, 5),
        "tflops": round(tflops, 2),
        "timing": (f"{held['launches']} launches back to back over {held['seconds']} s, events on the launch stream"
                   if held is not None else f"one HIP graph of {steps} launches, events on the launch stream"),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": read_traffic("gemm_4bit_g128_prefill", ["gemm_impl.h", "mfma16.h", "qaff_device.h", "../build.py"])},
    }
    if held is not None:
        res["sustained"] = held
        burst_tf = flop / (burst_ms * 1e-3) / 1e12
        res["burst"] = {"launches": steps, "ms_per_step": round(burst_ms, 5), "tflops": round(burst_tf, 2),
                        "frac": round(burst_tf / BF16_MFMA_PEAK_TFLOPS, 4),
                        "timing": f"one HIP graph of {steps} launches after the decode rows"}
    if cpu:
        import oracle
        threads = oracle.default_threads()
        rows = 64
        t0 = time.perf_counter()
        oracle.qmm(inp.x[:rows], "bf16", inp.packed, inp.scales, inp.biases, wl.group_size, wl.bits,
                   threads=threads)
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(2.0 * rows * wl.n * wl.k / el / 1e12, 6), "unit": "TFLOP/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"{rows} of the 2048 x rows against all of W, {el:.1f} s"}
    return res


def bench_prefill_small(torch, q, W, timer, m, steps, warmup, cpu, cpu_budget, name="prefill_4bit_g128_4096x14336",
                        f16=False):
    """A prefill GEMM on the automatic path: by default the prefill weight at a small batch
    (4-bit g128, W [4096, 14336], x bf16 [m, 14336]), whose few tiles split K through a workspace
    (qaff_qmm_ws); or another GEMM workload. Against the 16-bit MFMA peak (2·m·n·k flop per step;
    bf16 and float16 have the same). f16: x, scales and biases as float16 (the workload's values
    converted), the GEMM in float16."""
    import numpy as np
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, m=m)
    b = qmm_bytes(m, wl.n, wl.k, wl.bits, wl.group_size)
    copies = copies_for(b)
    if f16:
        to16 = lambda a: W.f32_from_bf16_bits(a).astype(np.float16).view(np.uint16)
        h16 = {"x": to16(inp.x), "scales": to16(inp.scales), "biases": to16(inp.biases)}
        h = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.float16)
        sets = [{"packed": torch.from_numpy(inp.packed.view(np.int32)).cuda(), "scales": h(h16["scales"]),
                 "biases": h(h16["biases"]), "x": h(h16["x"])} for _ in range(copies)]
    else:
        sets = replicate(torch, to_device(torch, inp), copies)
    ys = [torch.empty((m, wl.n), dtype=torch.float16 if f16 else torch.bfloat16, device="cuda") for _ in range(copies)]

    def launch(i):
        s = sets[i % copies]
        q.qmm(s["x"], s["packed"], s["scales"], s["biases"], wl.group_size, wl.bits, out=ys[i % copies])

    ms = timer(launch, steps, warmup)
    del sets, ys
    torch.cuda.empty_cache()
    flop = 2.0 * m * wl.n * wl.k
    tflops = flop / (ms * 1e-3) / 1e12
    lib = q._lib.load()
    splits = int(lib.qaff_qmm_workspace_size(m, wl.n, wl.k, wl.group_size, wl.bits)) > 0 and not f16
    kernel = "gemm_direct_kernel" + (" (general: K with a tail)" if wl.k % 1024 else "") + (", float16" if f16 else "")
    row = {"workload": f"{name} M={m}" + (" (small batch)" if splits else "") + (", float16 x, scales and biases" if f16 else ""),
           "kernel": kernel + (", K split through a workspace (qaff_qmm_ws)" if splits else ""),
           "splits_workspace_bytes": int(lib.qaff_qmm_workspace_size(m, wl.n, wl.k, wl.group_size, wl.bits)) if splits else 0,
           "bytes_per_step": b, "ms_per_step": round(ms, 6), "tflops": round(tflops, 2), "weight_copies": copies,
           "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None}}
    if cpu:
        import oracle
        threads = oracle.default_threads()
        rows = 64
        t0 = time.perf_counter()
        if f16:  # the typed oracle runs on one thread
            rows, threads = 8, 1
            oracle.qmm_typed(h16["x"][:rows], "f16", inp.packed, h16["scales"], h16["biases"], "f16", wl.group_size,
                             wl.bits)
        else:
            oracle.qmm(inp.x[:rows], "bf16", inp.packed, inp.scales, inp.biases, wl.group_size, wl.bits, threads=threads)
        el = time.perf_counter() - t0
        row["cpu_baseline"] = {"value": round(2.0 * rows * wl.n * wl.k / el / 1e12, 6), "unit": "TFLOP/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"{rows} of the {m} x rows against all of W, {el:.1f} s"}
    return row


def plain_read(torch, timer, aux, nbytes, steps, warmup, store=0):
    """The ceiling of a kernel that must read `nbytes` bytes once: a plain streaming read
    (qaff_bench_read) of that many bytes, rotated over about 1 GiB of copies like the product rows
    and timed the same way; the best of its eight launch shapes (1, 2, 4 or 8 16-byte loads per
    thread, with and without the non-temporal bit). With `store` (an element count), every wave
    also writes one dependent 2-byte result into an array of that many elements
    (qaff_bench_read_store): the ceiling of a kernel that reads the bytes and writes its output."""
    copies = (1 << 30) // nbytes + 1
    srcs = [torch.randint(0, 1 << 30, (nbytes // 4,), dtype=torch.int32, device="cuda") for _ in range(copies)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    outs = [torch.zeros(store, dtype=torch.int16, device="cuda") for _ in range(copies)] if store else None
    shapes = {}
    for per_thread in (1, 2, 4, 8):
        for nt in (0, 1):
            ms = timer(lambda i: aux.read(torch, srcs[i % copies], per_thread, nt, sink,
                                          outs[i % copies] if outs else None), steps, warmup)
            shapes[f"{per_thread}{'nt' if nt else ''}"] = round(ms * 1e3, 3)
    del srcs, outs
    torch.cuda.empty_cache()
    best = min(shapes, key=shapes.get)
    us = shapes[best]
    return {"bytes": nbytes, "us_per_step": us, "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "best_shape": best,
            "us_by_shape": shapes, "copies": copies}


def bench_context(torch, timer, aux, metrics=None, sustain_s=0.0):
    """What the same box does on the same sizes without this library, timed the same way: an
    empty kernel launch, a plain streaming read of the decode step's bytes and of the 8-bit step's
    (the ceiling of any kernel that reads them), the decode step's read with one dependent 2-byte
    store per wave into 4096 elements (the ceiling of a kernel that also writes y), a device copy
    of the decode step's bytes, and a
    dense bf16 matmul at the prefill shape (the vendor BLAS). Context for the roofline fractions,
    not a result of the path."""
    steps = 1000
    empty_ms = timer(lambda i: torch.cuda._sleep(0), steps, 100)
    read_decode = plain_read(torch, timer, aux, 9453568, steps, 100)
    read_store_decode = plain_read(torch, timer, aux, 9453568, steps, 100, store=4096)
    read_int8 = plain_read(torch, timer, aux, 62427136, 200, 20)

    nbytes = 9453568                                      # the decode step's algorithmic bytes
    copies = (1 << 30) // nbytes + 1                     # about 1 GiB: four times the MALL
    srcs = [torch.randint(0, 1 << 30, (nbytes // 4,), dtype=torch.int32, device="cuda") for _ in range(copies)]
    dsts = [torch.empty_like(t) for t in srcs]
    copy_ms = timer(lambda i: dsts[i % copies].copy_(srcs[i % copies]), steps, 100)
    del srcs, dsts

    g = torch.Generator(device="cuda").manual_seed(0)
    xs = torch.randn((2048, 14336), generator=g, device="cuda").to(torch.bfloat16)
    ws = torch.randn((4096, 14336), generator=g, device="cuda").to(torch.bfloat16)
    y = torch.empty((2048, 4096), dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        torch.matmul(xs, ws.t(), out=y)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    mm_steps = 20
    start.record()
    for _ in range(mm_steps):
        torch.matmul(xs, ws.t(), out=y)
    end.record()
    torch.cuda.synchronize()
    mm_ms = start.elapsed_time(end) / mm_steps
    flop = 2.0 * 2048 * 4096 * 14336
    held = (sustained(torch, lambda i: torch.matmul(xs, ws.t(), out=y), sustain_s, metrics, flop)
            if sustain_s > 0 else None)
    del xs, ws, y
    torch.cuda.empty_cache()
    res = {
        "empty_kernel_us_per_launch": round(empty_ms * 1e3, 3),
        "plain_read_decode_bytes": read_decode,
        "plain_read_store_decode_bytes": read_store_decode,
        "plain_read_int8_bytes": read_int8,
        "copy_of_decode_bytes": {"bytes_read": nbytes, "bytes_written": nbytes,
                                 "us_per_step": round(copy_ms * 1e3, 3),
                                 "GBps_moved": round(2 * nbytes / (copy_ms * 1e-3) / 1e9, 1),
                                 "how": f"device copy of a {nbytes}-byte tensor, {copies} rotated copies, "
                                        "same timing as the headline"},
        "dense_bf16_matmul_prefill": {"us_per_step": round(mm_ms * 1e3, 1),
                                      "tflops": round(flop / (mm_ms * 1e-3) / 1e12, 1),
                                      "frac": round(flop / (mm_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                                      "how": "torch.matmul x [2048, 14336] . W^T [14336, 4096], bf16 N(0,1), "
                                             f"{mm_steps} plain launches"},
    }
    if held is not None:
        res["dense_bf16_matmul_prefill"]["sustained"] = held
    return res


def copy_calibration(torch):
    """A plain device copy of 256 MiB, five times: reads and writes exactly 256 MiB each, the
    reference for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)


def short_row(row):
    """A row's name and fraction of its roofline, for the summary line."""
    return {"workload": row["workload"], "frac": row["roofline"]["frac"],
            "us": round(row["ms_per_step"] * 1e3, 2)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--row-steps", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-rows", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the empty-launch, plain-read, device-copy and dense-matmul context")
    ap.add_argument("--sustain", type=float, default=3.0,
                    help="seconds of back-to-back prefill GEMMs (and dense matmuls) with clock and power samples; 0: none")
    ap.add_argument("--eager", action="store_true", help="plain launches instead of one graph")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--full-out", default=None, help="also write the full record (every row, all context) here")
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
    if args.copy_calibration:
        copy_calibration(torch)
        return
    q._lib.load()
    aux = Aux()
    timer = Timer(torch, args.eager, aux)
    metrics = GpuMetrics() if args.sustain > 0 else None
    cpu = not args.no_cpu_baseline
    log = lambda msg: print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ---- decode GEMV (headline) ----
    log(f"decode GEMV M=1: warmup {args.warmup}, steps {args.steps}")
    row, gbs, ms, inp = bench_qmm(torch, q, W, timer, "decode_4bit_g64_4096x4096", 1, args.steps,
                                  args.warmup, False, 0)
    head_timing = dict(timer.last)
    wl = inp.wl
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
            "workload": "decode GEMV 4-bit g64, W [4096, 4096], x bf16 [1, 4096], y bf16; seed 0",
            "algorithmic_bytes_per_step": row["bytes_per_step"],
            "weight_copies": row["weight_copies"],
            "timing": ("plain launches, events" if args.eager else
                       "one HIP graph of K launches framed by device timestamps inside it"),
            "replay_us_per_step": round(head_timing.get("replay_ms", ms) * 1e3, 3),
        },
        "roofline": hbm_roofline(gbs, read_traffic("gemv_4bit_g64_4096x4096_m1", ["gemv.hip", "qaff_device.h", "../build.py"])),
    }
    full = {"headline_row": row, "headline_timing": head_timing}

    # ---- prefill GEMM ----
    if not args.no_prefill:
        log(f"prefill GEMM: steps {args.prefill_steps}")
        pg = bench_prefill(torch, q, W, timer, args.prefill_steps, cpu, metrics, args.sustain)
        full["prefill_gemm"] = pg
        summ = {"tflops": pg["tflops"], "frac": pg["roofline"]["frac"], "us": round(pg["ms_per_step"] * 1e3, 1),
                "traffic": pg["roofline"]["traffic"]}
        if "sustained" in pg:
            sd = pg["sustained"]
            summ["timing"] = f"{sd['launches']} back-to-back launches, {sd['seconds']} s"
            summ["gfxclk_mhz"] = sd.get("gfxclk_mhz_median")
            summ["power_w"] = sd.get("socket_power_w_median")
            summ["burst"] = {"tflops": pg["burst"]["tflops"], "frac": pg["burst"]["frac"]}
        result["prefill_gemm"] = summ
        log("prefill: " + json.dumps(summ))

    # ---- what the GPU does on the same sizes without this library ----
    if not args.no_context:
        log("context: empty launch, plain reads, device copy, dense bf16 matmul")
        ctx = bench_context(torch, timer, aux, metrics, args.sustain)
        full["context"] = ctx
        rd = ctx["plain_read_decode_bytes"]
        rw = ctx["plain_read_store_decode_bytes"]
        result["ceiling"] = {"plain_read_us": rd["us_per_step"], "plain_read_frac": rd["frac"],
                             "headline_over_plain_read": round(ms * 1e3 / rd["us_per_step"], 3),
                             "read_store_us": rw["us_per_step"], "read_store_frac": rw["frac"],
                             "empty_launch_us": ctx["empty_kernel_us_per_launch"],
                             "int8_plain_read_frac": ctx["plain_read_int8_bytes"]["frac"]}
        dm = ctx["dense_bf16_matmul_prefill"]
        result["ceiling"]["dense_bf16_gemm_frac"] = dm.get("sustained", {}).get("tflops", dm["tflops"])
        result["ceiling"]["dense_bf16_gemm_frac"] = round(result["ceiling"]["dense_bf16_gemm_frac"] /
                                                          BF16_MFMA_PEAK_TFLOPS, 4)
        log("context: " + json.dumps(result["ceiling"]))

    # ---- the other rows of the path ----
    if not args.no_rows:
        rows = []
        rs, rw = args.row_steps, max(10, args.row_steps // 10)

        def add(r):
            rows.append(r)
            log("row: " + json.dumps(r))
        log("row: prefill GEMM at M = 128 (K split)")
        add(bench_prefill_small(torch, q, W, timer, 128, rs, rw, cpu, 2.0))
        add(bench_prefill_small(torch, q, W, timer, 2048, max(20, rs // 10), 5, cpu, 2.0,
                                name="prefill_4bit_g128_4096x11008"))
        for name, m in (("decode_4bit_g64_4096x4096", 4), ("int8_g64_14336x4096", 1),
                        ("int8_g64_14336x4096", 8), ("odd_3bit_g32_11008x4096", 1),
                        ("odd_3bit_g32_11008x4096", 16), ("odd_6bit_g32_11008x4096", 1),
                        ("odd_6bit_g32_11008x4096", 16), ("ffn_down_4bit_g64_4096x14336", 4)):
            add(bench_qmm(torch, q, W, timer, name, m, rs, rw, cpu, 2.0)[0])
        for out_dtype in ("f32", "bf16"):
            add(bench_dequant(torch, q, W, timer, "decode_4bit_g64_4096x4096", out_dtype, rs, rw,
                              cpu, 2.0, gather=False))
            add(bench_dequant(torch, q, W, timer, "rows_4bit_g64_32768x4096", out_dtype, rs, rw,
                              cpu, 2.0, gather=True))
        for kind in ("gate_up", "silu_gate"):
            add(bench_fused(torch, q, W, timer, kind, rs, rw, cpu, 2.0))
        add(bench_qmm_nt(torch, q, W, timer, rs, rw, cpu, 2.0))
        add(bench_qmm_nt(torch, q, W, timer, rs, rw, cpu, 2.0, f16=True))
        add(bench_typed(torch, q, W, timer, rs, rw, cpu, 2.0))
        add(bench_typed(torch, q, W, timer, rs, rw, cpu, 2.0, m=4))
        add(bench_prefill_small(torch, q, W, timer, 2048, max(20, rs // 10), 5, cpu, 2.0, f16=True))
        add(bench_quantize(torch, q, W, timer, rs, rw, cpu, 2.0))
        add(bench_quantize(torch, q, W, timer, rs, rw, cpu, 2.0, dtype="f16"))
        for tokens in W.WORKLOADS["moe_4bit_g64_e128_768x2048"].ms:
            add(bench_gather(torch, q, W, timer, tokens, rs, rw, cpu, 2.0))
        add(bench_gather(torch, q, W, timer, W.WORKLOADS["moe_4bit_g64_e128_768x2048"].ms[-1], rs, rw, cpu, 2.0,
                         f16=True))
        wl_p = W.WORKLOADS["moe_prefill_4bit_g64_e128_768x2048"]
        add(bench_gather(torch, q, W, timer, wl_p.ms[0], max(20, rs // 10), 5, cpu, 2.0, name=wl_p.name))
        add(bench_gather(torch, q, W, timer, wl_p.ms[0], max(20, rs // 10), 5, cpu, 2.0, name=wl_p.name, f16=True))
        full["rows"] = rows
        result["rows"] = len(rows)

    # ---- CPU oracle on the host cores (headline workload) ----
    if cpu:
        import oracle
        log("cpu baseline (oracle)")
        threads = oracle.default_threads()
        runs, el = cpu_time(lambda: oracle.qmm(inp.x, "bf16", inp.packed, inp.scales, inp.biases,
                                               wl.group_size, wl.bits, threads=threads), 10.0, 100000)
        result["cpu_baseline"] = {
            "value": round(row["bytes_per_step"] * runs / el / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "sample": f"the whole decode step, {runs} runs in {el:.1f} s"}
    else:
        result["cpu_baseline"] = None

    if metrics is not None:
        metrics.close()
    if args.full_out:
        full["summary"] = result
        with open(args.full_out, "w") as f:
            json.dump(full, f, indent=1)
    # the per-row records went to stderr above (and to --full-out); the one result line stays short
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
