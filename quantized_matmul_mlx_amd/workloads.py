"""Seeded synthetic inputs for grouped affine quantized weights.

This module only draws random numbers. It holds none of the method's arithmetic: it does not
pack, unpack, dequantize, multiply or round results. Both the HIP path and the CPU oracle are
fed from it, and neither imports the other.

Conventions
-----------
* Packed codes are drawn as uniform random ``uint32`` words. Every bit of a uniform word is an
  independent fair coin, so every code of every width read out of those words is uniform over
  ``[0, 2**bits - 1]`` and independent of the others. No packing step is needed to produce
  "codes uniform in [0, 2^bits-1]" at any bit width.
* bf16 values are carried as ``uint16`` bit patterns. A bf16 input is a float32 draw with its low
  16 bits dropped (truncation toward zero). The generator therefore shares no rounding code with
  either side.
* The generator is ``numpy.random.default_rng(seed)`` (PCG64), a fresh one per (config, M). The
  draw order is packed words, scales, biases, x, then indices, so W is identical for every M of
  a config.

The configurations are the MLX-layout workloads used for parity and for the benchmark: a small
4-bit reference case, the 4096x4096 4-bit decode GEMV, an 8-bit 14336x4096 GEMV, the 4-bit
group-128 prefill GEMM, 3- and 6-bit group-32 odd widths, a gathered-row embedding table, a decode
FFN step and a mixture-of-experts layer.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    bits: int
    group_size: int
    n: int                      # out features (rows of W)
    k: int                      # in features (columns of W)
    scale_range: tuple          # uniform range of the bf16 scales
    bias_range: tuple           # uniform range of the bf16 biases
    ms: tuple = ()              # rows of x at which qmm runs
    x_dtype: str = "bf16"       # "bf16" or "f32"
    n_indices: int = 0          # gathered-row lookups (embedding table workloads)
    seed: int = 0
    experts: int = 0            # weight batches of a gathered (mixture-of-experts) product
    top_k: int = 0              # experts per token

    @property
    def packed_cols(self) -> int:
        return self.k * self.bits // 32

    @property
    def groups(self) -> int:
        return self.k // self.group_size


WORKLOADS = {
    # 4-bit g64, W [256, 512], fp32 x [4, 512]: small enough for exhaustive oracle comparison.
    "ref_4bit_g64_256x512": Workload("ref_4bit_g64_256x512", 4, 64, 256, 512,
                                     (1e-3, 5e-2), (-0.4, 0.0), ms=(4,), x_dtype="f32"),
    # Decode GEMV: 4-bit g64, W [4096, 4096], bf16 x at M = 1 and M = 4.
    "decode_4bit_g64_4096x4096": Workload("decode_4bit_g64_4096x4096", 4, 64, 4096, 4096,
                                          (1e-3, 2e-2), (-0.15, 0.0), ms=(1, 4)),
    # 8-bit g64 (byte packed, low byte = column 0), W [14336, 4096], M = 1 and M = 8.
    "int8_g64_14336x4096": Workload("int8_g64_14336x4096", 8, 64, 14336, 4096,
                                    (1e-4, 2e-3), (-0.15, 0.0), ms=(1, 8)),
    # Prefill GEMM: 4-bit g128, W [4096, 14336], bf16 x [2048, 14336].
    "prefill_4bit_g128_4096x14336": Workload("prefill_4bit_g128_4096x14336", 4, 128, 4096, 14336,
                                             (1e-3, 2e-2), (-0.15, 0.0), ms=(2048,)),
    # A prefill GEMM whose K is not a whole number of 1024 codes: a down projection of an FFN with
    # 11008 hidden units, 4-bit g128, W [4096, 11008], bf16 x [2048, 11008].
    "prefill_4bit_g128_4096x11008": Workload("prefill_4bit_g128_4096x11008", 4, 128, 4096, 11008,
                                             (1e-3, 2e-2), (-0.15, 0.0), ms=(2048,), seed=61),
    # Odd widths g32: codes straddle uint32 boundaries. W [11008, 4096], M = 1 and M = 16.
    "odd_3bit_g32_11008x4096": Workload("odd_3bit_g32_11008x4096", 3, 32, 11008, 4096,
                                        (1e-3, 2e-2), (-0.15, 0.0), ms=(1, 16)),
    "odd_6bit_g32_11008x4096": Workload("odd_6bit_g32_11008x4096", 6, 32, 11008, 4096,
                                        (1e-3, 2e-2), (-0.15, 0.0), ms=(1, 16)),
    # A decode FFN step at 4-bit g64 (the fused products): gate and up [14336, 4096] on one x row,
    # then down [4096, 14336] on silu(gate) * up plus the residual.
    "ffn_gate_4bit_g64_14336x4096": Workload("ffn_gate_4bit_g64_14336x4096", 4, 64, 14336, 4096,
                                             (1e-3, 2e-2), (-0.15, 0.0), ms=(1,), seed=31),
    "ffn_up_4bit_g64_14336x4096": Workload("ffn_up_4bit_g64_14336x4096", 4, 64, 14336, 4096,
                                           (1e-3, 2e-2), (-0.15, 0.0), ms=(1,), seed=32),
    "ffn_down_4bit_g64_4096x14336": Workload("ffn_down_4bit_g64_4096x14336", 4, 64, 4096, 14336,
                                             (1e-3, 2e-2), (-0.15, 0.0), ms=(1,), seed=33),
    # Embedding table: 4-bit g64 [32768, 4096], 4096 uniform-random gathered rows.
    "rows_4bit_g64_32768x4096": Workload("rows_4bit_g64_32768x4096", 4, 64, 32768, 4096,
                                         (1e-3, 2e-2), (-0.15, 0.0), n_indices=4096),
    # Quantization of a dense bf16 weight [4096, 4096] ~ N(0, 0.02^2) to 4-bit g64 (the decode shape).
    "quantize_4bit_g64_4096x4096": Workload("quantize_4bit_g64_4096x4096", 4, 64, 4096, 4096,
                                            (0.0, 0.0), (0.0, 0.0), seed=51),
    # Mixture of experts (gathered products): 128 experts of W [768, 2048] at 4-bit g64, 8 experts
    # per token; 1 token (a single decode step) and 64 tokens (a decode batch), rows sorted by expert.
    "moe_4bit_g64_e128_768x2048": Workload("moe_4bit_g64_e128_768x2048", 4, 64, 768, 2048,
                                           (1e-3, 2e-2), (-0.15, 0.0), ms=(1, 64), seed=41,
                                           experts=128, top_k=8),
    # The same layer at prefill: 2048 tokens (16384 rows, about 128 per expert).
    "moe_prefill_4bit_g64_e128_768x2048": Workload("moe_prefill_4bit_g64_e128_768x2048", 4, 64, 768, 2048,
                                                   (1e-3, 2e-2), (-0.15, 0.0), ms=(2048,), seed=42,
                                                   experts=128, top_k=8),
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 draw -> bf16 bit pattern by dropping the low half (truncation toward zero)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def f32_from_bf16_bits(h: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> float32 holding the same value (a reinterpretation, no rounding)."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    """One draw of a workload. Arrays are host numpy arrays, C-contiguous.

    packed  uint32 [n, k*bits/32]
    scales  uint16 (bf16 bits) [n, k/group_size]
    biases  uint16 (bf16 bits) [n, k/group_size]
    x       uint16 (bf16 bits) or float32 [m, k]   (None when m == 0 was not asked for)
    indices uint32 [n_indices]                     (None for matmul workloads)
    """
    wl: Workload
    packed: np.ndarray
    scales: np.ndarray
    biases: np.ndarray
    x: Optional[np.ndarray]
    x_dtype: str
    indices: Optional[np.ndarray]


def draw_weights(rng: np.random.Generator, n: int, k: int, bits: int, group_size: int,
                 scale_range, bias_range):
    packed = rng.integers(0, 2**32, size=(n, k * bits // 32), dtype=np.uint32)
    g = k // group_size
    scales = bf16_bits_from_f32(rng.uniform(scale_range[0], scale_range[1], (n, g)).astype(np.float32))
    biases = bf16_bits_from_f32(rng.uniform(bias_range[0], bias_range[1], (n, g)).astype(np.float32))
    return packed, scales, biases


def draw_x(rng: np.random.Generator, m: int, k: int, x_dtype: str) -> np.ndarray:
    x = rng.standard_normal((m, k), dtype=np.float32)
    if x_dtype == "bf16":
        return bf16_bits_from_f32(x)
    if x_dtype == "f32":
        return x
    raise ValueError(f"unknown x dtype {x_dtype!r}")


def make_inputs(wl: Workload, m: int = 0, n: Optional[int] = None, k: Optional[int] = None,
                x_dtype: Optional[str] = None, seed: Optional[int] = None) -> Inputs:
    """Draw a workload's inputs. ``n``/``k`` override the sizes (same distributions), which is
    how the parity tests build reduced shapes that still span several tiles and a ragged tail."""
    n = wl.n if n is None else n
    k = wl.k if k is None else k
    x_dtype = wl.x_dtype if x_dtype is None else x_dtype
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    packed, scales, biases = draw_weights(rng, n, k, wl.bits, wl.group_size,
                                          wl.scale_range, wl.bias_range)
    x = draw_x(rng, m, k, x_dtype) if m > 0 else None
    idx = None
    if wl.n_indices:
        idx = rng.integers(0, n, size=wl.n_indices, dtype=np.uint32)
    return Inputs(wl, packed, scales, biases, x, x_dtype, idx)


def random_inputs(bits: int, group_size: int, n: int, k: int, m: int, x_dtype: str = "bf16",
                  seed: int = 0, scale_range=(1e-3, 2e-2), bias_range=(-0.15, 0.0)) -> Inputs:
    """Inputs of arbitrary shape with the decode workload's distributions."""
    wl = Workload(f"random_{bits}bit_g{group_size}_{n}x{k}", bits, group_size, n, k,
                  scale_range, bias_range, ms=(m,), x_dtype=x_dtype, seed=seed)
    return make_inputs(wl, m=m)


@dataclasses.dataclass
class MoeInputs:
    """One draw of a mixture-of-experts workload, rows grouped by expert.

    packed  uint32 [experts, n, k*bits/32];  scales, biases uint16 (bf16 bits) [experts, n, k/G]
    x       uint16 (bf16 bits) [tokens, k]: the tokens' activations
    token   uint32 [rows]: the token of each row (rows = tokens * top_k), in expert order
    expert  uint32 [rows]: the expert of each row, non-decreasing
    x_rows  uint16 [rows, 1, k]: x[token], the product's input with its rows in expert order
    """
    wl: Workload
    packed: np.ndarray
    scales: np.ndarray
    biases: np.ndarray
    x: np.ndarray
    token: np.ndarray
    expert: np.ndarray
    x_rows: np.ndarray


def moe_inputs(wl: Workload, tokens: int, experts: Optional[int] = None, n: Optional[int] = None,
               k: Optional[int] = None, seed: Optional[int] = None) -> MoeInputs:
    """Experts' weights, token activations and a random routing: each token picks top_k distinct
    experts uniformly (a stand-in for a router's choice); the (token, expert) rows are then ordered
    by expert, ties by token, as a layer does before a sorted gathered product."""
    E = wl.experts if experts is None else experts
    n = wl.n if n is None else n
    k = wl.k if k is None else k
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    packed, scales, biases = draw_weights(rng, E * n, k, wl.bits, wl.group_size, wl.scale_range, wl.bias_range)
    x = draw_x(rng, tokens, k, "bf16")
    choice = np.argsort(rng.random((tokens, E)), axis=1)[:, :min(wl.top_k, E)]
    tok = np.repeat(np.arange(tokens, dtype=np.uint32), choice.shape[1])
    exp = choice.reshape(-1).astype(np.uint32)
    order = np.lexsort((tok, exp))
    tok, exp = tok[order], exp[order]
    return MoeInputs(wl, packed.reshape(E, n, -1), scales.reshape(E, n, -1), biases.reshape(E, n, -1), x,
                     tok, exp, x[tok][:, None, :])


def dense_weight(rows: int, cols: int, dtype: str = "bf16", std: float = 0.02, seed: int = 0) -> np.ndarray:
    """A dense weight ~ N(0, std^2) to quantize: float32, or bf16 bit patterns (truncated draws)."""
    w = (np.random.default_rng(seed).standard_normal((rows, cols), dtype=np.float32) * np.float32(std))
    return bf16_bits_from_f32(w) if dtype == "bf16" else w
