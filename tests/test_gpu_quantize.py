"""Quantization on the GPU against the CPU oracle, through the C ABI (via the binding).

Codes are integers and scales and biases values of their stored type (bias = group min and scale =
(max - min) / (2^bits - 1), float32 statistics stored as bf16, float16 or float32; code =
round-half-away of the exact value of (w - bias) / scale, clamped): the bar is bit-exact for all
three outputs, for float32, bf16 and float16 weights.
"""
import numpy as np
import pytest
import torch

import oracle as orc_mod
from gpu_util import banner, dev_bf16, dev_u32, dev_x, host_bits
from near_ties import bf16_rne, bf16_value, f16_value, f32_value, near_tie_groups, tie_example
from quantized_matmul_mlx_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    orc_mod.build()
    import quantized_matmul_mlx_amd as q
    q._lib.load()
    return orc_mod


def qaff():
    import quantized_matmul_mlx_amd as q
    return q


TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def run(w, dtype, G, bits, sb="bf16"):
    wd = dev_x(w, dtype)
    p, s, b = qaff().quantize(wd, G, bits, scales_dtype=TORCH[sb])
    torch.cuda.synchronize()
    return (p.cpu().numpy().view(np.uint32), host_bits(s), host_bits(b))


def check(orc, w, dtype, G, bits, sb="bf16"):
    got = run(w, dtype, G, bits, sb)
    ref = orc.quantize(w, dtype, G, bits, sb)
    for name, g, r in zip(("packed", "scales", "biases"), got, ref):
        assert g.shape == r.shape, name
        if g.dtype == np.float32:   # float32 scales: compare the bit patterns
            g, r = g.view(np.uint32), r.view(np.uint32)
        if not np.array_equal(g, r):
            bad = np.argwhere(g != r)[:5]
            raise AssertionError(f"{name} differs at {bad.tolist()}: got {g[tuple(bad[0])]:#x}, "
                                 f"oracle {r[tuple(bad[0])]:#x}")
    return got


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_quantize_bit_exact(orc, dtype, bits, G):
    # 37 rows (a ragged last thread block) of 5 groups
    w = W.dense_weight(37, 5 * G, dtype, seed=bits * 10 + G)
    banner(f"quantize {dtype} bits={bits} G={G}")
    check(orc, w, dtype, G, bits)


@pytest.mark.parametrize("bits,G", [(4, 64), (3, 32), (8, 128)])
def test_quantize_special_groups(orc, bits, G):
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((6, 4 * G)) * 0.5).astype(np.float32)
    w[0, :G] = 0.75                               # constant group: scale 0, code 0
    w[1, :] = 0.0                                 # all zero
    w[1, G:2 * G:2] = -0.0                        # +0 and -0 mixed: the first of equal minima
    w[2, :G] = np.round(w[2, :G] * 8) / 8         # many values on a coarse grid: exact ties
    w[3, G:2 * G] = np.linspace(1.005, 1.9, G)    # the stored bias rounds above the minimum
    w[4, :G] = np.where(np.arange(G) % 2, 1e30, -1e30)   # a huge range
    w[5, :G] = np.arange(G) * 2.0 ** -20          # a tiny range
    banner(f"quantize special groups bits={bits} G={G}")
    check(orc, w, "f32", G, bits)
    check(orc, W.bf16_bits_from_f32(w), "bf16", G, bits)


def test_quantize_exact_difference_decides_a_tie(orc):
    # w - bias is not a float32 here; the exact quotients 3.5 - 2^-96 and 5.5 - 2^-96 round to 3
    # and 5 (a float32 difference would land on the ties and give 4 and 6)
    banner("quantize tie decided by the exact difference")
    got = check(orc, tie_example(), "f32", 32, 4)
    assert list(orc.unpack_codes(got[0], 32, 4)[0, :4]) == [0, 15, 3, 5]


@pytest.mark.parametrize("bits,G", [(4, 64), (3, 32), (8, 128), (1, 32), (6, 64), (2, 128), (5, 32)])
def test_quantize_near_ties(orc, bits, G):
    # values within a few ulps of every boundary bias + (k + 1/2) scale, minima of very different
    # magnitudes: the exact decision on both sides
    w = near_tie_groups(40, 3, G, bits, seed=300 + bits)
    banner(f"quantize near ties bits={bits} G={G}")
    check(orc, w, "f32", G, bits)
    check(orc, bf16_rne(w), "bf16", G, bits)


def test_quantize_round_trip_through_qmm(orc):
    # quantize -> qmm on the GPU against the oracle's qmm of the oracle's quantization
    w = W.dense_weight(300, 1024, "bf16", seed=3)
    banner("quantize then qmm")
    q = qaff()
    p, s, b = q.quantize(dev_bf16(w), 64, 4)
    x = W.bf16_bits_from_f32(np.random.default_rng(4).standard_normal((4, 1024)).astype(np.float32))
    y = q.qmm(dev_bf16(x), p, s, b, 64, 4)
    torch.cuda.synchronize()
    rp, rs, rb = orc.quantize(w, "bf16", 64, 4)
    ref = orc.qmm(x, "bf16", rp, rs, rb, 64, 4)
    assert orc.max_row_rel_err(y.float().cpu().numpy().astype(np.float64), ref) <= 1.6e-2


def test_quantize_leading_dims_and_empty(orc):
    w = W.dense_weight(6, 128, "f32", seed=5).reshape(2, 3, 128)
    banner("quantize leading dims")
    p, s, b = qaff().quantize(dev_x(w, "f32"), 32, 4, scales_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert tuple(p.shape) == (2, 3, 16) and tuple(s.shape) == (2, 3, 4)
    rp, rs, rb = orc.quantize(w.reshape(6, 128), "f32", 32, 4)
    np.testing.assert_array_equal(p.cpu().numpy().view(np.uint32).reshape(6, 16), rp)
    np.testing.assert_array_equal(host_bits(s).reshape(6, 4), rs)
    e = qaff().quantize(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"), 64, 4)
    assert tuple(e[0].shape) == (0, 8)


def test_quantize_workload_full_size(orc):
    wl = W.WORKLOADS["quantize_4bit_g64_4096x4096"]
    w = W.dense_weight(wl.n, wl.k, "bf16", seed=wl.seed)
    banner("quantize 4096x4096 bf16 4-bit g64")
    check(orc, w, "bf16", wl.group_size, wl.bits)


# ---- float16 weights, and scales and biases in float32 or float16 ----------------------------------

def f16_bits(w32):
    return np.asarray(w32, np.float32).astype(np.float16).view(np.uint16)


def as_input(w32, dtype):
    return {"f32": lambda a: np.asarray(a, np.float32), "bf16": W.bf16_bits_from_f32, "f16": f16_bits}[dtype](w32)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("sb", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("bits,G", [(4, 64), (3, 32), (8, 128), (1, 32), (6, 128)])
def test_quantize_typed_bit_exact(orc, dtype, sb, bits, G):
    # 37 rows of 5 groups; scales and biases stored as sb
    w = as_input(W.dense_weight(37, 5 * G, "f32", seed=bits * 10 + G), dtype)
    banner(f"quantize {dtype} -> scales {sb} bits={bits} G={G}")
    check(orc, w, dtype, G, bits, sb)


@pytest.mark.parametrize("dtype,sb", [("f32", "f32"), ("f16", "f16"), ("f32", "f16"), ("bf16", "f16"),
                                      ("f16", "f32"), ("f16", "bf16")])
@pytest.mark.parametrize("bits,G", [(4, 64), (3, 32), (8, 128), (1, 32), (5, 32)])
def test_quantize_typed_near_ties(orc, dtype, sb, bits, G):
    # values within a few ulps of the boundaries of the stored scale and bias
    stored = {"f32": f32_value, "bf16": bf16_value, "f16": f16_value}[sb]
    w = near_tie_groups(40, 3, G, bits, seed=400 + bits, w_type=np.float16 if dtype == "f16" else np.float32,
                        stored=stored)
    wi = {"f32": w, "f16": w.view(np.uint16) if w.dtype == np.float16 else w, "bf16": bf16_rne(w)}[dtype]
    banner(f"quantize near ties {dtype} -> scales {sb} bits={bits} G={G}")
    check(orc, wi, dtype, G, bits, sb)


def test_quantize_float32_scale_exact_quotient_below_a_tie(orc):
    # scale 1 + 2^-20 (min 0, max 15 scale): values just below (k + 1/2) scale whose float32
    # quotient lands on the tie round down (see the oracle pin of the same case)
    s = np.float32(1.0 + 2.0 ** -20)
    w = np.zeros((1, 32), np.float32)
    w[0, 1] = np.float32(15.0 * (1.0 + 2.0 ** -20))
    for i, k in enumerate(range(1, 15)):
        v = np.float32((k + 0.5) * float(s))
        if np.float64(v) >= (k + 0.5) * float(s):
            v = np.nextafter(v, np.float32(-np.inf))
        w[0, 2 + i] = v
    banner("quantize float32 scale near a tie")
    got = check(orc, w, "f32", 32, 4, "f32")
    assert got[1][0, 0] == s


def test_quantize_default_scales_dtype_is_w_dtype(orc):
    w = W.dense_weight(4, 128, "f32", seed=9)
    q = qaff()
    for dtype, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16), ("f16", torch.float16)):
        banner(f"quantize default scales dtype {dtype}")
        p, s, b = q.quantize(dev_x(as_input(w, dtype), dtype), 64, 4)
        torch.cuda.synchronize()
        assert s.dtype == tdt and b.dtype == tdt
        rp, rs, rb = orc.quantize(as_input(w, dtype), dtype, 64, 4, dtype)
        np.testing.assert_array_equal(p.cpu().numpy().view(np.uint32), rp)
