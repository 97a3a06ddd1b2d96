"""Pins for the CPU oracle: what the pages print and what mathematics fixes.

The oracle is only trusted as far as these tests pin it. Each check is chosen so that a plausible
mistake fails it: MSB-first reading, a subtracted bias, swapped scale and bias, a wrong group
index, a straddling code read from the wrong word, a dropped term or transposed operand in the
matmul, a wrong rounding of bf16 outputs.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import golden
from near_ties import bf16_rne, bf16_value, f16_value, f32_value, near_tie_groups, tie_example
from quantized_matmul_mlx_amd import workloads as W


def _words(tokens):
    return np.array([int(t, 16) for t in tokens], np.uint32)


def _bf16(v):
    """bf16 bits of a value that bf16 holds exactly (the value's float32 upper half)."""
    a = np.array([v], np.float32).view(np.uint32) >> 16
    assert (np.array([v], np.float32).view(np.uint32) & 0xFFFF) == 0, "not exact in bf16"
    return a.astype(np.uint16)


# ---- printed examples ---------------------------------------------------------------------

def test_worked_example_lsb_first_plus_bias(oracle_lib):
    g = golden("lsb_first_plus_bias.txt")
    bits, G, cols = int(g["bits"][0]), int(g["group_size"][0]), int(g["cols"][0])
    packed = _words(g["packed"]).reshape(1, -1)
    s = _bf16(float(g["scale"][0])).reshape(1, 1)
    b = _bf16(float(g["bias"][0])).reshape(1, 1)
    out = oracle_lib.dequantize(packed, s, b, G, bits, cols=cols)
    expect = np.array([float(t) for t in g["expect"]], np.float32)
    np.testing.assert_array_equal(out[0], expect)
    # The readings the page calls wrong: MSB-first codes, or the bias subtracted.
    msb_first = 2.0 * np.arange(7, -1, -1) - 1.0
    minus_bias = 2.0 * np.arange(8) + 1.0
    assert not np.array_equal(out[0], msb_first)
    assert not np.array_equal(out[0], minus_bias)


def test_worked_example_at_group_32(oracle_lib):
    """The same word repeated over a 32-column group (the smallest group the library takes)."""
    packed = np.full((1, 4), 0x76543210, np.uint32)
    out = oracle_lib.dequantize(packed, _bf16(2.0).reshape(1, 1), _bf16(-1.0).reshape(1, 1), 32, 4)
    np.testing.assert_array_equal(out[0], np.tile(2.0 * np.arange(8) - 1.0, 4).astype(np.float32))


def test_identity_shape(oracle_lib):
    g = golden("identity_shape.txt")
    bits, G, cols = int(g["bits"][0]), int(g["group_size"][0]), int(g["cols"][0])
    packed = _words(g["packed"]).reshape(1, -1)
    out = oracle_lib.dequantize(packed, _bf16(1.0).reshape(1, 1), _bf16(0.0).reshape(1, 1), G, bits,
                                cols=cols)
    assert out.shape == (1, cols)
    np.testing.assert_array_equal(out[0], np.array([float(t) for t in g["expect"]], np.float32))


def test_int8_byte_order(oracle_lib):
    g = golden("int8_byte_order.txt")
    bits, cols = int(g["bits"][0]), int(g["cols"][0])
    packed = _words(g["packed"]).reshape(1, -1)
    codes = oracle_lib.unpack_codes(packed, cols, bits)
    np.testing.assert_array_equal(codes[0], np.array([int(t) for t in g["codes"]], np.uint8))
    np.testing.assert_array_equal(oracle_lib.pack_codes(codes, bits), packed)


def test_shape_rule(oracle_lib):
    g = golden("shape_rule.txt")
    bits, G = int(g["bits"][0]), int(g["group_size"][0])
    n, k = (int(t) for t in g["w_shape"])
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 2**bits, (n, k), dtype=np.uint8)
    packed = oracle_lib.pack_codes(codes, bits)
    assert list(packed.shape) == [int(t) for t in g["packed_shape"]]
    scales = np.full([int(t) for t in g["scales_shape"]], _bf16(0.5)[0], np.uint16)
    biases = np.full([int(t) for t in g["scales_shape"]], _bf16(-1.0)[0], np.uint16)
    assert oracle_lib.dequantize(packed, scales, biases, G, bits).shape == (n, k)
    x = np.ones([int(t) for t in g["x_shape"]], np.float32)
    y = oracle_lib.qmm(x, "f32", packed, scales, biases, G, bits)
    assert list(y.shape) == [int(t) for t in g["y_shape"]]


def test_odd_width_3bit_hand_words(oracle_lib):
    g = golden("odd_width_3bit.txt")
    bits, cols = int(g["bits"][0]), int(g["cols"][0])
    words = _words(g["packed"]).reshape(1, -1)
    codes = np.array([int(t) for t in g["codes"]], np.uint8).reshape(1, -1)
    np.testing.assert_array_equal(oracle_lib.pack_codes(codes, bits), words)
    np.testing.assert_array_equal(oracle_lib.unpack_codes(words, cols, bits), codes)


# ---- the bit stream, from an independent formulation ----------------------------------------

def _row_int(codes, bits):
    """A row as one little-endian integer: code j times 2**(bits*j)."""
    v = 0
    for j, c in enumerate(codes):
        v += int(c) << (bits * j)
    return v


def _int_words(v, nwords):
    return [(v >> (32 * i)) & 0xFFFFFFFF for i in range(nwords)]


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
def test_bit_stream_matches_big_integer(oracle_lib, bits):
    rng = np.random.default_rng(bits)
    cols = 32 * 5
    codes = rng.integers(0, 2**bits, (3, cols), dtype=np.uint8)
    packed = oracle_lib.pack_codes(codes, bits)
    for r in range(3):
        assert packed[r].tolist() == _int_words(_row_int(codes[r], bits), cols * bits // 32)
    # and the other way: random words read as one integer
    words = rng.integers(0, 2**32, (2, cols * bits // 32), dtype=np.uint32)
    got = oracle_lib.unpack_codes(words, cols, bits)
    for r in range(2):
        v = sum(int(w) << (32 * i) for i, w in enumerate(words[r]))
        assert got[r].tolist() == [(v >> (bits * j)) & ((1 << bits) - 1) for j in range(cols)]


@pytest.mark.parametrize("bits", [2, 3, 5, 6])
def test_straddling_positions(oracle_lib, bits):
    """A lone code of all ones at each index j sets exactly stream bits [j*bits, (j+1)*bits);
    the codes that cross a word boundary are exactly those with (j*bits) % 32 + bits > 32."""
    for j in range(32):
        codes = np.zeros((1, 32), np.uint8)
        codes[0, j] = 2**bits - 1
        v = sum(int(w) << (32 * i) for i, w in enumerate(oracle_lib.pack_codes(codes, bits)[0]))
        assert v == ((1 << bits) - 1) << (j * bits)
    straddle = [j for j in range(32) if (j * bits) % 32 + bits > 32]
    expect = {2: [], 3: [10, 21], 5: [6, 12, 19, 25], 6: [5, 10, 21, 26]}[bits]
    assert straddle == expect


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
def test_pack_unpack_round_trip(oracle_lib, bits):
    rng = np.random.default_rng(10 + bits)
    codes = rng.integers(0, 2**bits, (4, 256), dtype=np.uint8)
    np.testing.assert_array_equal(oracle_lib.unpack_codes(oracle_lib.pack_codes(codes, bits), 256, bits), codes)


# ---- the affine rule -------------------------------------------------------------------------

@pytest.mark.parametrize("bits,G", [(2, 32), (3, 32), (4, 64), (5, 128), (6, 32), (8, 64), (8, 128)])
def test_dequant_is_one_rounding_of_exact_affine(oracle_lib, bits, G):
    """Invariant: a bf16 scale (8 significant bits) times a code of at most 8 bits is exact in
    float32, so scale*code + bias equals the exact value rounded once to float32. The codes are
    read through the big-integer formulation, the group as column // G."""
    n, k = 5, 4 * G
    inp = W.random_inputs(bits, G, n, k, 0, seed=bits * 1000 + G)
    got = oracle_lib.dequantize(inp.packed, inp.scales, inp.biases, G, bits)
    s = W.f32_from_bf16_bits(inp.scales).astype(np.float64)
    b = W.f32_from_bf16_bits(inp.biases).astype(np.float64)
    for r in range(n):
        v = sum(int(w) << (32 * i) for i, w in enumerate(inp.packed[r]))
        codes = np.array([(v >> (bits * j)) & ((1 << bits) - 1) for j in range(k)], np.float64)
        grp = np.arange(k) // G
        exact = s[r, grp] * codes + b[r, grp]   # exact in float64: <= 16-bit product, 8-bit addend
        np.testing.assert_array_equal(got[r], exact.astype(np.float32))


def test_scale_and_bias_not_swapped(oracle_lib):
    # code 3 with scale 0.5 and bias 4: 0.5*3 + 4 = 5.5; swapped would give 4*3 + 0.5 = 12.5
    packed = np.array([[0x33333333] * 4], np.uint32)
    out = oracle_lib.dequantize(packed, _bf16(0.5).reshape(1, 1), _bf16(4.0).reshape(1, 1), 32, 4)
    np.testing.assert_array_equal(out, np.full((1, 32), 5.5, np.float32))


def test_group_index_per_column(oracle_lib):
    # two groups of 32 with different scales: columns 0..31 use scale 1, 32..63 use scale 3
    packed = np.full((1, 8), 0x11111111, np.uint32)        # every code 1
    s = np.concatenate([_bf16(1.0), _bf16(3.0)]).reshape(1, 2)
    b = np.concatenate([_bf16(0.0), _bf16(0.25)]).reshape(1, 2)
    out = oracle_lib.dequantize(packed, s, b, 32, 4)
    np.testing.assert_array_equal(out[0, :32], 1.0)
    np.testing.assert_array_equal(out[0, 32:], 3.25)


def test_rejects_parameters_outside_the_format(oracle_lib):
    with pytest.raises(ValueError):
        oracle_lib.dequantize(np.zeros((1, 4), np.uint32), np.zeros((1, 1), np.uint16),
                              np.zeros((1, 1), np.uint16), 24, 4, cols=32)


# ---- bf16 rounding ----------------------------------------------------------------------------

def test_bf16_rne_known_values(oracle_lib):
    cases = {
        0x3F800000: 0x3F80,   # 1.0 exact
        0x3F808000: 0x3F80,   # midpoint, even neighbour below
        0x3F818000: 0x3F82,   # midpoint, odd below -> up
        0x3F808001: 0x3F81,   # just above the midpoint
        0x3F807FFF: 0x3F80,   # just below the midpoint
        0xBF808001: 0xBF81,   # sign is carried
        0x80000000: 0x8000,   # -0.0
        0x7F7FFFFF: 0x7F80,   # largest finite rounds to +inf
        0x7F800000: 0x7F80,   # +inf
        0x00000001: 0x0000,   # smallest subnormal rounds to zero
        0x007FFFFF: 0x0080,   # largest subnormal rounds up to the smallest normal
    }
    a = np.array(list(cases), np.uint32).view(np.float32)
    got = oracle_lib.f32_to_bf16(a)
    assert [hex(v) for v in got.tolist()] == [hex(v) for v in cases.values()]
    nan = oracle_lib.f32_to_bf16(np.array([0x7F800001, 0xFFC00000], np.uint32).view(np.float32))
    assert np.isnan(W.f32_from_bf16_bits(nan)).all()


def test_bf16_rne_matches_torch(oracle_lib):
    rng = np.random.default_rng(3)
    a = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        rng.integers(0, 2**32, 200000, dtype=np.uint32).view(np.float32)])
    a = a[np.isfinite(a)]
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle_lib.f32_to_bf16(a), ref)


def test_bf16_widening_is_exact(oracle_lib):
    h = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    f = oracle_lib.bf16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(f.view(np.uint32), ref.view(np.uint32))


# ---- the matmul --------------------------------------------------------------------------------

def _exact(v):
    return Fraction(float(v))


@pytest.mark.parametrize("bits,G,k,x_dtype", [(4, 32, 64, "f32"), (3, 32, 32, "bf16"),
                                              (8, 64, 64, "bf16"), (2, 32, 64, "f32")])
def test_qmm_brute_force_exact_rationals(oracle_lib, bits, G, k, x_dtype):
    m, n = 3, 4
    inp = W.random_inputs(bits, G, n, k, m, x_dtype=x_dtype, seed=7 + bits)
    w = oracle_lib.dequantize(inp.packed, inp.scales, inp.biases, G, bits)
    xf = W.f32_from_bf16_bits(inp.x) if x_dtype == "bf16" else inp.x
    y = oracle_lib.qmm(inp.x, x_dtype, inp.packed, inp.scales, inp.biases, G, bits)
    for i in range(m):
        for j in range(n):
            exact = sum(_exact(xf[i, t]) * _exact(w[j, t]) for t in range(k))
            denom = max(abs(exact), Fraction(1, 10**9))
            assert abs(Fraction(float(y[i, j])) - exact) / denom < Fraction(1, 10**12)


@pytest.mark.parametrize("bits,G", [(4, 64), (6, 32), (8, 128)])
def test_qmm_matches_float64_matmul(oracle_lib, bits, G):
    inp = W.random_inputs(bits, G, 37, 256, 5, x_dtype="bf16", seed=bits)
    w = oracle_lib.dequantize(inp.packed, inp.scales, inp.biases, G, bits).astype(np.float64)
    x = W.f32_from_bf16_bits(inp.x).astype(np.float64)
    y = oracle_lib.qmm(inp.x, "bf16", inp.packed, inp.scales, inp.biases, G, bits)
    np.testing.assert_allclose(y, x @ w.T, rtol=1e-12, atol=1e-12)


def test_qmm_one_hot_selects_a_column(oracle_lib):
    bits, G, n, k = 4, 64, 9, 128
    inp = W.random_inputs(bits, G, n, k, 0, seed=5)
    w = oracle_lib.dequantize(inp.packed, inp.scales, inp.biases, G, bits)
    x = np.zeros((3, k), np.float32)
    cols = [0, 77, 127]
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    y = oracle_lib.qmm(x, "f32", inp.packed, inp.scales, inp.biases, G, bits)
    for i, c in enumerate(cols):
        np.testing.assert_array_equal(y[i], w[:, c].astype(np.float64))


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_qmm_closed_forms(oracle_lib, bits):
    G, n, k = 32, 6, 128
    inp = W.random_inputs(bits, G, n, k, 2, x_dtype="f32", seed=11)
    s = W.f32_from_bf16_bits(inp.scales).astype(np.float64)
    b = W.f32_from_bf16_bits(inp.biases).astype(np.float64)
    xg = inp.x.astype(np.float64).reshape(2, k // G, G).sum(-1)        # [m, groups]
    # every code zero: y = sum_g b_g * sum_{k in g} x_k
    zeros = np.zeros_like(inp.packed)
    y0 = oracle_lib.qmm(inp.x, "f32", zeros, inp.scales, inp.biases, G, bits)
    np.testing.assert_allclose(y0, xg @ b.T, rtol=1e-12, atol=1e-12)
    # every code at its maximum, x = 1: y = sum_g G * (s_g * (2^bits - 1) + b_g)
    ones_w = np.full_like(inp.packed, 0xFFFFFFFF)
    x1 = np.ones((1, k), np.float32)
    y1 = oracle_lib.qmm(x1, "f32", ones_w, inp.scales, inp.biases, G, bits)
    w_max = (s * (2**bits - 1) + b).astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(y1[0], G * w_max.sum(-1), rtol=1e-12)


def test_qmm_is_linear_in_x(oracle_lib):
    bits, G = 5, 32
    inp = W.random_inputs(bits, G, 7, 96, 2, x_dtype="f32", seed=13)
    y = oracle_lib.qmm(inp.x, "f32", inp.packed, inp.scales, inp.biases, G, bits)
    x2 = np.ascontiguousarray((inp.x[0:1] + inp.x[1:2]).astype(np.float32))
    y2 = oracle_lib.qmm(x2, "f32", inp.packed, inp.scales, inp.biases, G, bits)
    # float32 rounding of x0 + x1 is the only difference; compare loosely
    np.testing.assert_allclose(y2[0], y[0] + y[1], rtol=1e-5, atol=1e-5)


def test_qmm_empty_shapes(oracle_lib):
    inp = W.random_inputs(4, 32, 3, 64, 0)
    y = oracle_lib.qmm(np.zeros((0, 64), np.uint16), "bf16", inp.packed, inp.scales, inp.biases, 32, 4)
    assert y.shape == (0, 3)


# ---- gathered rows -----------------------------------------------------------------------------

def test_dequant_rows_identity_and_gather(oracle_lib):
    bits, G, rows, cols = 4, 64, 40, 256
    inp = W.random_inputs(bits, G, rows, cols, 0, seed=17)
    full = oracle_lib.dequantize(inp.packed, inp.scales, inp.biases, G, bits)
    same = oracle_lib.dequant_rows(inp.packed, inp.scales, inp.biases, np.arange(rows), G, bits)
    np.testing.assert_array_equal(same.view(np.uint32), full.view(np.uint32))
    idx = np.array([39, 0, 5, 5, 17], np.uint32)
    got = oracle_lib.dequant_rows(inp.packed, inp.scales, inp.biases, idx, G, bits)
    np.testing.assert_array_equal(got, full[idx])
    bf = oracle_lib.dequant_rows(inp.packed, inp.scales, inp.biases, idx, G, bits, out="bf16")
    np.testing.assert_array_equal(bf, oracle_lib.f32_to_bf16(full[idx]))


def test_dequant_rows_out_of_range_is_nan_row(oracle_lib):
    inp = W.random_inputs(4, 32, 4, 64, 0, seed=19)
    got = oracle_lib.dequant_rows(inp.packed, inp.scales, inp.biases,
                                  np.array([1, 4, 2**32 - 1], np.uint32), 32, 4)
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all() and not np.isnan(got[0]).any()


# ---- the comparison and the generator ----------------------------------------------------------

def test_max_row_rel_err(oracle_lib):
    ref = np.array([[1.0, -4.0], [0.0, 0.0]])
    y = np.array([[1.0, -3.9], [0.0, 1e-3]])
    assert oracle_lib.max_row_rel_err(y, ref) == pytest.approx(max(0.1 / 4.0, 1e-3))


def test_generator_is_seeded_and_uniform():
    wl = W.WORKLOADS["ref_4bit_g64_256x512"]
    a, b = W.make_inputs(wl, m=4), W.make_inputs(wl, m=4)
    np.testing.assert_array_equal(a.packed, b.packed)
    np.testing.assert_array_equal(a.x, b.x)
    assert a.packed.shape == (256, 64) and a.scales.shape == (256, 8) and a.x.shape == (4, 512)
    s = W.f32_from_bf16_bits(a.scales)
    bb = W.f32_from_bf16_bits(a.biases)
    assert s.min() >= 1e-3 * 0.99 and s.max() <= 5e-2 and bb.min() >= -0.4 and bb.max() <= 0
    # the M = 1 and M = 4 draws of one workload share their weights
    wl2 = W.WORKLOADS["decode_4bit_g64_4096x4096"]
    p1 = W.make_inputs(wl2, m=1, n=64)
    p4 = W.make_inputs(wl2, m=4, n=64)
    np.testing.assert_array_equal(p1.packed, p4.packed)


# ---- fused decode products (spark_runtime gemv_silu_gate, gemv_silu_gate_resid) ----------------

def _bf16v(vals):
    return np.concatenate([_bf16(v) for v in vals])


def test_silu_known_values(oracle_lib):
    # logistic(1) = 0.7310585786300049 and logistic(2) = 0.8807970779778823 (tabulated values),
    # so silu(1), silu(-1) = -(1 - logistic(1)), silu(2) and silu(-2) follow
    h = oracle_lib.silu_gate(_bf16v([0.0, 1.0, -1.0, 2.0, -2.0]), _bf16v([1.0] * 5))
    expect = [0.0, 0.7310585786300049, -0.2689414213699951, 2 * 0.8807970779778823,
              -2 * (1 - 0.8807970779778823)]
    np.testing.assert_allclose(h, expect, rtol=1e-15, atol=1e-16)


def test_silu_odd_part_and_saturation(oracle_lib):
    # silu(v) - silu(-v) = v for every v (sigmoid(v) + sigmoid(-v) = 1); a sign slip or a dropped
    # factor breaks it. Far out, silu saturates to v and to 0.
    rng = np.random.default_rng(3)
    v = W.bf16_bits_from_f32(rng.uniform(-12, 12, 500).astype(np.float32))
    neg = v ^ np.uint16(0x8000)
    one = _bf16v([1.0] * v.size)
    hv = oracle_lib.silu_gate(v, one)
    hn = oracle_lib.silu_gate(neg, one)
    np.testing.assert_allclose(hv - hn, W.f32_from_bf16_bits(v).astype(np.float64), rtol=0, atol=1e-14)
    far = oracle_lib.silu_gate(_bf16v([64.0, -64.0]), _bf16v([1.0, 1.0]))
    assert far[0] == 64.0 and -1e-25 < far[1] < 0


def test_silu_gate_qmm_reduces_to_qmm(oracle_lib):
    # gate = 64 makes silu(gate) = 64 exactly in double, so with up = x / 64 (exact in bf16) the
    # fused product is the plain matmul of x
    inp = W.random_inputs(4, 64, 9, 256, 3, seed=11)
    x = W.f32_from_bf16_bits(inp.x)
    up = W.bf16_bits_from_f32(x / 64)
    assert np.array_equal(W.f32_from_bf16_bits(up) * 64, x)
    gate = np.full_like(inp.x, _bf16(64.0)[0])
    y = oracle_lib.silu_gate_qmm(gate, up, None, inp.packed, inp.scales, inp.biases, 64, 4)
    ref = oracle_lib.qmm(inp.x, "bf16", inp.packed, inp.scales, inp.biases, 64, 4)
    np.testing.assert_array_equal(y, ref)


def test_silu_gate_residual_and_linearity(oracle_lib):
    inp = W.random_inputs(3, 32, 7, 128, 2, seed=12)
    rng = np.random.default_rng(5)
    gate = W.bf16_bits_from_f32(rng.standard_normal((2, 128)).astype(np.float32))
    up = W.bf16_bits_from_f32(rng.standard_normal((2, 128)).astype(np.float32))
    resid = W.bf16_bits_from_f32(rng.standard_normal((2, 7)).astype(np.float32))
    # a zero weight (scales and biases 0) leaves exactly the residual
    zs = np.zeros_like(inp.scales)
    y0 = oracle_lib.silu_gate_qmm(gate, up, resid, inp.packed, zs, zs, 32, 3)
    np.testing.assert_array_equal(y0, W.f32_from_bf16_bits(resid).astype(np.float64))
    # the residual is added, not subtracted or scaled
    y = oracle_lib.silu_gate_qmm(gate, up, None, inp.packed, inp.scales, inp.biases, 32, 3)
    yr = oracle_lib.silu_gate_qmm(gate, up, resid, inp.packed, inp.scales, inp.biases, 32, 3)
    np.testing.assert_allclose(yr - y, W.f32_from_bf16_bits(resid), rtol=0, atol=1e-12)
    # doubling up (exact in bf16) doubles y: up enters as a factor, gate through silu
    up2 = W.bf16_bits_from_f32(W.f32_from_bf16_bits(up) * 2)
    y2 = oracle_lib.silu_gate_qmm(gate, up2, None, inp.packed, inp.scales, inp.biases, 32, 3)
    np.testing.assert_allclose(y2, 2 * y, rtol=1e-14, atol=1e-14)
    # up = 0 gives 0 whatever the gate
    yz = oracle_lib.silu_gate_qmm(gate, np.zeros_like(up), None, inp.packed, inp.scales, inp.biases, 32, 3)
    assert not yz.any()


# ---- gathered products (mixture of experts) -----------------------------------------------------

def _experts(oracle_lib, experts, n, k, G, bits, seed):
    """`experts` random weights of [n, k], stacked: packed [E, n, k*bits/32], scales/biases [E, n, k/G]."""
    parts = [W.random_inputs(bits, G, n, k, 1, seed=seed + e) for e in range(experts)]
    return (np.stack([p.packed for p in parts]), np.stack([p.scales for p in parts]),
            np.stack([p.biases for p in parts]))


def test_gather_qmm_worked_example(oracle_lib):
    g = golden("gather_qmm_two_experts.txt")
    E, n, k = int(g["experts"][0]), int(g["n"][0]), int(g["k"][0])
    G, bits = int(g["group_size"][0]), int(g["bits"][0])
    codes = np.stack([np.full((n, k), int(c), np.uint8) for c in g["codes"]])
    packed = np.stack([oracle_lib.pack_codes(codes[e], bits) for e in range(E)])
    sc = np.stack([np.full((n, k // G), _bf16(float(v))[0], np.uint16) for v in g["scale"]])
    bi = np.stack([np.full((n, k // G), _bf16(float(v))[0], np.uint16) for v in g["bias"]])
    # the hand-built experts really are all-ones and all-twos
    for e in range(E):
        assert np.all(oracle_lib.dequantize(packed[e], sc[e], bi[e], G, bits) == e + 1)
    x = np.ones((int(g["tokens"][0]), 1, k), np.float32)
    rhs = np.array([int(v) for v in g["rhs"]], np.uint32)
    y = oracle_lib.gather_qmm(x, "f32", packed, sc, bi, G, bits, rhs=rhs)
    assert list(y.shape) == [int(v) for v in g["shape"]]
    assert list(y.reshape(-1)[:5]) == [float(v) for v in g["expect_first5"]]
    # the rest follows from the same rule: token i takes expert rhs[i], whose rows sum to 64 (e + 1)
    np.testing.assert_array_equal(y[:, 0, :], np.repeat((64.0 * (rhs + 1))[:, None], n, axis=1))


def test_gather_qmm_default_indices_are_per_batch_qmm(oracle_lib):
    packed, sc, bi = _experts(oracle_lib, 3, 9, 128, 32, 3, seed=40)
    x = W.bf16_bits_from_f32(np.random.default_rng(41).standard_normal((3, 2, 128)).astype(np.float32))
    y = oracle_lib.gather_qmm(x, "bf16", packed, sc, bi, 32, 3)
    assert y.shape == (3, 2, 9)
    for b in range(3):
        np.testing.assert_array_equal(y[b], oracle_lib.qmm(x[b], "bf16", packed[b], sc[b], bi[b], 32, 3))


def test_gather_qmm_indices_against_numpy(oracle_lib):
    # x batches and experts differ in number, so swapped index arrays land out of range; every pair
    # is checked against a float64 numpy product of the (pinned) dequantized expert
    E, n, k, G, bits = 5, 7, 128, 64, 4
    packed, sc, bi = _experts(oracle_lib, E, n, k, G, bits, seed=50)
    x = np.random.default_rng(51).standard_normal((4, 3, k)).astype(np.float32)
    lhs = np.array([3, 0, 0, 2, 1, 3], np.uint32)
    rhs = np.array([4, 4, 1, 0, 2, 3], np.uint32)
    y = oracle_lib.gather_qmm(x, "f32", packed, sc, bi, G, bits, lhs=lhs, rhs=rhs)
    assert y.shape == (6, 3, n)
    for i in range(6):
        w = oracle_lib.dequantize(packed[rhs[i]], sc[rhs[i]], bi[rhs[i]], G, bits).astype(np.float64)
        np.testing.assert_allclose(y[i], x[lhs[i]].astype(np.float64) @ w.T, rtol=1e-12, atol=1e-12)


def test_gather_qmm_broadcasts_indices(oracle_lib):
    packed, sc, bi = _experts(oracle_lib, 3, 5, 64, 32, 2, seed=60)
    x = np.random.default_rng(61).standard_normal((2, 1, 64)).astype(np.float32)
    lhs = np.array([[1], [0]], np.int64)      # [2, 1]
    rhs = np.array([2, 0, 1], np.int32)       # [3]  -> batch [2, 3]
    y = oracle_lib.gather_qmm(x, "f32", packed, sc, bi, 32, 2, lhs=lhs, rhs=rhs)
    assert y.shape == (2, 3, 1, 5)
    for a in range(2):
        for b in range(3):
            ref = oracle_lib.qmm(x[lhs[a, 0]], "f32", packed[rhs[b]], sc[rhs[b]], bi[rhs[b]], 32, 2)
            np.testing.assert_array_equal(y[a, b], ref)
    # an absent lhs defaults to every x batch in order and broadcasts the same way
    y2 = oracle_lib.gather_qmm(x[:1], "f32", packed, sc, bi, 32, 2, rhs=rhs)
    np.testing.assert_array_equal(y2, y[1])  # lhs[1] = 0
    with pytest.raises(ValueError):
        oracle_lib.gather_qmm(x, "f32", packed, sc, bi, 32, 2, rhs=np.array([0.0, 1.0]))
    with pytest.raises(ValueError):   # 2 and 3 do not broadcast
        oracle_lib.gather_qmm(x, "f32", packed, sc, bi, 32, 2, lhs=np.array([0, 1]), rhs=rhs)


def test_gather_qmm_out_of_range_is_nan(oracle_lib):
    packed, sc, bi = _experts(oracle_lib, 2, 4, 64, 64, 8, seed=70)
    x = np.random.default_rng(71).standard_normal((2, 1, 64)).astype(np.float32)
    y = oracle_lib.gather_qmm(x, "f32", packed, sc, bi, 64, 8, lhs=np.array([0, 2, 1], np.uint32),
                              rhs=np.array([1, 0, 2], np.uint32))
    assert np.isnan(y[1]).all() and np.isnan(y[2]).all()
    np.testing.assert_array_equal(y[0], oracle_lib.qmm(x[0], "f32", packed[1], sc[1], bi[1], 64, 8))


# ---- quantize -----------------------------------------------------------------------------------

def test_quantize_module_example_shapes(oracle_lib):
    # nuvec_core module example: w[i] = i / 64 as [4, 64], group 64, 4 bits -> 8 words per row
    w = (np.arange(256, dtype=np.float32) / 64).reshape(4, 64)
    packed, sc, bi = oracle_lib.quantize(w, "f32", 64, 4)
    assert packed.shape == (4, 8) and sc.shape == (4, 1) and bi.shape == (4, 1)
    restored = oracle_lib.dequantize(packed, sc, bi, 64, 4)
    assert restored.shape == w.shape
    # bias = the group minimum (row r starts at r, exact in bf16)
    assert list(W.f32_from_bf16_bits(bi[:, 0])) == [0.0, 1.0, 2.0, 3.0]


def test_quantize_then_gather_qmm_worked_example(oracle_lib):
    # the page's two-expert example end to end, now with quantize: experts of all ones and all
    # twos must dequantize exactly for the printed 128 = 64 * 2
    g = golden("gather_qmm_two_experts.txt")
    E, n, k = int(g["experts"][0]), int(g["n"][0]), int(g["k"][0])
    G, bits = int(g["group_size"][0]), int(g["bits"][0])
    w = np.concatenate([np.full((n, k), e + 1.0, np.float32) for e in range(E)])
    packed, sc, bi = oracle_lib.quantize(w, "f32", G, bits)
    assert np.all(oracle_lib.dequantize(packed, sc, bi, G, bits) == w)
    x = np.ones((int(g["tokens"][0]), 1, k), np.float32)
    y = oracle_lib.gather_qmm(x, "f32", packed.reshape(E, n, -1), sc.reshape(E, n, -1), bi.reshape(E, n, -1),
                              G, bits, rhs=np.array([int(v) for v in g["rhs"]], np.uint32))
    assert list(y.shape) == [int(v) for v in g["shape"]]
    assert list(y.reshape(-1)[:5]) == [float(v) for v in g["expect_first5"]]


@pytest.mark.parametrize("bits,G,step,base", [(4, 32, 0.25, 0.5), (8, 128, 2.0 ** -4, -1.0),
                                              (3, 64, 0.75, -3.0), (2, 32, 4.0, 8.0), (6, 64, 2.0 ** -6, 0.0)])
def test_quantize_exact_grid(oracle_lib, bits, G, step, base):
    # values on the grid base + step * c, with both extreme codes present: quantize must return
    # exactly that step, that base and those codes (a denominator of 2^bits, a bias other than
    # the minimum, or another packing order fails here)
    top = 2 ** bits - 1
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, top + 1, size=(3, 2 * G)).astype(np.uint8)
    codes[:, 0], codes[:, 1], codes[:, G], codes[:, G + 1] = 0, top, top, 0
    w = (base + step * codes.astype(np.float64)).astype(np.float32)
    assert np.all(w.astype(np.float64) == base + step * codes)          # exact in float32
    wb = W.bf16_bits_from_f32(w)
    assert np.all(W.f32_from_bf16_bits(wb) == w)                         # and in bf16
    for dt, wi in (("f32", w), ("bf16", wb)):
        packed, sc, bi = oracle_lib.quantize(wi, dt, G, bits)
        assert np.all(W.f32_from_bf16_bits(sc) == step) and np.all(W.f32_from_bf16_bits(bi) == base)
        np.testing.assert_array_equal(oracle_lib.unpack_codes(packed, 2 * G, bits), codes)


def test_quantize_ties_round_away_from_zero(oracle_lib):
    # min 0, max 15 at 4 bits: scale exactly 1, so each value is its own quotient
    vals = [0.0, 15.0, 2.5, 3.5, 7.5, 14.5, 0.5, 1.25, 6.75] + [5.0] * 23
    w = np.array([vals], np.float32)
    packed, sc, bi = oracle_lib.quantize(w, "f32", 32, 4)
    assert W.f32_from_bf16_bits(sc)[0, 0] == 1.0 and W.f32_from_bf16_bits(bi)[0, 0] == 0.0
    codes = oracle_lib.unpack_codes(packed, 32, 4)[0]
    assert list(codes[:9]) == [0, 15, 3, 4, 8, 15, 1, 1, 7]   # halves go up; ties-to-even would give 2, 4, 8, 14, 0


def _round_half_away(q: Fraction) -> int:
    # the Rust `round` of the page, on an exact rational
    return int(q + Fraction(1, 2)) if q >= 0 else -int(-q + Fraction(1, 2))


def _exact_codes(w, sc, bi, G, bits):
    """round((w - bias) / scale) clamped, each quotient an exact rational (Fraction)."""
    top = 2 ** bits - 1
    s = W.f32_from_bf16_bits(sc).astype(np.float64)
    b = W.f32_from_bf16_bits(bi).astype(np.float64)
    out = np.zeros(w.shape, np.int64)
    for r in range(w.shape[0]):
        for j in range(w.shape[1]):
            sg, bg = s[r, j // G], b[r, j // G]
            if sg == 0.0:
                continue
            c = _round_half_away((Fraction(float(w[r, j])) - Fraction(bg)) / Fraction(sg))
            out[r, j] = min(max(c, 0), top)
    return out


def test_quantize_exact_difference_decides_a_tie(oracle_lib):
    # nuvec_core stores round((w - bias) / scale). Here w - bias is not a float32: the group's
    # minimum (and so its bias) is 2^-100, its maximum 0.9375, so scale = 0.9375 / 15 = 0.0625
    # exactly, and w = 3.5 * 0.0625 gives the exact quotient 3.5 - 2^-96, which rounds to 3. A
    # float32 difference would round w - bias onto 3.5 * 0.0625 and the tie up to 4 (the same for
    # 5.5 * 0.0625: 5, not 6). The expected codes come from exact rationals.
    w = tie_example()
    tiny = w[0, 0]
    assert np.float32(w[0, 2] - tiny) == w[0, 2]                  # the float32 difference rounds
    packed, sc, bi = oracle_lib.quantize(w, "f32", 32, 4)
    assert W.f32_from_bf16_bits(sc)[0, 0] == 0.0625 and W.f32_from_bf16_bits(bi)[0, 0] == tiny
    codes = oracle_lib.unpack_codes(packed, 32, 4)[0]
    expect = _exact_codes(w, sc, bi, 32, 4)[0]
    assert list(expect[:5]) == [0, 15, 3, 5, 8]
    np.testing.assert_array_equal(codes, expect)


def test_float32_quotient_of_a_float32_difference_is_exact_at_ties():
    # Why no pin separates an exact quotient from a float32 one: for a float32 d and a bf16 scale
    # s, fl32(d / s) is a half-integer only when d / s is (moving d by one ulp moves the quotient
    # by more than half an ulp). Checked on values within a few ulps of every tie k + 1/2.
    rng = np.random.default_rng(5)
    s = W.f32_from_bf16_bits(bf16_rne(rng.uniform(1e-3, 4.0, 20000)))
    k = rng.integers(0, 256, 20000)
    p = ((k + 0.5) * s.astype(np.float64)).astype(np.float32)           # exact: 9 + 8 bits
    d = p.copy()
    steps = rng.integers(-3, 4, 20000)
    for i in range(d.size):
        for _ in range(abs(int(steps[i]))):
            d[i] = np.nextafter(d[i], np.float32(np.inf if steps[i] > 0 else -np.inf))
    q32 = d / s
    on_tie = q32.astype(np.float64) == k + 0.5
    assert on_tie.sum() > 1000
    for i in np.flatnonzero(on_tie):
        assert Fraction(float(d[i])) / Fraction(float(s[i])) == Fraction(2 * int(k[i]) + 1, 2)


@pytest.mark.parametrize("bits,G", [(4, 64), (3, 32), (8, 128), (1, 32), (6, 64)])
def test_quantize_codes_are_exact_rational_rounding(oracle_lib, bits, G):
    # groups with values within a few float32 ulps of every kind of tie b + (k + 1/2) s, and
    # minima of very different magnitudes (so that w - bias often rounds): every code equals the
    # exact rational rounding of (w - bias) / scale, and the scales and biases are the bf16
    # roundings of the float32 statistics
    rows, top = 24, 2 ** bits - 1
    w = near_tie_groups(rows, 2, G, bits, seed=200 + bits)
    for dt in ("f32", "bf16"):
        wi = w if dt == "f32" else bf16_rne(w)
        wf = w if dt == "f32" else W.f32_from_bf16_bits(wi)
        packed, sc, bi = oracle_lib.quantize(wi, dt, G, bits)
        wg = wf.reshape(rows, -1, G)
        lo, hi = wg.min(-1), wg.max(-1)
        np.testing.assert_array_equal(sc, bf16_rne((hi - lo) / np.float32(top)))
        np.testing.assert_array_equal(bi, bf16_rne(lo))
        codes = oracle_lib.unpack_codes(packed, 2 * G, bits).astype(np.int64)
        np.testing.assert_array_equal(codes, _exact_codes(wf, sc, bi, G, bits))


def test_quantize_clamps(oracle_lib):
    # the stored bias rounds above the minimum (1.005 -> bf16 1.0078125): the minimum's quotient
    # is negative and clamps to 0; the scale rounds so that the maximum's quotient passes 2^bits - 1
    w = np.linspace(1.005, 1.9, 32, dtype=np.float32)[None, :]
    packed, sc, bi = oracle_lib.quantize(w, "f32", 32, 4)
    b = W.f32_from_bf16_bits(bi)[0, 0]
    assert b > w.min()
    codes = oracle_lib.unpack_codes(packed, 32, 4)[0]
    assert codes[0] == 0 and codes.max() <= 15
    s = W.f32_from_bf16_bits(sc)[0, 0]
    if (w.max() - b) / s > 15:
        assert codes[-1] == 15


def test_quantize_constant_and_zero_groups(oracle_lib):
    w = np.zeros((2, 64), np.float32)
    w[0, :32] = -0.375
    w[1, 32:] = 3.0
    packed, sc, bi = oracle_lib.quantize(w, "f32", 32, 5)
    assert not sc.any()                                     # every group is constant: scale 0
    assert not packed.any()                                 # ... and code 0
    np.testing.assert_array_equal(oracle_lib.dequantize(packed, sc, bi, 32, 5), w)


@pytest.mark.parametrize("bits,G", [(4, 64), (3, 32), (8, 128), (2, 64), (5, 32), (6, 128)])
def test_quantize_round_trip_bound(oracle_lib, bits, G):
    # |dequantize(quantize(w)) - w| <= scale / 2 plus what storing the bias and scale in bf16
    # moves the grid by (|bias - min| and (2^bits - 1) |scale - range / (2^bits - 1)|)
    rng = np.random.default_rng(100 + bits)
    w = (rng.standard_normal((16, 4 * G)) * 0.02).astype(np.float32)
    packed, sc, bi = oracle_lib.quantize(w, "f32", G, bits)
    r = oracle_lib.dequantize(packed, sc, bi, G, bits).astype(np.float64)
    top = 2 ** bits - 1
    wg = w.reshape(16, -1, G).astype(np.float64)
    lo, hi = wg.min(-1), wg.max(-1)
    s = W.f32_from_bf16_bits(sc).astype(np.float64)
    b = W.f32_from_bf16_bits(bi).astype(np.float64)
    bound = s / 2 + np.abs(b - lo) + top * np.abs(s - (hi - lo) / top) + 1e-7
    err = np.abs(r.reshape(16, -1, G) - wg).max(-1)
    assert np.all(err <= bound), float((err - bound).max())
    # codes use the whole range: the minimum's code is 0 and the maximum's is 2^bits - 1 or one below
    codes = oracle_lib.unpack_codes(packed, 4 * G, bits).reshape(16, -1, G)
    assert np.all(codes.min(-1) == 0) and np.all(codes.max(-1) >= top - 1)


# ---- the product without the transpose ----------------------------------------------------------

def test_qmm_nt_one_hot_selects_a_row(oracle_lib):
    # x = e_k picks row k of the dequantized [k, n] weight, exactly
    inp = W.random_inputs(3, 32, 12, 96, 0, seed=21)     # a [12, 96] weight read as W [k=12, n=96]
    w = oracle_lib.dequantize(inp.packed, inp.scales, inp.biases, 32, 3)
    x = np.eye(12, dtype=np.float32)[[0, 7, 11]]
    y = oracle_lib.qmm_nt(x, "f32", inp.packed, inp.scales, inp.biases, 32, 3)
    np.testing.assert_array_equal(y, w[[0, 7, 11]].astype(np.float64))


@pytest.mark.parametrize("bits,G", [(4, 64), (8, 32), (2, 128), (5, 32)])
def test_qmm_nt_matches_float64_matmul(oracle_lib, bits, G):
    # against numpy's float64 product of the pinned dequantization: x [3, k] . W [k, n]; a
    # transposed operand (the other form) would not even have these shapes
    inp = W.random_inputs(bits, G, 40, 2 * G, 0, seed=22 + bits)
    w = oracle_lib.dequantize(inp.packed, inp.scales, inp.biases, G, bits).astype(np.float64)
    x = np.random.default_rng(5).standard_normal((3, 40)).astype(np.float32)
    y = oracle_lib.qmm_nt(x, "f32", inp.packed, inp.scales, inp.biases, G, bits)
    assert y.shape == (3, 2 * G)
    np.testing.assert_allclose(y, x.astype(np.float64) @ w, rtol=1e-12, atol=1e-12)


def test_qmm_nt_and_qmm_agree_on_a_symmetric_weight(oracle_lib):
    # a weight with w[i, j] = w[j, i] dequantizes to the same matrix read either way, so the
    # product with and without the transpose must agree to the bit
    n = 64
    codes = np.random.default_rng(8).integers(0, 16, size=(n, n)).astype(np.uint8)
    codes = np.triu(codes) + np.triu(codes, 1).T
    packed = oracle_lib.pack_codes(codes, 4)
    sc = np.full((n, 1), _bf16(0.25)[0], np.uint16)   # one group per row, the same everywhere
    bi = np.full((n, 1), _bf16(-1.0)[0], np.uint16)
    x = np.random.default_rng(9).standard_normal((2, n)).astype(np.float32)
    y_nt = oracle_lib.qmm_nt(x, "f32", packed, sc, bi, 64, 4)
    y_t = oracle_lib.qmm(x, "f32", packed, sc, bi, 64, 4)
    np.testing.assert_array_equal(y_nt, y_t)


# ---- float16 and float32 scales, biases and x -----------------------------------------------------

def test_f16_widening_matches_numpy(oracle_lib):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)      # every binary16 pattern
    got = oracle_lib.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_narrowing_matches_numpy(oracle_lib):
    rng = np.random.default_rng(3)
    a = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 5, 200000),
        # exact midpoints between neighbours (ties), around subnormals, near the overflow point
        (np.arange(1, 2048, dtype=np.float32) + 0.5) * np.float32(2.0 ** -24),
        (np.arange(1024, 2048, dtype=np.float32) + 0.5) * np.float32(2.0 ** -10),
        np.array([65504.0, 65519.0, 65520.0, 70000.0, -65520.0, 0.0, -0.0, 6e-8, 3e-8, 2.9e-8], np.float32),
    ]).astype(np.float32)
    got = oracle_lib.f32_to_f16(a)
    with np.errstate(over="ignore"):
        ref = a.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("sb", ["f16", "f32", "bf16"])
def test_dequantize_typed_is_the_affine_rule(oracle_lib, sb):
    # w = s * c then + b in float32, with s and b read in their own type: against numpy float32
    # arithmetic on the same widened values (two roundings, as written)
    inp = W.random_inputs(5, 32, 6, 128, 0, seed=31)
    rng = np.random.default_rng(32)
    s32 = rng.uniform(1e-3, 2e-2, (6, 4)).astype(np.float32)
    b32 = rng.uniform(-0.15, 0.0, (6, 4)).astype(np.float32)
    if sb == "f16":
        sc, bi = s32.astype(np.float16).view(np.uint16), b32.astype(np.float16).view(np.uint16)
        sw, bw = sc.view(np.float16).astype(np.float32), bi.view(np.float16).astype(np.float32)
    elif sb == "bf16":
        sc, bi = W.bf16_bits_from_f32(s32), W.bf16_bits_from_f32(b32)
        sw, bw = W.f32_from_bf16_bits(sc), W.f32_from_bf16_bits(bi)
    else:
        sc, bi, sw, bw = s32, b32, s32, b32
    codes = oracle_lib.unpack_codes(inp.packed, 128, 5).astype(np.float32)
    g = np.arange(128) // 32
    ref = (sw[:, g] * codes).astype(np.float32) + bw[:, g]
    got = oracle_lib.dequantize_typed(inp.packed, sc, bi, sb, 32, 5)
    np.testing.assert_array_equal(got.view(np.uint32), ref.astype(np.float32).view(np.uint32))
    if sb == "bf16":   # the typed form with bf16 scales is the plain dequantization
        np.testing.assert_array_equal(got, oracle_lib.dequantize(inp.packed, sc, bi, 32, 5))


def test_qmm_typed_reduces_to_qmm(oracle_lib):
    inp = W.random_inputs(4, 64, 9, 256, 3, seed=33)
    np.testing.assert_array_equal(
        oracle_lib.qmm_typed(inp.x, "bf16", inp.packed, inp.scales, inp.biases, "bf16", 64, 4),
        oracle_lib.qmm(inp.x, "bf16", inp.packed, inp.scales, inp.biases, 64, 4))
    # a float16 x holding the same values as the bf16 one gives the same product
    xf = W.f32_from_bf16_bits(inp.x)
    x16 = xf.astype(np.float16)
    exact = x16.astype(np.float32) == xf
    xf = np.where(exact, xf, 0).astype(np.float32)
    y16 = oracle_lib.qmm_typed(xf.astype(np.float16).view(np.uint16), "f16", inp.packed, inp.scales, inp.biases,
                               "bf16", 64, 4)
    y32 = oracle_lib.qmm_typed(xf, "f32", inp.packed, inp.scales, inp.biases, "bf16", 64, 4)
    np.testing.assert_array_equal(y16, y32)
    # against numpy float64 over the typed dequantization
    s16 = W.f32_from_bf16_bits(inp.scales).astype(np.float16).view(np.uint16)
    b16 = W.f32_from_bf16_bits(inp.biases).astype(np.float16).view(np.uint16)
    w = oracle_lib.dequantize_typed(inp.packed, s16, b16, "f16", 64, 4).astype(np.float64)
    y = oracle_lib.qmm_typed(xf, "f32", inp.packed, s16, b16, "f16", 64, 4)
    np.testing.assert_allclose(y, xf.astype(np.float64) @ w.T, rtol=1e-12, atol=1e-12)


def test_qmm_nt_typed_reduces_to_qmm_nt(oracle_lib):
    # bf16 scales: the typed form is the plain product without the transpose, for bf16 and f32 x
    inp = W.random_inputs(4, 64, 24, 128, 0, seed=34)         # W [k=24, n=128]
    xb = W.random_inputs(4, 64, 8, 64, 3, seed=35).x[:, :24].copy()
    for x, dt in ((xb, "bf16"), (W.f32_from_bf16_bits(xb), "f32")):
        np.testing.assert_array_equal(
            oracle_lib.qmm_nt_typed(x, dt, inp.packed, inp.scales, inp.biases, "bf16", 64, 4),
            oracle_lib.qmm_nt(x, dt, inp.packed, inp.scales, inp.biases, 64, 4))


@pytest.mark.parametrize("x_dt,sb_dt", [("f16", "f16"), ("f32", "f16"), ("bf16", "f32"), ("f16", "bf16")])
def test_qmm_nt_typed_against_numpy(oracle_lib, x_dt, sb_dt):
    # numpy's float64 product of the pinned typed dequantization, x [3, k] . W [k, n]; x holds
    # multiples of 1/64 below 4 in magnitude, which all three types represent exactly
    bits, G = 5, 32
    inp = W.random_inputs(bits, G, 40, 96, 0, seed=36)
    conv = {"f16": lambda a: a.astype(np.float16).view(np.uint16), "f32": lambda a: a.astype(np.float32),
            "bf16": lambda a: W.bf16_bits_from_f32(a.astype(np.float32))}
    sf = W.f32_from_bf16_bits(inp.scales)
    bf = W.f32_from_bf16_bits(inp.biases)
    sc, bi = conv[sb_dt](sf), conv[sb_dt](bf)
    w = oracle_lib.dequantize_typed(inp.packed, sc, bi, sb_dt, G, bits).astype(np.float64)
    xf = (np.random.default_rng(6).integers(-255, 256, size=(3, 40)) / 64).astype(np.float32)
    x = conv[x_dt](xf)
    y = oracle_lib.qmm_nt_typed(x, x_dt, inp.packed, sc, bi, sb_dt, G, bits)
    assert y.shape == (3, 96)
    np.testing.assert_allclose(y, xf.astype(np.float64) @ w, rtol=1e-12, atol=1e-12)
    # x = e_k picks row k of the typed dequantization, exactly
    e = conv[x_dt](np.eye(40, dtype=np.float32)[[0, 13, 39]])
    np.testing.assert_array_equal(oracle_lib.qmm_nt_typed(e, x_dt, inp.packed, sc, bi, sb_dt, G, bits),
                                  w[[0, 13, 39]])


def test_qmm_nt_typed_and_qmm_typed_agree_on_a_symmetric_weight(oracle_lib):
    # float16 scales on a symmetric weight: the product with and without the transpose agree to the bit
    n = 64
    codes = np.random.default_rng(18).integers(0, 16, size=(n, n)).astype(np.uint8)
    codes = np.triu(codes) + np.triu(codes, 1).T
    packed = oracle_lib.pack_codes(codes, 4)
    sc = np.full((n, 1), np.float16(0.3).view(np.uint16), np.uint16)
    bi = np.full((n, 1), np.float16(-1.1).view(np.uint16), np.uint16)
    x = np.random.default_rng(19).standard_normal((2, n)).astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle_lib.qmm_nt_typed(x, "f16", packed, sc, bi, "f16", 64, 4),
                                  oracle_lib.qmm_typed(x, "f16", packed, sc, bi, "f16", 64, 4))


# ---- quantize with float16 / float32 weights, scales and biases ----------------------------------

_TYPE = {"f32": np.float32, "bf16": None, "f16": np.float16}


def _as_type(w32, dt):
    """float32 values (exact in dt) as the oracle's input for dtype dt."""
    if dt == "f32":
        return w32.astype(np.float32)
    if dt == "f16":
        return w32.astype(np.float16).view(np.uint16)
    return W.bf16_bits_from_f32(w32)


def _widen(a, dt):
    """An oracle array of dtype dt as float64, widened by numpy and torch (not the oracle)."""
    if dt == "f32":
        return a.astype(np.float64)
    if dt == "f16":
        return a.view(np.float16).astype(np.float64)
    return W.f32_from_bf16_bits(a).astype(np.float64)


def _exact_codes_f(w64, s64, b64, G, bits):
    """round((w - bias) / scale) clamped, each quotient an exact rational (Fraction)."""
    top = 2 ** bits - 1
    out = np.zeros(w64.shape, np.int64)
    for r in range(w64.shape[0]):
        for j in range(w64.shape[1]):
            sg, bg = s64[r, j // G], b64[r, j // G]
            if sg == 0.0:
                continue
            c = _round_half_away((Fraction(float(w64[r, j])) - Fraction(float(bg))) / Fraction(float(sg)))
            out[r, j] = min(max(c, 0), top)
    return out


@pytest.mark.parametrize("w_dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("sb_dt", ["f32", "bf16", "f16"])
def test_quantize_typed_exact_grid(oracle_lib, w_dt, sb_dt):
    # values base + step * c, exact in every type, both extreme codes present: the scale is step and
    # the bias base in the scales' own type, and the codes come back (nuvec_core: scales and biases
    # in w's dtype; any of the three here)
    G, bits, step, base = 32, 4, 0.125, -1.5
    rng = np.random.default_rng(41)
    codes = rng.integers(0, 16, size=(3, 2 * G)).astype(np.uint8)
    codes[:, 0], codes[:, 1], codes[:, G], codes[:, G + 1] = 0, 15, 15, 0
    w32 = (base + step * codes.astype(np.float64)).astype(np.float32)
    packed, sc, bi = oracle_lib.quantize(_as_type(w32, w_dt), w_dt, G, bits, sb_dt)
    assert sc.dtype == (np.float32 if sb_dt == "f32" else np.uint16)
    assert np.all(_widen(sc, sb_dt) == step) and np.all(_widen(bi, sb_dt) == base)
    np.testing.assert_array_equal(oracle_lib.unpack_codes(packed, 2 * G, bits), codes)


@pytest.mark.parametrize("w_dt,sb_dt", [("f32", "f32"), ("f16", "f16"), ("f32", "f16"), ("bf16", "f16"),
                                        ("f16", "f32"), ("f16", "bf16")])
@pytest.mark.parametrize("bits,G", [(4, 64), (3, 32), (8, 128)])
def test_quantize_typed_codes_are_exact_rational_rounding(oracle_lib, w_dt, sb_dt, bits, G):
    # values within a few ulps of the boundaries of the stored scale and bias: every code is the
    # exact rational rounding of (w - bias) / scale, and the scales and biases are the roundings of
    # the float32 statistics to their type (numpy's float16 conversion, torch's bf16 one)
    rows = 12
    stored = {"f32": f32_value, "bf16": bf16_value, "f16": f16_value}[sb_dt]
    w_type = np.float16 if w_dt == "f16" else np.float32
    w = near_tie_groups(rows, 2, G, bits, seed=300 + bits, w_type=w_type, stored=stored)
    wf = w.astype(np.float32)
    if w_dt == "bf16":
        wi = bf16_rne(wf)
        wf = W.f32_from_bf16_bits(wi)
    else:
        wi = w if w_dt == "f32" else w.view(np.uint16)
    packed, sc, bi = oracle_lib.quantize(wi, w_dt, G, bits, sb_dt)
    wg = wf.reshape(rows, -1, G)
    lo, hi = wg.min(-1), wg.max(-1)
    q = (hi - lo) / np.float32(2 ** bits - 1)
    np.testing.assert_array_equal(_widen(sc, sb_dt), stored(q).astype(np.float64))
    np.testing.assert_array_equal(_widen(bi, sb_dt), stored(lo).astype(np.float64))
    codes = oracle_lib.unpack_codes(packed, 2 * G, bits).astype(np.int64)
    np.testing.assert_array_equal(codes, _exact_codes_f(wf.astype(np.float64), _widen(sc, sb_dt),
                                                        _widen(bi, sb_dt), G, bits))


def test_quantize_float32_scale_exact_quotient_below_a_tie(oracle_lib):
    # With a float32 scale, (k + 1/2) * scale needs more than 24 bits, so a float32 value can sit
    # just below it while its float32 quotient lands on the tie: scale 1 + 2^-20 (min 0, max 15 *
    # scale, exact in float32), w = fl32((k + 1/2) * scale) rounded down. The exact quotient is
    # below k + 1/2 and rounds to k; rounding the float32 quotient would give k + 1.
    s = np.float32(1.0 + 2.0 ** -20)
    lo, hi = np.float32(0.0), np.float32(15.0 * (1.0 + 2.0 ** -20))
    assert float(hi) == 15.0 * (1.0 + 2.0 ** -20) and np.float32(hi / np.float32(15)) == s
    picks = []
    for k in range(15):
        exact = Fraction(2 * k + 1, 2) * Fraction(float(s))
        v = np.float32(float(exact))
        if Fraction(float(v)) == exact:
            continue                      # (k + 1/2) * scale is itself a float32: no such value
        if Fraction(float(v)) > exact:
            v = np.nextafter(v, np.float32(-np.inf))
        assert Fraction(float(v)) < exact
        if float(np.float32(v / s)) == k + 0.5:
            picks.append((k, v))
    assert len(picks) >= 3
    w = np.full((1, 32), lo, np.float32)
    w[0, 1] = hi
    for i, (k, v) in enumerate(picks[:8]):
        w[0, 2 + i] = v
    packed, sc, bi = oracle_lib.quantize(w, "f32", 32, 4, "f32")
    assert sc[0, 0] == s and bi[0, 0] == 0.0
    codes = oracle_lib.unpack_codes(packed, 32, 4)[0]
    assert [int(codes[2 + i]) for i in range(len(picks[:8]))] == [k for k, _ in picks[:8]]


# ---- gathered products with float16 / float32 x, scales and biases -------------------------------

def test_gather_qmm_typed_against_numpy(oracle_lib):
    # batch i: x[lhs[i]] . dequantize_typed(W[rhs[i]])^T (the typed dequantization is pinned above)
    # in numpy float64, NaN past either operand, for a float16 x and float32 / float16 scales
    E, n, k, G, bits, m = 3, 10, 128, 32, 5, 2
    inp = W.random_inputs(bits, G, E * n, k, 0, seed=51)
    packed = inp.packed.reshape(E, n, -1)
    rng = np.random.default_rng(52)
    x32 = rng.standard_normal((4, m, k)).astype(np.float16).astype(np.float32)
    lhs = np.array([0, 3, 2, 4, 1], np.uint32)
    rhs = np.array([2, 0, 1, 1, 5], np.uint32)
    s32 = rng.uniform(1e-3, 2e-2, (E, n, k // G)).astype(np.float32)
    b32 = rng.uniform(-0.2, 0.0, (E, n, k // G)).astype(np.float32)
    for x_dt, sb_dt in (("f16", "f32"), ("f16", "f16"), ("f32", "f16"), ("bf16", "f32")):
        sc, bi = _as_type(s32, sb_dt), _as_type(b32, sb_dt)
        xi = _as_type(x32, x_dt)
        got = oracle_lib.gather_qmm_typed(xi, x_dt, packed, sc, bi, sb_dt, G, bits, lhs=lhs, rhs=rhs)
        assert got.shape == (5, m, n)
        for i, (li, ri) in enumerate(zip(lhs, rhs)):
            if li >= 4 or ri >= E:
                assert np.isnan(got[i]).all()
                continue
            w = oracle_lib.dequantize_typed(packed[ri], sc[ri], bi[ri], sb_dt, G, bits).astype(np.float64)
            np.testing.assert_allclose(got[i], _widen(xi[li], x_dt) @ w.T, rtol=1e-12, atol=1e-12)


def test_gather_qmm_typed_reduces_to_gather_qmm(oracle_lib):
    # bf16 scales and a float32 or bf16 x: the plain gathered product
    E, n, k, G, bits = 4, 12, 256, 64, 4
    inp = W.random_inputs(bits, G, E * n, k, 0, seed=53)
    p, sc, bi = (a.reshape(E, n, -1) for a in (inp.packed, inp.scales, inp.biases))
    x = W.bf16_bits_from_f32(np.random.default_rng(54).standard_normal((3, 2, k)).astype(np.float32))
    lhs, rhs = np.array([2, 0, 1, 2], np.uint32), np.array([3, 3, 0, 1], np.uint32)
    np.testing.assert_array_equal(oracle_lib.gather_qmm_typed(x, "bf16", p, sc, bi, "bf16", G, bits, lhs, rhs),
                                  oracle_lib.gather_qmm(x, "bf16", p, sc, bi, G, bits, lhs=lhs, rhs=rhs))
