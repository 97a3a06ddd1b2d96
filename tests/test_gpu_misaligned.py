"""Operands that are not 16-byte aligned (a tensor at a 2-byte offset into a buffer, a row slice)
through the C ABI, for every entry point, against the oracle.

x, y, out, w, gate, up and resid need only their element size of alignment. The vector kernels
take 16-byte aligned operands; the others are served element by element: dequantize,
dequant_rows and quantize by kernels of the same arithmetic (bit for bit, as always), the products
by a GEMV of the same float32 arithmetic in another summation order (the qmm bars, and the tight
bars of the VALU GEMV: 1e-4 for float32 y, 4e-3 for bf16 y, float16 1e-3). The MFMA paths, forced,
refuse such operands (UNSUPPORTED)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as orc_mod
from gpu_util import at_offset, banner, dev_bf16, dev_u32, dev_weights, dev_x, host_bits, host_f64
from quantized_matmul_mlx_amd import _lib
from quantized_matmul_mlx_amd import workloads as W

pytestmark = pytest.mark.gpu

BF16, F32, F16 = _lib.QAFF_BF16, _lib.QAFF_F32, _lib.QAFF_F16
TIGHT = {"f32": 1e-4, "bf16": 4e-3}


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    orc_mod.build()
    return _lib.load()


def S():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def P(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def off(t, elements=1):
    v = at_offset(t, elements)
    assert v.data_ptr() % 16 != 0
    return v


def empty_off(shape, dtype, elements=1):
    return off(torch.full(shape, float("nan"), dtype=dtype, device="cuda"), elements)


@pytest.mark.parametrize("bits,G", [(4, 64), (3, 32), (8, 128), (1, 32)])
def test_dequantize_and_rows_bit_exact(lib, bits, G):
    inp = W.random_inputs(bits, G, 37, 5 * G, 0, seed=bits + G)
    p, s, b = dev_weights(inp)
    idx_np = np.array([36, 0, 5, 5, 37, 2**32 - 1, 11], np.uint32)
    idx = dev_u32(idx_np)
    for out, tdt, view, shift in (("bf16", torch.bfloat16, np.uint16, 1), ("f32", torch.float32, np.uint32, 1),
                                  ("bf16", torch.bfloat16, np.uint16, 3)):
        banner(f"misaligned dequantize bits={bits} G={G} out={out} shift={shift}")
        o = empty_off((37, 5 * G), tdt, shift)
        _lib.check(lib.qaff_dequantize(P(p), P(s), P(b), 37, 5 * G, G, bits, P(o), BF16 if out == "bf16" else F32, S()))
        r = empty_off((7, 5 * G), tdt, shift)
        _lib.check(lib.qaff_dequant_rows(P(p), P(s), P(b), 37, 5 * G, G, bits, P(idx), 7, P(r),
                                         BF16 if out == "bf16" else F32, S()))
        torch.cuda.synchronize()
        ref = orc_mod.dequantize(inp.packed, inp.scales, inp.biases, G, bits, out=out)
        np.testing.assert_array_equal(host_bits(o).view(view), ref.view(view))
        rref = orc_mod.dequant_rows(inp.packed, inp.scales, inp.biases, idx_np, G, bits, out=out)
        np.testing.assert_array_equal(host_bits(r).view(view), rref.view(view))


@pytest.mark.parametrize("x_dtype,m", [("bf16", 1), ("bf16", 4), ("bf16", 40), ("f32", 3)])
@pytest.mark.parametrize("bits,G", [(4, 64), (6, 32), (8, 128)])
def test_qmm(lib, x_dtype, m, bits, G):
    k = 4 * G * 5
    inp = W.random_inputs(bits, G, 150, k, m, x_dtype=x_dtype, seed=bits + G + m)
    p, s, b = dev_weights(inp)
    x = off(dev_x(inp.x, x_dtype))
    tdt = torch.bfloat16 if x_dtype == "bf16" else torch.float32
    y = empty_off((m, 150), tdt)
    xdt = BF16 if x_dtype == "bf16" else F32
    banner(f"misaligned qmm x={x_dtype} m={m} bits={bits} G={G}")
    _lib.check(lib.qaff_qmm(P(x), xdt, m, P(p), P(s), P(b), 150, k, G, bits, P(y), S()))
    torch.cuda.synchronize()
    ref = orc_mod.qmm(inp.x, x_dtype, inp.packed, inp.scales, inp.biases, G, bits)
    got = host_f64(y)
    assert np.isfinite(got).all()
    assert orc_mod.max_row_rel_err(got, ref) <= TIGHT[x_dtype]
    # with a workspace (qaff_qmm_ws) the same
    y2 = empty_off((m, 150), tdt)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    _lib.check(lib.qaff_qmm_ws(P(x), xdt, m, P(p), P(s), P(b), 150, k, G, bits, P(ws), ws.numel(), P(y2), S()))
    torch.cuda.synchronize()
    assert orc_mod.max_row_rel_err(host_f64(y2), ref) <= TIGHT[x_dtype]


def test_forced_mfma_paths_refuse(lib):
    inp = W.random_inputs(4, 64, 64, 512, 4, seed=3)
    p, s, b = dev_weights(inp)
    x = off(dev_x(inp.x, "bf16"))
    y = torch.empty((4, 64), dtype=torch.bfloat16, device="cuda")
    for path in (_lib.PATHS["gemm"], _lib.PATHS["gemv_mfma"]):
        rc = lib.qaff_qmm_ex(P(x), BF16, 4, P(p), P(s), P(b), 64, 512, 64, 4, P(y), S(), path)
        assert rc == _lib.QAFF_ERR_UNSUPPORTED and b"16-byte" in lib.qaff_last_error()


def test_gate_up(lib):
    a = W.random_inputs(4, 64, 300, 1024, 3, seed=11)
    c = W.random_inputs(4, 64, 300, 1024, 3, seed=12)
    pa, sa, ba = dev_weights(a)
    pc, sc, bc = dev_weights(c)
    x = off(dev_x(a.x, "bf16"))
    gy, uy = empty_off((3, 300), torch.bfloat16), empty_off((3, 300), torch.bfloat16, 3)
    banner("misaligned gemv_gate_up")
    _lib.check(lib.qaff_gemv_gate_up(P(x), 3, P(pa), P(sa), P(ba), P(pc), P(sc), P(bc), 300, 1024, 64, 4,
                                     P(gy), P(uy), S()))
    torch.cuda.synchronize()
    for got, w in ((gy, a), (uy, c)):
        ref = orc_mod.qmm(a.x, "bf16", w.packed, w.scales, w.biases, 64, 4)
        assert orc_mod.max_row_rel_err(host_f64(got), ref) <= TIGHT["bf16"]


@pytest.mark.parametrize("with_resid", [False, True])
def test_silu_gate(lib, with_resid):
    inp = W.random_inputs(3, 32, 200, 2048, 2, seed=13)
    p, s, b = dev_weights(inp)
    rng = np.random.default_rng(14)
    gate = W.bf16_bits_from_f32((rng.standard_normal((2, 2048)) * 2).astype(np.float32))
    up = W.bf16_bits_from_f32(rng.standard_normal((2, 2048)).astype(np.float32))
    resid = W.bf16_bits_from_f32((rng.standard_normal((2, 200)) * 0.5).astype(np.float32)) if with_resid else None
    g, u = off(dev_bf16(gate)), off(dev_bf16(up), 3)
    r = off(dev_bf16(resid)) if with_resid else None
    y = empty_off((2, 200), torch.bfloat16)
    banner(f"misaligned gemv_silu_gate resid={with_resid}")
    _lib.check(lib.qaff_gemv_silu_gate(P(g), P(u), 2, P(p), P(s), P(b), 200, 2048, 32, 3, P(r), P(y), S()))
    torch.cuda.synchronize()
    h16 = orc_mod.f32_to_bf16(orc_mod.silu_gate(gate, up).astype(np.float32))
    tight = orc_mod.qmm(h16, "bf16", inp.packed, inp.scales, inp.biases, 32, 3)
    if with_resid:
        tight = tight + W.f32_from_bf16_bits(resid)
    got = host_f64(y)
    assert orc_mod.max_row_rel_err(got, orc_mod.silu_gate_qmm(gate, up, resid, inp.packed, inp.scales, inp.biases,
                                                              32, 3)) <= 1.6e-2
    assert orc_mod.max_row_rel_err(got, tight) <= TIGHT["bf16"]


def test_gather_qmm(lib):
    E, n, k, m = 5, 96, 512, 2
    wl = W.random_inputs(4, 64, E * n, k, 0, seed=15)
    p, s, b = dev_weights(wl)
    xs = W.bf16_bits_from_f32(np.random.default_rng(16).standard_normal((3, m, k)).astype(np.float32))
    lhs = np.array([2, 0, 1, 7, 2], np.uint32)
    rhs = np.array([4, 4, 0, 1, 9], np.uint32)
    x = off(dev_bf16(xs))
    y = empty_off((5, m, n), torch.bfloat16)
    lhs_d, rhs_d = dev_u32(lhs), dev_u32(rhs)   # held until the launch has run
    banner("misaligned gather_qmm")
    _lib.check(lib.qaff_gather_qmm(P(x), BF16, 3, m, P(p), P(s), P(b), E, n, k, 64, 4, P(lhs_d), P(rhs_d), 5, 0,
                                   P(y), S()))
    torch.cuda.synchronize()
    ref = orc_mod.gather_qmm(xs, "bf16", wl.packed.reshape(E, n, -1), wl.scales.reshape(E, n, -1),
                             wl.biases.reshape(E, n, -1), 64, 4, lhs=lhs, rhs=rhs)
    got = host_f64(y)
    for i in range(5):
        if lhs[i] >= 3 or rhs[i] >= E:
            assert np.isnan(got[i]).all()
        else:
            assert orc_mod.max_row_rel_err(got[i], ref[i]) <= TIGHT["bf16"]


@pytest.mark.parametrize("dtype,shift", [("bf16", 1), ("f32", 1), ("bf16", 5)])
@pytest.mark.parametrize("bits,G", [(4, 64), (5, 32), (8, 128)])
def test_quantize_bit_exact(lib, dtype, shift, bits, G):
    w = W.dense_weight(21, 3 * G, dtype, seed=bits + G)
    wd = off(dev_x(w, dtype), shift)
    packed = torch.empty((21, 3 * G * bits // 32), dtype=torch.int32, device="cuda")
    sc = torch.empty((21, 3), dtype=torch.bfloat16, device="cuda")
    bi = torch.empty((21, 3), dtype=torch.bfloat16, device="cuda")
    banner(f"misaligned quantize {dtype} shift={shift} bits={bits} G={G}")
    _lib.check(lib.qaff_quantize(P(wd), BF16 if dtype == "bf16" else F32, 21, 3 * G, G, bits, P(packed), P(sc), P(bi),
                                 S()))
    torch.cuda.synchronize()
    rp, rs, rb = orc_mod.quantize(w, dtype, G, bits)
    np.testing.assert_array_equal(packed.cpu().numpy().view(np.uint32), rp)
    np.testing.assert_array_equal(host_bits(sc), rs)
    np.testing.assert_array_equal(host_bits(bi), rb)


@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_qmm_nt(lib, x_dtype):
    k, n, m = 300, 4 * 64, 3
    inp = W.random_inputs(4, 64, k, n, 0, seed=17)        # a [k, n] weight
    xh = np.random.default_rng(18).standard_normal((m, k)).astype(np.float32)
    if x_dtype == "bf16":
        xh = W.bf16_bits_from_f32(xh)
    p, s, b = dev_weights(inp)
    x = off(dev_x(xh, x_dtype))
    tdt = torch.bfloat16 if x_dtype == "bf16" else torch.float32
    y = empty_off((m, n), tdt)
    need = int(lib.qaff_qmm_nt_workspace_size(m, k, n, 4))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    banner(f"misaligned qmm_nt x={x_dtype}")
    _lib.check(lib.qaff_qmm_nt(P(x), BF16 if x_dtype == "bf16" else F32, m, P(p), P(s), P(b), k, n, 64, 4, P(ws), need,
                               P(y), S()))
    torch.cuda.synchronize()
    ref = orc_mod.qmm_nt(xh, x_dtype, inp.packed, inp.scales, inp.biases, 64, 4)
    assert orc_mod.max_row_rel_err(host_f64(y), ref) <= TIGHT[x_dtype]


def test_typed(lib):
    inp = W.random_inputs(4, 64, 120, 1024, 2, seed=19)
    s16 = W.f32_from_bf16_bits(inp.scales).astype(np.float16).view(np.uint16)
    b16 = W.f32_from_bf16_bits(inp.biases).astype(np.float16).view(np.uint16)
    x16 = W.f32_from_bf16_bits(inp.x).astype(np.float16).view(np.uint16)
    p = dev_u32(inp.packed)
    h = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.float16)
    sd, bd, x = h(s16), h(b16), off(h(x16))
    y = empty_off((2, 120), torch.float16)
    banner("misaligned typed qmm and dequantize")
    _lib.check(lib.qaff_qmm_typed(P(x), F16, 2, P(p), P(sd), P(bd), F16, 120, 1024, 64, 4, P(y), S()))
    o = empty_off((120, 1024), torch.float16)
    _lib.check(lib.qaff_dequantize_typed(P(p), P(sd), P(bd), F16, 120, 1024, 64, 4, P(o), F16, S()))
    torch.cuda.synchronize()
    ref = orc_mod.qmm_typed(x16, "f16", inp.packed, s16, b16, "f16", 64, 4)
    assert orc_mod.max_row_rel_err(y.float().cpu().numpy().astype(np.float64), ref) <= 1e-3
    dref = orc_mod.dequantize_typed(inp.packed, s16, b16, "f16", 64, 4, out="f16")
    np.testing.assert_array_equal(o.cpu().view(torch.int16).numpy().view(np.uint16), dref)


# Scales and biases at a 2-byte offset (their element size of alignment) on every decode and GEMM
# route: the long-row VALU GEMV (its staged scale windows need 4-byte words, so it takes the
# per-block loads), the matrix-core decode kernels (4-byte words: the VALU GEMV instead), and the
# GEMM (its general variant's element loads); bf16 through qaff_qmm and float16 through
# qaff_qmm_typed.
@pytest.mark.parametrize("m,k", [(1, 14336), (4, 4096), (4, 14336), (40, 2048)])
def test_scales_at_two_byte_offset(lib, m, k):
    G, bits, n = 64, 4, 96
    inp = W.random_inputs(bits, G, n, k, m, seed=m + k)
    p, s, b = dev_weights(inp)
    so, bo = off(s), off(b)
    banner(f"scales at a 2-byte offset m={m} k={k}")
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    xb = dev_x(inp.x, "bf16")
    _lib.check(lib.qaff_qmm(P(xb), BF16, m, P(p), P(so), P(bo), n, k, G, bits, P(y), S()))
    torch.cuda.synchronize()
    ref = orc_mod.qmm(inp.x, "bf16", inp.packed, inp.scales, inp.biases, G, bits)
    # the GEMM multiplies bf16-rounded weights: the parity bound against the float32 weights
    assert orc_mod.max_row_rel_err(host_f64(y), ref) <= (1.6e-2 if m > 16 else TIGHT["bf16"])
    # float16 x, scales and biases
    to16 = lambda a: W.f32_from_bf16_bits(a).astype(np.float16).view(np.uint16)
    s16, b16, x16 = to16(inp.scales), to16(inp.biases), to16(inp.x)
    h = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.float16)
    y16 = torch.empty((m, n), dtype=torch.float16, device="cuda")
    # every operand held in a variable for the call (a temporary's memory would go back to the
    # allocator as soon as its address is taken, and the next one could reuse it)
    xd, sd, bd = h(x16), off(h(s16)), off(h(b16))
    _lib.check(lib.qaff_qmm_typed(P(xd), F16, m, P(p), P(sd), P(bd), F16, n, k, G, bits, P(y16), S()))
    torch.cuda.synchronize()
    ref16 = orc_mod.qmm_typed(x16, "f16", inp.packed, s16, b16, "f16", G, bits)
    assert orc_mod.max_row_rel_err(y16.float().cpu().numpy().astype(np.float64), ref16) <= 1e-3
