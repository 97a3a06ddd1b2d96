"""The fused decode products (spark_runtime gemv_gate_up, gemv_silu_gate, gemv_silu_gate_resid) on
the GPU through the C ABI, against the oracle.

Bars as for qmm (tests/test_gpu_parity.py): per-row max relative error of at most 1.6e-2 against
the float64 oracle, and 4e-3 against the kernel's own arithmetic composed from the oracle's pieces.
For the silu product that reference rounds h = silu(gate) * up to bf16 (the kernel's input to the
product, by the reading in include/qaff.h) before the float64 matmul; h's float32 rounding on the
GPU may still differ from it by one bf16 step in rare elements, which moves y far less than 4e-3.
"""
import numpy as np
import pytest
import torch

import oracle as orc_mod
from gpu_util import banner, dev_weights, dev_x, host_f64
from quantized_matmul_mlx_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL, TIGHT = 1.6e-2, 4e-3
KB_FOR_G = {32: 97, 64: 98, 128: 100}   # ragged: not a multiple of the 64 lanes


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


def bf16_rand(rng, shape, scale=1.0):
    return W.bf16_bits_from_f32((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("m", [1, 3, 16])
def test_gate_up(orc, bits, G, m):
    k = KB_FOR_G[G] * 32
    a = W.random_inputs(bits, G, 150, k, m, seed=bits * 5 + G + m)
    b = W.random_inputs(bits, G, 150, k, m, seed=bits * 5 + G + m + 1000)
    banner(f"gate_up bits={bits} G={G} m={m}")
    x = dev_x(a.x, "bf16")
    gw, uw = dev_weights(a), dev_weights(b)
    gy, uy = qaff().gemv_gate_up(x, gw, uw, G, bits)
    torch.cuda.synchronize()
    for inp, y in ((a, gy), (b, uy)):
        ref = orc.qmm(a.x, "bf16", inp.packed, inp.scales, inp.biases, G, bits)
        assert orc.max_row_rel_err(host_f64(y), ref) <= TIGHT
    # the same arithmetic as the VALU GEMV on each weight alone, to the bit
    for w, y in ((gw, gy), (uw, uy)):
        y1 = qaff().qmm(x, *w, G, bits, path="gemv")
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("m,with_resid", [(1, False), (1, True), (3, True), (16, False)])
def test_silu_gate(orc, bits, G, m, with_resid):
    k = KB_FOR_G[G] * 32
    inp = W.random_inputs(bits, G, 150, k, m, seed=bits * 7 + G + m)
    rng = np.random.default_rng(bits * 100 + G + m)
    gate = bf16_rand(rng, (m, k), 2.0)
    up = bf16_rand(rng, (m, k))
    resid = bf16_rand(rng, (m, 150), 0.5) if with_resid else None
    banner(f"silu_gate bits={bits} G={G} m={m} resid={with_resid}")
    p, s, b = dev_weights(inp)
    y = qaff().gemv_silu_gate(dev_x(gate, "bf16"), dev_x(up, "bf16"), p, s, b, G, bits,
                              resid=dev_x(resid, "bf16") if with_resid else None)
    torch.cuda.synchronize()
    got = host_f64(y)
    ref = orc.silu_gate_qmm(gate, up, resid, inp.packed, inp.scales, inp.biases, G, bits)
    assert np.isfinite(got).all()
    assert orc.max_row_rel_err(got, ref) <= TOL
    h16 = orc.f32_to_bf16(orc.silu_gate(gate, up).astype(np.float32))
    tight = orc.qmm(h16, "bf16", inp.packed, inp.scales, inp.biases, G, bits)
    if with_resid:
        tight = tight + W.f32_from_bf16_bits(resid)
    assert orc.max_row_rel_err(got, tight) <= TIGHT


def test_fused_ffn_decode_shapes(orc):
    # a decode FFN step at 4-bit g64: gate and up [14336, 4096] on x [1, 4096], then down
    # [4096, 14336] on silu(gate) * up with the residual
    wl_up = W.Workload("ffn_up_4bit_g64_14336x4096", 4, 64, 14336, 4096, (1e-3, 2e-2), (-0.15, 0.0),
                       ms=(1,), x_dtype="bf16", seed=21)
    a = W.make_inputs(wl_up, m=1)
    b = W.make_inputs(W.Workload("ffn_gate_4bit_g64_14336x4096", 4, 64, 14336, 4096, (1e-3, 2e-2),
                                 (-0.15, 0.0), ms=(1,), x_dtype="bf16", seed=22), m=1)
    banner("ffn decode gate_up 14336x4096")
    gy, uy = qaff().gemv_gate_up(dev_x(a.x, "bf16"), dev_weights(b), dev_weights(a), 64, 4)
    torch.cuda.synchronize()
    for inp, y in ((b, gy), (a, uy)):
        ref = orc.qmm(a.x, "bf16", inp.packed, inp.scales, inp.biases, 64, 4)
        assert orc.max_row_rel_err(host_f64(y), ref) <= TIGHT
    down = W.make_inputs(W.Workload("ffn_down_4bit_g64_4096x14336", 4, 64, 4096, 14336, (1e-3, 2e-2),
                                    (-0.15, 0.0), ms=(1,), x_dtype="bf16", seed=23), m=1)
    rng = np.random.default_rng(24)
    resid = bf16_rand(rng, (1, 4096))
    banner("ffn decode silu_gate 4096x14336 + residual")
    g16 = gy.view(torch.int16).cpu().numpy().view(np.uint16)
    u16 = uy.view(torch.int16).cpu().numpy().view(np.uint16)
    y = qaff().gemv_silu_gate(gy, uy, *dev_weights(down), 64, 4, resid=dev_x(resid, "bf16"))
    torch.cuda.synchronize()
    ref = orc.silu_gate_qmm(g16, u16, resid, down.packed, down.scales, down.biases, 64, 4)
    assert orc.max_row_rel_err(host_f64(y), ref) <= TOL


def test_silu_gate_k_zero_copies_the_residual(orc):
    p = torch.zeros((8, 0), dtype=torch.int32, device="cuda")
    s = torch.zeros((8, 0), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((2, 0), dtype=torch.bfloat16, device="cuda")
    r = torch.randn((2, 8), device="cuda").to(torch.bfloat16)
    banner("silu_gate k=0")
    y = qaff().gemv_silu_gate(g, g, p, s, s, 32, 4, resid=r)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), r.view(torch.int16))
