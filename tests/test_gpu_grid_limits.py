"""Launches that split their grid: one grid dimension holds at most 65535 blocks, so long x (the
GEMVs' rows of x per block), many output batches (the gathered products), many experts (the
grouped walk) and many output rows (dequantize, dequant_rows) go out in several launches. Checked against the CPU oracle at the smallest sizes
that cross the limit (k small so that the oracle finishes in seconds)."""
import numpy as np
import pytest
import torch

import oracle as orc_mod
from gpu_util import banner, dev_bf16, dev_u32, dev_weights, dev_x, host_bits, host_f64
from quantized_matmul_mlx_amd import workloads as W

pytestmark = pytest.mark.gpu

TIGHT = {"f32": 1e-4, "bf16": 4e-3}


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


@pytest.mark.parametrize("x_dtype,m", [("f32", 65535 * 4 + 7), ("bf16", 65535 * 8 + 9)])
def test_gemv_over_m_slices(orc, x_dtype, m):
    # the VALU GEMV takes 4 (float32) or 8 (bf16) x rows per block in grid y
    inp = W.random_inputs(4, 32, 40, 32, m, x_dtype=x_dtype, seed=m % 97)
    banner(f"gemv m={m} {x_dtype} (several launches)")
    p, s, b = dev_weights(inp)
    y = qaff().qmm(dev_x(inp.x, x_dtype), p, s, b, 32, 4, path="gemv")
    torch.cuda.synchronize()
    ref = orc.qmm(inp.x, x_dtype, inp.packed, inp.scales, inp.biases, 32, 4)
    got = host_f64(y)
    # every row, and the rows at the launch boundaries in particular
    assert orc.max_row_rel_err(got, ref) <= TIGHT[x_dtype]


def test_gather_over_batch_slices(orc):
    # the VALU gathered GEMV: grid z = output batch, 65535 per launch
    E, n, k, G, bits, batch = 3, 40, 64, 32, 4, 65535 + 300
    inp = W.random_inputs(bits, G, E * n, k, 0, seed=5)
    packed, scales, biases = (inp.packed.reshape(E, n, -1), inp.scales.reshape(E, n, -1),
                              inp.biases.reshape(E, n, -1))
    rng = np.random.default_rng(6)
    x = W.bf16_bits_from_f32(rng.standard_normal((7, 1, k)).astype(np.float32))
    lhs = rng.integers(0, 7, batch).astype(np.uint32)
    rhs = rng.integers(0, E, batch).astype(np.uint32)
    banner(f"gather batch={batch} (several launches)")
    y = qaff().gather_qmm(dev_x(x, "bf16"), dev_u32(packed), dev_bf16(scales), dev_bf16(biases), G, bits,
                          lhs_indices=dev_u32(lhs), rhs_indices=dev_u32(rhs), path="gemv")
    torch.cuda.synchronize()
    # one oracle call per batch: single-threaded, so that no thread pool starts 65835 times
    ref = orc.gather_qmm(x, "bf16", packed, scales, biases, G, bits, lhs=lhs, rhs=rhs, threads=1)
    assert orc.max_row_rel_err(host_f64(y).reshape(-1, n), ref.reshape(-1, n)) <= TIGHT["bf16"]


def test_grouped_walk_over_expert_slices(orc):
    # the grouped walk: grid y = experts + 1, 65535 per launch; 70000 experts of [16, 512]
    E, n, k, G, bits = 70000, 16, 512, 128, 2
    inp = W.random_inputs(bits, G, E * n, k, 0, seed=7)
    packed, scales, biases = (inp.packed.reshape(E, n, -1), inp.scales.reshape(E, n, -1),
                              inp.biases.reshape(E, n, -1))
    rng = np.random.default_rng(8)
    rhs = np.sort(rng.integers(0, E, 2000)).astype(np.uint32)
    rhs[-3:] = E - 1                                         # rows for the last expert (the last launch)
    rhs = np.sort(rhs)
    x = W.bf16_bits_from_f32(rng.standard_normal((rhs.size, 1, k)).astype(np.float32))
    banner(f"grouped walk over {E} experts (several launches)")
    y = qaff().gather_qmm(dev_x(x, "bf16"), dev_u32(packed), dev_bf16(scales), dev_bf16(biases), G, bits,
                          rhs_indices=dev_u32(rhs), sorted_indices=True, path="gemv_mfma")
    torch.cuda.synchronize()
    ref = orc.gather_qmm(x, "bf16", packed, scales, biases, G, bits, rhs=rhs, threads=1)
    got = host_f64(y).reshape(-1, n)
    assert np.isfinite(got).all()
    assert orc.max_row_rel_err(got, ref.reshape(-1, n)) <= 1.6e-2


def test_typed_gather_over_batch_slices(orc):
    # the typed gathered GEMV: grid z = output batch, 65535 per launch (float16 x, float32 scales)
    E, n, k, G, bits, batch = 3, 40, 64, 32, 4, 65535 + 300
    inp = W.random_inputs(bits, G, E * n, k, 0, seed=9)
    packed = inp.packed.reshape(E, n, -1)
    rng = np.random.default_rng(10)
    sc = rng.uniform(1e-3, 2e-2, (E, n, k // G)).astype(np.float32)
    bi = rng.uniform(-0.15, 0.0, (E, n, k // G)).astype(np.float32)
    x = rng.standard_normal((7, 1, k)).astype(np.float16)
    lhs = rng.integers(0, 7, batch).astype(np.uint32)
    rhs = rng.integers(0, E, batch).astype(np.uint32)
    rhs[-5:] = E + 2                                          # NaN batches in the last launch
    banner(f"typed gather batch={batch} (several launches)")
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.float16)
    y = qaff().gather_qmm(xd, dev_u32(packed), torch.from_numpy(sc).cuda(), torch.from_numpy(bi).cuda(), G, bits,
                          lhs_indices=dev_u32(lhs), rhs_indices=dev_u32(rhs))
    torch.cuda.synchronize()
    assert y.dtype == torch.float32
    ref = orc.gather_qmm_typed(x.view(np.uint16), "f16", packed, sc, bi, "f32", G, bits, lhs=lhs, rhs=rhs)
    got = host_f64(y).reshape(-1, n)
    ref = ref.reshape(-1, n)
    nan = np.isnan(ref).all(axis=1)
    assert nan.sum() == 5 and np.isnan(got[nan]).all()
    assert orc.max_row_rel_err(got[~nan], ref[~nan]) <= TIGHT["f32"]


OUTS = (("f32", torch.float32, np.uint32), ("bf16", torch.bfloat16, np.uint16))


def test_dequantize_over_row_slices(orc):
    # grid y = output rows, 65535 per launch; 3-bit codes straddle words
    rows, cols, G, bits = 65535 + 37, 96, 32, 3
    inp = W.random_inputs(bits, G, rows, cols, 0, seed=8)
    p, s, b = dev_weights(inp)
    for out, tdt, view in OUTS:
        banner(f"dequantize rows={rows} -> {out} (several launches)")
        got = host_bits(qaff().dequantize(p, s, b, G, bits, tdt))
        ref = orc.dequantize(inp.packed, inp.scales, inp.biases, G, bits, out=out)
        np.testing.assert_array_equal(got.view(view), ref.view(view))


def test_dequant_rows_over_index_slices(orc):
    # grid y = indices, 65535 per launch; some indices past the table (rows of NaN)
    table, cols, G, bits = 300, 64, 32, 4
    inp = W.random_inputs(bits, G, table, cols, 0, seed=9)
    idx = np.random.default_rng(10).integers(0, table, 65535 + 41).astype(np.uint32)
    idx[[5, 65534, 65535, 65560]] = [table, 2**32 - 1, table + 7, 0]
    p, s, b = dev_weights(inp)
    it = torch.from_numpy(idx.view(np.int32)).cuda()
    for out, tdt, view in OUTS:
        banner(f"dequant_rows {idx.size} indices -> {out} (several launches)")
        got = host_bits(qaff().dequant_rows(p, s, b, it, G, bits, tdt))
        ref = orc.dequant_rows(inp.packed, inp.scales, inp.biases, idx, G, bits, out=out)
        np.testing.assert_array_equal(got.view(view), ref.view(view))


def test_dequantize_past_2_pow_31_elements_per_launch(orc):
    # 65535 + 17 rows of 65536 codes: the first launch covers 2^32 - 2^16 outputs, so element
    # offsets pass 2^31 inside one launch, and the float32 output (17.2 GB) passes 2^34 bytes.
    # Inputs drawn on the device from a seeded generator (any words are valid codes); the output
    # starts as NaN, so that every element must be written, and whole rows on both sides of each
    # boundary are compared with the oracle to the bit.
    rows, cols, G, bits = 65535 + 17, 65536, 64, 4
    gen = torch.Generator(device="cuda").manual_seed(11)
    p = torch.randint(-2**31, 2**31 - 1, (rows, cols * bits // 32), dtype=torch.int32, device="cuda",
                      generator=gen)
    s = torch.empty((rows, cols // G), device="cuda").uniform_(1e-3, 2e-2, generator=gen).to(torch.bfloat16)
    b = torch.empty((rows, cols // G), device="cuda").uniform_(-0.15, 0.0, generator=gen).to(torch.bfloat16)
    sel = np.array([0, 1, 32767, 32768, 65534, 65535, 65536, rows - 1])
    st = torch.from_numpy(sel).cuda()
    hp = p[st].cpu().numpy().view(np.uint32)
    hs, hb = (host_bits(t[st]) for t in (s, b))
    for out, tdt, view in OUTS:
        banner(f"dequantize {rows}x{cols} -> {out} (past 2^31 elements per launch)")
        buf = torch.full((rows, cols), float("nan"), dtype=tdt, device="cuda")
        qaff().dequantize(p, s, b, G, bits, tdt, out=buf)
        assert not bool(torch.isnan(buf).any())
        got = host_bits(buf[st])
        del buf
        torch.cuda.empty_cache()
        ref = orc.dequantize(hp, hs, hb, G, bits, out=out)
        np.testing.assert_array_equal(got.view(view), ref.view(view))
