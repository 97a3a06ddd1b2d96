"""The product without the transpose, y = x . dequantize(W) for W stored [k, n], on the GPU against
the CPU oracle through the C ABI (via the binding).

Bars as for qmm: per-row max relative error against the float64 oracle of at most 2e-3 (float32 y)
and 1.6e-2 (bf16 y). The kernel multiplies float32 weights (x s times the code, plus x b), so the
tight bound from its own arithmetic (1e-4 / 4e-3) applies against the oracle itself.
"""
import numpy as np
import pytest
import torch

import oracle as orc_mod
from gpu_util import banner, dev_weights, dev_x, host_f64
from quantized_matmul_mlx_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-3, "bf16": 1.6e-2}
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


def run_check(orc, bits, G, k, n, m, x_dtype, seed):
    inp = W.random_inputs(bits, G, k, n, 0, seed=seed)       # a [k, n] weight: groups along n
    x = np.random.default_rng(seed + 1).standard_normal((m, k)).astype(np.float32)
    if x_dtype == "bf16":
        x = W.bf16_bits_from_f32(x)
    p, s, b = dev_weights(inp)
    y = qaff().qmm(dev_x(x, x_dtype), p, s, b, G, bits, transpose=False)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (m, n)
    ref = orc.qmm_nt(x, x_dtype, inp.packed, inp.scales, inp.biases, G, bits)
    got = host_f64(y)
    assert np.isfinite(got).all()
    err = orc.max_row_rel_err(got, ref)
    assert err <= TIGHT[x_dtype], f"max row rel err {err:.3e} > {TIGHT[x_dtype]}"
    return y


@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_qmm_nt(orc, x_dtype, bits, G):
    # k = 100 rows (not a multiple of the 16 row phases), n = 5 G (a ragged column tile), M = 3
    # (a slice of 2 rows and one of 1)
    banner(f"qmm_nt {x_dtype} bits={bits} G={G}")
    run_check(orc, bits, G, 100, 5 * G, 3, x_dtype, seed=bits * 100 + G)


@pytest.mark.parametrize("m,k,n", [(1, 4096, 4096), (2, 777, 1024), (5, 2048, 544), (1, 16, 32), (4, 9000, 96)])
def test_qmm_nt_shapes(orc, m, k, n):
    banner(f"qmm_nt m={m} k={k} n={n}")
    run_check(orc, 4, 32, k, n, m, "bf16", seed=m + k + n)


def test_qmm_nt_one_dim_x_and_k_zero(orc):
    inp = W.random_inputs(4, 64, 64, 128, 0, seed=3)
    p, s, b = dev_weights(inp)
    x = W.bf16_bits_from_f32(np.random.default_rng(4).standard_normal(64).astype(np.float32))
    banner("qmm_nt 1-D x")
    y = qaff().qmm(dev_x(x, "bf16"), p, s, b, 64, 4, transpose=False)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (128,)
    ref = orc.qmm_nt(x[None], "bf16", inp.packed, inp.scales, inp.biases, 64, 4)
    assert orc.max_row_rel_err(host_f64(y)[None], ref) <= TIGHT["bf16"]
    # determinism: the K chunks are added in a fixed order
    y2 = qaff().qmm(dev_x(x, "bf16"), p, s, b, 64, 4, transpose=False)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


@pytest.mark.parametrize("m,k,n", [(1, 5000, 2048), (4, 4096, 14336), (3, 4097, 3072), (1, 1, 2048)])
def test_qmm_nt_wide_shapes(orc, m, k, n):
    # wide outputs, K with a ragged last chunk, a single row of K
    banner(f"qmm_nt wide m={m} k={k} n={n}")
    run_check(orc, 4, 64, k, n, m, "bf16", seed=m + k + n + 1)
