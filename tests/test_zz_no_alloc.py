"""qaff_qmm_nt_static (the product without the transpose for callers that cannot allocate) through
the C ABI: its output equals qaff_qmm_nt's with a caller workspace, bit for bit (the same kernels),
on consecutive calls that share the per-device scratch array, the second with a smaller input."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as orc_mod
from gpu_util import banner, dev_weights, dev_x
from quantized_matmul_mlx_amd import _lib
from quantized_matmul_mlx_amd import workloads as W

pytestmark = pytest.mark.gpu

DT = {"bf16": _lib.QAFF_BF16, "f32": _lib.QAFF_F32}


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return _lib.load()


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def both(lib, bits, G, m, k, n, x_dtype, seed):
    """The same product through qaff_qmm_nt (workspace) and qaff_qmm_nt_static."""
    inp = W.random_inputs(bits, G, k, n, 0, seed=seed)       # a [k, n] weight: groups along n
    xh = np.random.default_rng(seed + 1).standard_normal((m, k)).astype(np.float32)
    if x_dtype == "bf16":
        xh = W.bf16_bits_from_f32(xh)
    p, s, b = dev_weights(inp)
    x = dev_x(xh, x_dtype)
    tdt = torch.bfloat16 if x_dtype == "bf16" else torch.float32
    y_ws = torch.full((m, n), float("nan"), dtype=tdt, device="cuda")
    y_st = torch.full((m, n), float("nan"), dtype=tdt, device="cuda")
    need = int(lib.qaff_qmm_nt_workspace_size(m, k, n, bits))
    assert 0 < need <= int(lib.qaff_qmm_nt_static_max_bytes())
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    args = (x.data_ptr(), DT[x_dtype], m, p.data_ptr(), s.data_ptr(), b.data_ptr(), k, n, G, bits)
    _lib.check(lib.qaff_qmm_nt(*args, ws.data_ptr(), need, y_ws.data_ptr(), stream()))
    _lib.check(lib.qaff_qmm_nt_static(*args, y_st.data_ptr(), stream()))
    torch.cuda.synchronize()
    return inp, xh, y_ws, y_st


def test_static_scratch_matches_workspace_on_consecutive_calls(lib):
    orc_mod.build()
    # the first call fills more of the scratch than the second reads
    cases = [(4, 64, 3, 4096, 4096, "bf16", 1), (4, 64, 1, 1024, 2048, "bf16", 2), (3, 32, 2, 640, 96, "f32", 3)]
    for bits, G, m, k, n, xd, seed in cases:
        banner(f"qaff_qmm_nt_static bits={bits} G={G} m={m} k={k} n={n} x={xd}")
        inp, xh, y_ws, y_st = both(lib, bits, G, m, k, n, xd, seed)
        view = torch.int16 if xd == "bf16" else torch.int32
        assert torch.equal(y_st.view(view), y_ws.view(view)), "static scratch differs from the workspace"
        # and the product itself is right (the oracle's float64 product, the qmm bar)
        ref = orc_mod.qmm_nt(xh, xd, inp.packed, inp.scales, inp.biases, G, bits)
        err = orc_mod.max_row_rel_err(y_st.float().cpu().numpy().astype(np.float64), ref)
        assert err <= (1.6e-2 if xd == "bf16" else 2e-3), err


def test_static_scratch_rejects_sizes_past_its_maximum(lib):
    # 300 chunks of 128 rows x 2 rows x 4096 columns of float32 partial sums: more than 8 MiB
    m, k, n = 2, 128 * 300, 4096
    assert lib.qaff_qmm_nt_workspace_size(m, k, n, 4) > lib.qaff_qmm_nt_static_max_bytes()
    a = ctypes.c_void_p(0x10000)
    rc = lib.qaff_qmm_nt_static(a, _lib.QAFF_BF16, m, a, a, a, k, n, 64, 4, a, None)
    assert rc == _lib.QAFF_ERR_UNSUPPORTED
    assert b"static scratch" in lib.qaff_last_error()
