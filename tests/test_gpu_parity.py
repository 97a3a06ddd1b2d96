"""Parity of the HIP path with the CPU oracle, on the GPU, through the C ABI (via the binding).

Bars:
* dequantize / dequant_rows: bit-exact, float32 and bf16 (both sides form s*c in float32, add the
  bias in float32, and round bf16 to nearest even).
* qmm: per-row max relative error (max_n |y - ref| / max_n |ref|) against the float64 oracle of at
  most 2e-3 for float32 y and 1.6e-2 for bf16 y.
* A tighter check, derived from each kernel's arithmetic, catches single-code mistakes that the
  bars above would let through. Its reference is the oracle's own pieces composed the way the kernel
  computes: the VALU GEMV uses the float32 weights (the oracle as is), the two MFMA kernels (GEMM
  and matrix-core decode) their weights rounded to bf16 (the oracle's bf16 dequantization, then a
  float64 matmul), except where the matrix-core decode kernel takes 4-bit codes exactly (scale and
  bias applied to each group's sums: the oracle as is). What is left is float32
  summation order (~1e-6 relative) and, for a bf16 y, one rounding of each output to nearest even:
  bf16 keeps 8 significant bits, so that rounding moves y by at most 2^-8 = 3.91e-3 of |y| <=
  max|ref|. Bound: 4e-3 for bf16 y, 1e-4 for float32 y.
"""
import numpy as np
import pytest
import torch

import oracle as orc_mod
from gpu_util import at_offset, banner, dev_weights, dev_x, host_bits, host_f64, mfma_exact_codes
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


def run_qmm(inp, m_rows=None, path="auto"):
    packed, scales, biases = dev_weights(inp)
    x = dev_x(inp.x, inp.x_dtype)
    y = qaff().qmm(x, packed, scales, biases, inp.wl.group_size, inp.wl.bits, path=path)
    torch.cuda.synchronize()
    return y


def mfma_decode_takes(inp):
    """Shapes the matrix-core decode kernel takes: 1 <= m <= 16, k a multiple of 512 up to 32768."""
    m, k = inp.x.shape[0], inp.wl.k
    return 1 <= m <= 16 and k % 512 == 0 and k <= 32768


def kernel_of(inp, path):
    """Which kernel ran: "gemm" (bf16-MFMA GEMM), "gemv_mfma" (matrix-core decode kernel) or
    "gemv" (VALU GEMV), as the dispatch in the library picks them."""
    m = inp.x.shape[0]
    if inp.x_dtype != "bf16":
        return "gemv"
    wl = inp.wl
    if path == "auto" and decode_slices(m, wl.n, wl.k) and \
            qaff()._lib.load().qaff_qmm_workspace_size(m, wl.n, wl.k, wl.group_size, wl.bits) == 0:
        return "slices"
    if path == "gemm" or (path == "auto" and m > qaff().gemv_max_m()):
        return "gemm"
    # the binding's automatic path passes a workspace when one is sized: decode-sized m beyond
    # the matrix-core decode kernel's K range then take the GEMM with K split
    wl = inp.wl
    if path == "auto" and qaff()._lib.load().qaff_qmm_workspace_size(m, wl.n, wl.k, wl.group_size, wl.bits) > 0:
        return "gemm"
    if path == "gemv_mfma" or (path == "auto" and m >= qaff().gemv_mfma_min_m(wl.k) and mfma_decode_takes(inp)):
        return "gemv_mfma"
    return "gemv"


def decode_slices(m, n, k):
    """Where the automatic path runs 17 to 128 rows as 16-row slices of the decode path (with no K
    split): the matrix-core decode kernel takes K, and up to 3 slices at any n, 6 where n <= 8192,
    8 where n <= 4096."""
    s = (m + 15) // 16
    return 16 < m <= 128 and k % 512 == 0 and 0 < k <= 32768 and (s <= 3 or (s <= 6 and n <= 8192) or n <= 4096)


def slices_of(inp, path="auto"):
    """The automatic path's result row slice by slice: each 16-row slice as a call of its own."""
    packed, scales, biases = dev_weights(inp)
    x = dev_x(inp.x, inp.x_dtype)
    m = inp.x.shape[0]
    ys = [qaff().qmm(x[m0:m0 + 16], packed, scales, biases, inp.wl.group_size, inp.wl.bits, path=path)
          for m0 in range(0, m, 16)]
    torch.cuda.synchronize()
    return torch.cat(ys)


def bf16_weight_ref(orc, inp, x_rows):
    """x . bf16(W)^T in float64: the oracle's bf16 dequantization, widened, through numpy matmul."""
    wl = inp.wl
    w16 = orc.dequantize(inp.packed, inp.scales, inp.biases, wl.group_size, wl.bits, out="bf16")
    w = orc.bf16_to_f32(w16).astype(np.float64)
    x = orc.bf16_to_f32(x_rows).astype(np.float64)
    return x @ w.T


def check_qmm(orc, inp, y, rows=None, path="auto", kernel=None):
    wl = inp.wl
    x = inp.x if rows is None else inp.x[rows]
    ref = orc.qmm(x, inp.x_dtype, inp.packed, inp.scales, inp.biases, wl.group_size, wl.bits)
    got = host_f64(y) if rows is None else host_f64(y)[rows]
    assert np.isfinite(got).all()
    err = orc.max_row_rel_err(got, ref)
    kind = inp.x_dtype
    assert err <= TOL[kind], f"max row rel err {err:.3e} > {TOL[kind]}"
    # both MFMA kernels multiply bf16-rounded weights, except the matrix-core decode kernel with
    # exact 4-bit codes
    kernel = kernel or kernel_of(inp, path)
    exact = kernel == "gemv_mfma" and mfma_exact_codes(wl.bits, wl.group_size, inp.x.shape[0])
    tight_ref = ref if kernel == "gemv" or exact else bf16_weight_ref(orc, inp, x)
    if kernel == "slices":   # each slice against the arithmetic of the kernel that ran it
        wref = bf16_weight_ref(orc, inp, x)
        tight_ref = ref.copy()
        m = inp.x.shape[0]
        for m0 in range(0, m, 16):
            mm = min(16, m - m0)
            on_mfma = mm >= qaff().gemv_mfma_min_m(wl.k)
            if on_mfma and not mfma_exact_codes(wl.bits, wl.group_size, mm):
                tight_ref[m0:m0 + mm] = wref[m0:m0 + mm]
    terr = orc.max_row_rel_err(got, tight_ref)
    assert terr <= TIGHT[kind], f"{kernel}: max row rel err {terr:.3e} against its " \
                                f"own arithmetic, above {TIGHT[kind]}"
    return err


# ---- the 4-bit g64 [256, 512] reference workload ------------------------------------------------

def test_ref_workload_dequant_bit_exact(orc):
    wl = W.WORKLOADS["ref_4bit_g64_256x512"]
    inp = W.make_inputs(wl, m=4)
    banner("ref dequant")
    p, s, b = dev_weights(inp)
    for out in ("f32", "bf16"):
        got = host_bits(qaff().dequantize(p, s, b, wl.group_size, wl.bits,
                                          torch.float32 if out == "f32" else torch.bfloat16))
        ref = orc.dequantize(inp.packed, inp.scales, inp.biases, wl.group_size, wl.bits, out=out)
        np.testing.assert_array_equal(got.view(np.uint32 if out == "f32" else np.uint16),
                                      ref.view(np.uint32 if out == "f32" else np.uint16))


def test_ref_workload_qmm_f32(orc):
    wl = W.WORKLOADS["ref_4bit_g64_256x512"]
    inp = W.make_inputs(wl, m=4)
    banner("ref qmm f32")
    y = run_qmm(inp)
    assert y.dtype == torch.float32 and tuple(y.shape) == (4, 256)
    check_qmm(orc, inp, y)


@pytest.mark.parametrize("path", ["gemv", "gemm"])
def test_ref_workload_qmm_bf16_paths(orc, path):
    wl = W.WORKLOADS["ref_4bit_g64_256x512"]
    inp = W.make_inputs(wl, m=4, x_dtype="bf16")
    banner(f"ref qmm bf16 {path}")
    y = run_qmm(inp, path=path)
    assert y.dtype == torch.bfloat16
    check_qmm(orc, inp, y, path=path)


# ---- dequantize at every bit width and group size ----------------------------------------------

@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
def test_dequant_bit_exact(orc, bits, G):
    inp = W.random_inputs(bits, G, 67, G * 6, 0, seed=100 + bits * 7 + G)
    banner(f"dequant bits={bits} G={G}")
    p, s, b = dev_weights(inp)
    for out, tdt, view in (("f32", torch.float32, np.uint32), ("bf16", torch.bfloat16, np.uint16)):
        got = host_bits(qaff().dequantize(p, s, b, G, bits, tdt))
        ref = orc.dequantize(inp.packed, inp.scales, inp.biases, G, bits, out=out)
        np.testing.assert_array_equal(got.view(view), ref.view(view))


# ---- GEMV and GEMM at every bit width, ragged shapes --------------------------------------------

KB_FOR_G = {32: 97, 64: 98, 128: 100}   # blocks per row: > 64 lanes, not a multiple of 64


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("m,x_dtype", [(1, "bf16"), (3, "bf16"), (16, "bf16"), (4, "f32"), (5, "f32")])
def test_gemv(orc, bits, G, m, x_dtype):
    k = KB_FOR_G[G] * 32
    inp = W.random_inputs(bits, G, 150, k, m, x_dtype=x_dtype, seed=bits * 31 + G + m)
    banner(f"gemv bits={bits} G={G} m={m} x={x_dtype}")
    y = run_qmm(inp, path="gemv")
    check_qmm(orc, inp, y, path="gemv")


# Long rows at M <= 2 take wider passes (8 or 4 blocks per lane): 300 blocks (one ragged pass) and
# 520 blocks (more than one pass at M = 1, ragged).
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("m,kb", [(1, 300), (2, 300), (1, 520)])
def test_gemv_long_rows(orc, bits, G, m, kb):
    k = kb * 32 // G * G
    inp = W.random_inputs(bits, G, 70, k, m, seed=bits * 3 + G + m + kb)
    banner(f"gemv long rows bits={bits} G={G} m={m} k={k}")
    y = run_qmm(inp, path="gemv")
    check_qmm(orc, inp, y, path="gemv")


@pytest.mark.parametrize("m", [1, 2])
def test_gemv_long_rows_scales_at_two_byte_offset(orc, m):
    # k = 14336 at G = 64 (an even number of groups per row): with 4-byte aligned scales the long
    # pass stages them through LDS in 16-byte loads; at a 2-byte offset it must read them per block
    inp = W.random_inputs(4, 64, 300, 14336, m, seed=41 + m)
    p, s, b = dev_weights(inp)
    s2, b2 = at_offset(s), at_offset(b)
    assert s2.data_ptr() % 4 == 2 and b2.data_ptr() % 4 == 2
    x = dev_x(inp.x, "bf16")
    banner(f"gemv long rows, scales at a 2-byte offset, m={m}")
    y = qaff().qmm(x, p, s2, b2, 64, 4, path="gemv")
    torch.cuda.synchronize()
    check_qmm(orc, inp, y, path="gemv")
    y_aligned = run_qmm(inp, path="gemv")
    assert torch.equal(y.view(torch.int16), y_aligned.view(torch.int16))


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G", [32, 128])
@pytest.mark.parametrize("m,n", [(17, 129), (130, 200), (257, 64)])
def test_gemm(orc, bits, G, m, n):
    k = (G // 32) * 7 * 32     # an odd number of 32-code blocks when G = 32: a ragged K tile
    inp = W.random_inputs(bits, G, n, k, m, seed=bits * 17 + G + m)
    banner(f"gemm bits={bits} G={G} m={m} n={n} k={k}")
    y = run_qmm(inp, path="gemm")
    check_qmm(orc, inp, y, path="gemm")


# K a multiple of 1024 takes the 128 x 256 tile kernel that dequantizes W into registers (at any m): every group size, ragged m and n tails, one to three 16-step loop iterations, and grids
# with and without the 4 x 8 tile blocks per XCD (512 x 2048: 4 x 8 tiles; the others are not
# multiples of 8 tiles).
@pytest.mark.parametrize("G,m,n,k", [(32, 256, 256, 1024), (64, 300, 520, 2048), (128, 512, 2048, 1024),
                                     (128, 257, 300, 3072), (32, 384, 1000, 2048)])
def test_gemm_direct_tiles(orc, G, m, n, k):
    inp = W.random_inputs(4, G, n, k, m, seed=G + m + n)
    banner(f"gemm direct G={G} m={m} n={n} k={k}")
    y = run_qmm(inp, path="gemm")
    check_qmm(orc, inp, y, path="gemm")


# Fewer than 256 rows of x take the same kernel (one or two rows of tiles, the rest of the tile
# clamped): m just above the decode range, a ragged single tile row, and one and a half tile rows.
@pytest.mark.parametrize("bits,G,m,n,k", [(4, 64, 17, 300, 1024), (4, 128, 100, 520, 2048), (3, 32, 200, 264, 1024),
                                          (8, 128, 33, 256, 2048)])
def test_gemm_direct_small_m(orc, bits, G, m, n, k):
    inp = W.random_inputs(bits, G, n, k, m, seed=bits + G + m + n)
    banner(f"gemm direct small m bits={bits} G={G} m={m} n={n} k={k}")
    y = run_qmm(inp, path="gemm")
    check_qmm(orc, inp, y, path="gemm")


# The automatic path of a bf16 x with few GEMM tiles splits K through a workspace that the binding
# allocates (qaff_qmm_ws): 8, 3, 4 and 14 ranges of 1024 codes with ragged m and n, and a shape with
# a single chunk of K, which cannot split. Against the oracle and against the unsplit kernel.
@pytest.mark.parametrize("bits,G,m,n,k,splits", [(4, 128, 17, 300, 8192, True), (4, 64, 100, 520, 3072, True),
                                                 (3, 32, 260, 264, 4096, True), (8, 128, 33, 256, 14336, True),
                                                 (4, 128, 300, 4096, 1024, False)])
def test_gemm_split_k(orc, bits, G, m, n, k, splits):
    inp = W.random_inputs(bits, G, n, k, m, seed=bits + G + m + n + k)
    lib = qaff()._lib.load()
    assert (lib.qaff_qmm_workspace_size(m, n, k, G, bits) > 0) == splits
    banner(f"gemm split K bits={bits} G={G} m={m} n={n} k={k}")
    y = run_qmm(inp, path="auto")
    check_qmm(orc, inp, y, path="auto")
    whole = run_qmm(inp, path="gemm")
    a, b = host_f64(y), host_f64(whole)
    assert orc.max_row_rel_err(a, b) <= 1e-2  # two float32 summation orders, each rounded to bf16


# Decode-sized m with K past the matrix-core decode kernel's range (32768 codes): from 8 rows on the
# automatic path takes the split GEMM (faster than the VALU GEMV there); below, the VALU GEMV.
@pytest.mark.parametrize("bits,G,m,k,gemm", [(4, 128, 8, 33792, True), (4, 64, 16, 34816, True),
                                             (6, 32, 12, 33792, True), (4, 128, 7, 33792, False)])
def test_decode_sized_m_split_gemm(orc, bits, G, m, k, gemm):
    n = 300
    inp = W.random_inputs(bits, G, n, k, m, seed=bits + G + m + k)
    assert (kernel_of(inp, "auto") == "gemm") == gemm
    banner(f"decode-sized m split gemm bits={bits} G={G} m={m} k={k}")
    y = run_qmm(inp, path="auto")
    check_qmm(orc, inp, y, path="auto")


# The same kernel at every other bit width (a block of 32 codes is BITS words; 3-, 5- and 6-bit
# codes straddle words), with a ragged tile in m and in n.
@pytest.mark.parametrize("bits", [1, 2, 3, 5, 6, 8])
@pytest.mark.parametrize("G,m,n,k", [(32, 260, 300, 1024), (128, 300, 520, 2048)])
def test_gemm_direct_widths(orc, bits, G, m, n, k):
    inp = W.random_inputs(bits, G, n, k, m, seed=bits * 7 + G + m)
    banner(f"gemm direct bits={bits} G={G} m={m} n={n} k={k}")
    y = run_qmm(inp, path="gemm")
    check_qmm(orc, inp, y, path="gemm")


# K that is not a whole number of 1024-code chunks: the kernel's general variant walks the whole
# chunks as usual and the remaining 64-code steps one at a time. K = 11008 (10 chunks and 12 steps),
# 4160 (65 groups of 64 per row: scale rows only 2-byte aligned), 1056 at G = 32 (33 blocks: half a
# step), 2176 and 3136 (short tails), and K below one chunk (only the tail).
@pytest.mark.parametrize("bits,G,m,n,k", [(4, 128, 300, 300, 11008), (4, 64, 257, 264, 4160), (3, 32, 130, 200, 1056),
                                          (8, 128, 64, 256, 2176), (5, 64, 200, 300, 3136), (6, 32, 140, 72, 800)])
def test_gemm_general_k_tails(orc, bits, G, m, n, k):
    inp = W.random_inputs(bits, G, n, k, m, seed=bits + G + m + k)
    banner(f"gemm K tail bits={bits} G={G} m={m} n={n} k={k}")
    y = run_qmm(inp, path="gemm")
    check_qmm(orc, inp, y, path="gemm")


# The same with K split through the workspace (the last split also takes the tail).
@pytest.mark.parametrize("bits,G,m,n,k", [(4, 128, 64, 300, 11008), (4, 64, 17, 520, 4160)])
def test_gemm_general_split_k(orc, bits, G, m, n, k):
    inp = W.random_inputs(bits, G, n, k, m, seed=bits + G + m + k + 1)
    assert qaff()._lib.load().qaff_qmm_workspace_size(m, n, k, G, bits) > 0
    banner(f"gemm K tail, split K, bits={bits} G={G} m={m} n={n} k={k}")
    y = run_qmm(inp, path="auto")
    check_qmm(orc, inp, y, path="auto")


# Scales and biases at a 2-byte offset with whole chunks of K: the general variant's element loads
# of the scale windows, the same arithmetic as the aligned kernel (equal bits).
def test_gemm_scales_at_two_byte_offset(orc):
    inp = W.random_inputs(4, 64, 300, 2048, 300, seed=97)
    p, s, b = dev_weights(inp)
    s2, b2 = at_offset(s), at_offset(b)
    assert s2.data_ptr() % 16 == 2 and b2.data_ptr() % 16 == 2
    banner("gemm, scales at a 2-byte offset")
    y = qaff().qmm(dev_x(inp.x, "bf16"), p, s2, b2, 64, 4, path="gemm")
    torch.cuda.synchronize()
    check_qmm(orc, inp, y, path="gemm")
    assert torch.equal(y.view(torch.int16), run_qmm(inp, path="gemm").view(torch.int16))


@pytest.mark.parametrize("m", [1, 2, 3, 4, 15, 16, 17, 18])
def test_dispatch_boundary_all_paths(orc, m):
    assert qaff().gemv_max_m() == 16
    inp = W.random_inputs(4, 64, 96, 1024, m, seed=m)
    banner(f"dispatch m={m}")
    paths = ("auto", "gemv", "gemm") + (("gemv_mfma",) if m <= 16 else ())
    ys = {p: run_qmm(inp, path=p) for p in paths}
    for p, y in ys.items():
        check_qmm(orc, inp, y, path=p)
    auto = kernel_of(inp, "auto")
    assert auto == ("slices" if m > 16 else "gemv_mfma" if m >= qaff().gemv_mfma_min_m() else "gemv")
    want = slices_of(inp) if auto == "slices" else ys[auto]
    assert torch.equal(ys["auto"].view(torch.int16), want.view(torch.int16))


# 17 to 128 rows through qaff_qmm (no workspace, so no K split): 16-row slices of the decode path,
# each equal to the slice run as a call of its own (bit for bit) and within the kernels' bars;
# the edges of the rule (n = 8192 at 64 and 96 rows against 100 rows, n = 4096 at 128 rows, n =
# 8200 at 64 rows), K past 4096 (two-row decode slices on the matrix cores), 3- and 5-bit codes,
# and K that the decode kernel does not take (the GEMM).
@pytest.mark.parametrize("bits,G,m,n,k", [(4, 64, 17, 150, 2048), (3, 32, 33, 300, 4096), (8, 128, 48, 96, 5120),
                                          (4, 64, 64, 8192, 1024), (4, 64, 96, 8192, 1024), (4, 64, 100, 8192, 1024),
                                          (4, 64, 128, 4096, 1024), (4, 64, 64, 8200, 1024), (6, 32, 50, 150, 1536),
                                          (5, 32, 113, 300, 2048), (4, 128, 18, 96, 8192), (4, 32, 20, 96, 1056)])
def test_decode_slices(orc, bits, G, m, n, k):
    import ctypes
    from quantized_matmul_mlx_amd import _lib
    inp = W.random_inputs(bits, G, n, k, m, seed=bits + G + m + n + k)
    packed, scales, biases = dev_weights(inp)
    x = dev_x(inp.x, "bf16")
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    banner(f"decode slices bits={bits} G={G} m={m} n={n} k={k}")
    _lib.check(_lib.load().qaff_qmm(P(x), _lib.QAFF_BF16, m, P(packed), P(scales), P(biases), n, k, G, bits, P(y),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    torch.cuda.synchronize()
    slices = decode_slices(m, n, k)
    check_qmm(orc, inp, y, kernel="slices" if slices else "gemm")
    if slices:
        assert torch.equal(y.view(torch.int16), slices_of(inp).view(torch.int16))
    else:
        assert torch.equal(y.view(torch.int16), run_qmm(inp, path="gemm").view(torch.int16))


# The matrix-core decode kernel: every width and group size, m from 1 to 16, ragged n (not a
# multiple of 16), K from one to eight 512-code slices, and n large enough for 2 and 4 row tiles
# per block.
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("m,n,k", [(1, 150, 512), (3, 150, 1536), (8, 77, 4096), (16, 150, 2048)])
def test_gemv_mfma(orc, bits, G, m, n, k):
    inp = W.random_inputs(bits, G, n, k, m, seed=bits * 13 + G + m + n)
    banner(f"gemv_mfma bits={bits} G={G} m={m} n={n} k={k}")
    y = run_qmm(inp, path="gemv_mfma")
    check_qmm(orc, inp, y, path="gemv_mfma")


# Tiles of 16 rows per block: with M = 16 and K = 4096 one block fills a compute unit's LDS, so on
# 256 compute units n = 4100, 8200 and 12300 take 2, 3 and 4 tiles per block (8-bit codes at most 2).
@pytest.mark.parametrize("bits,n", [(4, 4100), (4, 8200), (4, 12300), (3, 12300), (8, 12300)])
def test_gemv_mfma_row_tiles(orc, bits, n):
    inp = W.random_inputs(bits, 32, n, 4096, 16, seed=n + bits)
    banner(f"gemv_mfma row tiles bits={bits} n={n}")
    y = run_qmm(inp, path="gemv_mfma")
    check_qmm(orc, inp, y, path="gemv_mfma")


# The same tile counts at 4 bits with groups of 64 and 128.
@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("n", [4100, 8200, 12300])
def test_gemv_mfma_row_tiles_groups(orc, G, n):
    inp = W.random_inputs(4, G, n, 4096, 16, seed=n + G)
    banner(f"gemv_mfma row tiles G={G} n={n}")
    y = run_qmm(inp, path="gemv_mfma")
    check_qmm(orc, inp, y, path="gemv_mfma")


# Exact 4-bit codes in bands of the operand rows, at 2, 3 and 4 tiles per block: with K = 4096 a
# block of 4 x rows (34 KB of LDS) fits 4 times on a compute unit and one of 8 rows (67 KB) twice,
# so on 256 compute units these n take 2, 3, 4 (m = 4) and 2, 3, 4 (m = 8) tiles.
@pytest.mark.parametrize("G,m,n", [(32, 4, 16400), (32, 4, 33000), (64, 4, 49200),
                                   (64, 8, 8200), (64, 8, 16400), (128, 8, 24600)])
def test_gemv_mfma_exact_codes_row_tiles(orc, G, m, n):
    assert mfma_exact_codes(4, G, m)
    inp = W.random_inputs(4, G, n, 4096, m, seed=n + G + m)
    banner(f"gemv_mfma exact codes G={G} m={m} n={n}")
    y = run_qmm(inp, path="gemv_mfma")
    check_qmm(orc, inp, y, path="gemv_mfma")


# At m = 5..8 (x rows rounded to 8) two blocks fit a compute unit; for 8192 < n <= 12288 three
# tiles per block put at most 48 rows on a unit where two would put 64 on some.
@pytest.mark.parametrize("bits,n", [(3, 8300), (6, 11008)])
def test_gemv_mfma_balanced_tiles(orc, bits, n):
    inp = W.random_inputs(bits, 32, n, 4096, 8, seed=n + bits)
    banner(f"gemv_mfma balanced tiles bits={bits} n={n} m=8")
    y = run_qmm(inp, path="gemv_mfma")
    check_qmm(orc, inp, y, path="gemv_mfma")


# K past 4096: each wave takes S slices of 512 codes in turn (S = 2, 4 or 8, blocks of up to 16
# waves where two register sets fit 128 registers, else 8). 4608 codes (9 slices) leave the last
# wave one slice (its second set loads unused data, its second multiply is skipped); 14336 takes
# 14 waves of 2 (or 7 of 4); 16896 (33 slices) 9 waves of 4 (or 5 of 8), the last with one; 32768
# 16 waves of 4 (or 8 of 8). Ragged n, every width and group size, m from 1 to 16.
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("m,n,k", [(1, 40, 4608), (4, 150, 14336), (8, 77, 16896), (16, 40, 32768),
                                   (3, 150, 8192), (12, 33, 14336)])
def test_gemv_mfma_long_k(orc, bits, G, m, n, k):
    inp = W.random_inputs(bits, G, n, k, m, seed=bits * 7 + G + m + n + k)
    banner(f"gemv_mfma long k bits={bits} G={G} m={m} n={n} k={k}")
    y = run_qmm(inp, path="gemv_mfma")
    check_qmm(orc, inp, y, path="gemv_mfma")


# The automatic path at K past 4096 takes the matrix-core decode kernel from 2 rows on, and its
# results are those of the forced path.
@pytest.mark.parametrize("m", [1, 2, 5, 16])
def test_long_k_dispatch(orc, m):
    inp = W.random_inputs(4, 64, 96, 5120, m, seed=m + 5)
    banner(f"long k dispatch m={m}")
    y = run_qmm(inp)
    check_qmm(orc, inp, y)
    assert kernel_of(inp, "auto") == ("gemv_mfma" if m >= 2 else "gemv")
    want = run_qmm(inp, path=kernel_of(inp, "auto"))
    assert torch.equal(y.view(torch.int16), want.view(torch.int16))


def test_gemv_mfma_rejects_other_shapes(orc):
    inp = W.random_inputs(4, 32, 8, 768, 4, seed=1)   # k not a multiple of 512
    p, s, b = dev_weights(inp)
    with pytest.raises(qaff().QaffError, match="matrix-core decode"):
        qaff().qmm(dev_x(inp.x, "bf16"), p, s, b, 32, 4, path="gemv_mfma")
    inp = W.random_inputs(4, 32, 8, 33280, 4, seed=1)  # k above 32768
    p, s, b = dev_weights(inp)
    with pytest.raises(qaff().QaffError, match="matrix-core decode"):
        qaff().qmm(dev_x(inp.x, "bf16"), p, s, b, 32, 4, path="gemv_mfma")
    inp = W.random_inputs(4, 32, 8, 512, 17, seed=1)  # m above 16
    p, s, b = dev_weights(inp)
    with pytest.raises(qaff().QaffError, match="matrix-core decode"):
        qaff().qmm(dev_x(inp.x, "bf16"), p, s, b, 32, 4, path="gemv_mfma")


# ---- edge cases ----------------------------------------------------------------------------------

def test_k_zero_writes_zeros(orc):
    p = torch.zeros((8, 0), dtype=torch.int32, device="cuda")
    s = torch.zeros((8, 0), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((3, 0), dtype=torch.bfloat16, device="cuda")
    banner("k=0")
    y = qaff().qmm(x, p, s, s, 32, 4)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (3, 8) and (y == 0).all()


def test_empty_m_and_n(orc):
    inp = W.random_inputs(4, 32, 8, 64, 0)
    p, s, b = dev_weights(inp)
    banner("m=0")
    y = qaff().qmm(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"), p, s, b, 32, 4)
    assert tuple(y.shape) == (0, 8)
    e = qaff().dequant_rows(p, s, b, torch.zeros((0,), dtype=torch.int32, device="cuda"), 32, 4)
    assert tuple(e.shape) == (0, 64)


def test_one_dimensional_x_is_a_row(orc):
    inp = W.random_inputs(4, 64, 40, 256, 1, seed=3)
    p, s, b = dev_weights(inp)
    x = dev_x(inp.x, "bf16")
    banner("1-D x")
    y1 = qaff().qmm(x[0], p, s, b, 64, 4)
    y2 = qaff().qmm(x, p, s, b, 64, 4)
    torch.cuda.synchronize()
    assert tuple(y1.shape) == (40,)
    assert torch.equal(y1.view(torch.int16), y2[0].view(torch.int16))


def test_repeat_runs_are_bitwise_identical(orc):
    for path, m in (("gemv", 4), ("gemm", 64)):
        inp = W.random_inputs(4, 128, 300, 2048, m, seed=5)
        banner(f"determinism {path}")
        a = run_qmm(inp, path=path)
        b = run_qmm(inp, path=path)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---- the full-size workloads -------------------------------------------------------------------

def _full_qmm(orc, name, m, rows=None):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, m=m)
    banner(f"full {name} m={m}")
    y = run_qmm(inp)
    assert tuple(y.shape) == (m, wl.n)
    return check_qmm(orc, inp, y, rows=rows)


@pytest.mark.parametrize("m", [1, 4])
def test_full_decode_gemv(orc, m):
    _full_qmm(orc, "decode_4bit_g64_4096x4096", m)


@pytest.mark.parametrize("m", [1, 8])
def test_full_int8_gemv(orc, m):
    _full_qmm(orc, "int8_g64_14336x4096", m)


@pytest.mark.parametrize("name", ["odd_3bit_g32_11008x4096", "odd_6bit_g32_11008x4096"])
@pytest.mark.parametrize("m", [1, 16])
def test_full_odd_widths(orc, name, m):
    _full_qmm(orc, name, m)


def test_full_prefill_gemm_every_row(orc):
    # all 2048 x rows against the oracle (every tile, sub-tile and accumulator slot of the launch
    # the benchmark times)
    _full_qmm(orc, "prefill_4bit_g128_4096x14336", 2048)


def test_full_prefill_k_tail_gemm_every_row(orc):
    # K = 11008 (ten whole chunks and a tail of twelve steps) at the batch the benchmark times
    _full_qmm(orc, "prefill_4bit_g128_4096x11008", 2048)


@pytest.mark.parametrize("m", [4, 16])
def test_full_down_projection_long_k(orc, m):
    # [4096, 14336] 4-bit g64: the long-K matrix-core decode kernel, every row against the oracle
    _full_qmm(orc, "ffn_down_4bit_g64_4096x14336", m)


def test_full_decode_dequant_bit_exact(orc):
    wl = W.WORKLOADS["decode_4bit_g64_4096x4096"]
    inp = W.make_inputs(wl)
    p, s, b = dev_weights(inp)
    banner("full dequant 4096x4096")
    for out, tdt, view in (("f32", torch.float32, np.uint32), ("bf16", torch.bfloat16, np.uint16)):
        got = host_bits(qaff().dequantize(p, s, b, wl.group_size, wl.bits, tdt))
        ref = orc.dequantize(inp.packed, inp.scales, inp.biases, wl.group_size, wl.bits, out=out)
        np.testing.assert_array_equal(got.view(view), ref.view(view))


def test_full_dequant_rows_bit_exact(orc):
    wl = W.WORKLOADS["rows_4bit_g64_32768x4096"]
    inp = W.make_inputs(wl)
    p, s, b = dev_weights(inp)
    idx = torch.from_numpy(inp.indices.view(np.int32)).cuda()
    banner("full dequant_rows 32768x4096 / 4096")
    for out, tdt, view in (("f32", torch.float32, np.uint32), ("bf16", torch.bfloat16, np.uint16)):
        got = host_bits(qaff().dequant_rows(p, s, b, idx, wl.group_size, wl.bits, tdt))
        ref = orc.dequant_rows(inp.packed, inp.scales, inp.biases, inp.indices, wl.group_size,
                               wl.bits, out=out)
        np.testing.assert_array_equal(got.view(view), ref.view(view))


def test_dequant_rows_duplicates_and_out_of_range(orc):
    inp = W.random_inputs(3, 32, 50, 256, 0, seed=23)
    p, s, b = dev_weights(inp)
    idx_np = np.array([49, 0, 7, 7, 50, 2**32 - 1, 13], np.uint32)
    idx = torch.from_numpy(idx_np.view(np.int32)).cuda()
    banner("dequant_rows oob")
    for out, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        got = host_bits(qaff().dequant_rows(p, s, b, idx, 32, 3, tdt))
        ref = orc.dequant_rows(inp.packed, inp.scales, inp.biases, idx_np, 32, 3, out=out)
        view = np.uint32 if out == "f32" else np.uint16
        np.testing.assert_array_equal(got.view(view), ref.view(view))
