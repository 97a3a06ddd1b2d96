"""Gathered quantized products (mixture-of-experts batches) on the GPU against the CPU oracle,
through the C ABI (via the binding).

Output batch i is x[lhs[i]] . dequantize(W[rhs[i]])^T. The bars are those of the plain product:
per-row max relative error against the float64 oracle of at most 2e-3 (float32 y) and 1.6e-2
(bf16 y), and the tighter bound from the kernel's own arithmetic (1e-4 / 4e-3) against the oracle
composed the way the kernel computes: float32 weights for the VALU GEMV and for the matrix-core
kernel where it takes 4-bit codes exactly, weights rounded to bf16 for the matrix-core kernel
otherwise and for the grouped GEMM. An index past its operand gives a NaN batch on both sides.
"""
import numpy as np
import pytest
import torch

import oracle as orc_mod
from gpu_util import banner, dev_bf16, dev_u32, dev_x, grouped_rows_per_tile, host_f64, mfma_exact_codes
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


def experts(bits, G, E, n, k, seed):
    """E random experts [n, k], stacked, with the decode workload's distributions."""
    inp = W.random_inputs(bits, G, E * n, k, 0, seed=seed)
    return inp.packed.reshape(E, n, -1), inp.scales.reshape(E, n, -1), inp.biases.reshape(E, n, -1)


def draw_x(shape, x_dtype, seed):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32)
    return W.bf16_bits_from_f32(x) if x_dtype == "bf16" else x


def bf16_weight_gather_ref(orc, x, x_dtype, packed, scales, biases, G, bits, lhs, rhs):
    """Batch i: x[lhs[i]] . bf16(W[rhs[i]])^T in float64 (NaN past either operand)."""
    out = []
    for li, ri in zip(lhs, rhs):
        if li >= x.shape[0] or ri >= packed.shape[0]:
            out.append(np.full((x.shape[1], packed.shape[1]), np.nan))
            continue
        w = orc.bf16_to_f32(orc.dequantize(packed[ri], scales[ri], biases[ri], G, bits, out="bf16"))
        xs = orc.bf16_to_f32(x[li]) if x_dtype == "bf16" else x[li]
        out.append(xs.astype(np.float64) @ w.astype(np.float64).T)
    return np.stack(out)


def run(x, x_dtype, packed, scales, biases, G, bits, lhs=None, rhs=None, sorted_=False, path="auto"):
    xd = dev_x(x, x_dtype)
    y = qaff().gather_qmm(xd, dev_u32(packed), dev_bf16(scales), dev_bf16(biases), G, bits,
                          lhs_indices=None if lhs is None else dev_u32(lhs),
                          rhs_indices=None if rhs is None else dev_u32(rhs), sorted_indices=sorted_, path=path)
    torch.cuda.synchronize()
    return host_f64(y)


def check(orc, got, x, x_dtype, packed, scales, biases, G, bits, lhs, rhs, kernel, grouped=False):
    """got [batch, m, n] against the oracle; lhs/rhs are the explicit (expanded) index arrays;
    grouped: the matrix-core kernel walked sorted rows by expert (rows per tile from the mean count)."""
    ref = orc.gather_qmm(x, x_dtype, packed, scales, biases, G, bits, lhs=lhs, rhs=rhs)
    assert got.shape == ref.shape
    nan = np.isnan(ref).all(axis=(1, 2))
    assert np.isnan(got[nan]).all(), "out-of-range batches must be NaN"
    assert np.isfinite(got[~nan]).all()
    g2 = got[~nan].reshape(-1, got.shape[-1])
    r2 = ref[~nan].reshape(-1, ref.shape[-1])
    if g2.size == 0:
        return
    err = orc.max_row_rel_err(g2, r2)
    assert err <= TOL[x_dtype], f"max row rel err {err:.3e} > {TOL[x_dtype]}"
    rows = grouped_rows_per_tile(got.shape[0], packed.shape[0]) if grouped else got.shape[1]
    if kernel == "gemv_mfma" and not mfma_exact_codes(bits, G, rows):
        tref = bf16_weight_gather_ref(orc, x, x_dtype, packed, scales, biases, G, bits, lhs, rhs)
        tref = tref[~nan].reshape(-1, ref.shape[-1])
    else:
        tref = r2
    terr = orc.max_row_rel_err(g2, tref)
    assert terr <= TIGHT[x_dtype], f"{kernel}: max row rel err {terr:.3e} against its own arithmetic"


# ---- batched: any lhs / rhs ------------------------------------------------------------------------

@pytest.mark.parametrize("bits,G,x_dtype,m", [(4, 64, "bf16", 1), (3, 32, "f32", 3), (8, 128, "bf16", 2), (1, 32, "f32", 2),
                                              (6, 32, "bf16", 5), (2, 64, "f32", 1), (5, 128, "bf16", 17)])
def test_gather_valu_batched(orc, bits, G, x_dtype, m):
    E, n, k = 4, 150, 640   # 20 blocks of 32 per row: not a whole pass of the GEMV
    packed, scales, biases = experts(bits, G, E, n, k, seed=100 + bits)
    x = draw_x((3, m, k), x_dtype, seed=200 + bits)
    lhs = np.array([2, 0, 0, 1, 2, 1, 0], np.uint32)
    rhs = np.array([3, 3, 0, 2, 1, 0, 1], np.uint32)
    banner(f"gather valu batched bits={bits} G={G} {x_dtype} m={m}")
    got = run(x, x_dtype, packed, scales, biases, G, bits, lhs, rhs, path="gemv")
    check(orc, got, x, x_dtype, packed, scales, biases, G, bits, lhs, rhs, "gemv")


@pytest.mark.parametrize("bits,G,m,k", [(4, 64, 1, 512), (4, 128, 5, 2048), (3, 32, 16, 1024), (8, 64, 20, 512), (1, 64, 3, 1024),
                                        (6, 32, 4, 4096), (2, 128, 9, 1536), (5, 64, 33, 512)])
def test_gather_mfma_batched(orc, bits, G, m, k):
    E, n = 5, 150
    packed, scales, biases = experts(bits, G, E, n, k, seed=300 + bits)
    x = draw_x((4, m, k), "bf16", seed=400 + m)
    lhs = np.array([3, 0, 0, 2, 1, 3], np.uint32)
    rhs = np.array([4, 4, 1, 0, 2, 3], np.uint32)
    banner(f"gather mfma batched bits={bits} G={G} m={m} k={k}")
    got = run(x, "bf16", packed, scales, biases, G, bits, lhs, rhs, path="gemv_mfma")
    check(orc, got, x, "bf16", packed, scales, biases, G, bits, lhs, rhs, "gemv_mfma")


# Two row tiles per block: 128 output batches of 10 tiles each (n = 160) are more tiles than one
# round of the compute units holds (at most 4 blocks of this size per unit), so the launcher takes
# two tiles per block. Every width, M = 4 and 16.
@pytest.mark.parametrize("bits,G", [(1, 32), (2, 64), (3, 32), (4, 128), (5, 64), (6, 32), (8, 64)])
@pytest.mark.parametrize("m", [4, 16])
def test_gather_mfma_batched_two_tiles(orc, bits, G, m):
    E, n, k, batch = 16, 160, 512, 128
    packed, scales, biases = experts(bits, G, E, n, k, seed=800 + bits)
    x = draw_x((8, m, k), "bf16", seed=810 + m)
    rng = np.random.default_rng(820 + bits)
    lhs = rng.integers(0, 8, batch).astype(np.uint32)
    rhs = rng.integers(0, E, batch).astype(np.uint32)
    banner(f"gather mfma batched two tiles bits={bits} G={G} m={m}")
    got = run(x, "bf16", packed, scales, biases, G, bits, lhs, rhs, path="gemv_mfma")
    check(orc, got, x, "bf16", packed, scales, biases, G, bits, lhs, rhs, "gemv_mfma")


# ---- grouped: sorted rhs, one row per batch, each expert's weights read once -----------------------

def sorted_rows(counts):
    return np.repeat(np.arange(len(counts), dtype=np.uint32), counts)


@pytest.mark.parametrize("bits,G,k,counts", [
    (4, 64, 2048, [0, 3, 20, 1, 0, 16]),         # empty experts, one of several tiles, one of a tile
    (4, 32, 512, [1, 1, 1, 1, 1, 1, 1, 1]),      # one row each
    (8, 128, 1024, [40, 0, 0, 2]),               # several tiles of 16
    (3, 32, 4096, [5, 9, 0, 0, 0, 7]),
    (6, 64, 1536, [0, 0, 0, 0, 0, 0, 0, 12]),    # only the last expert
    (2, 64, 512, [33]),
    (1, 128, 2048, [2, 0, 7]),
])
def test_gather_mfma_grouped(orc, bits, G, k, counts):
    E, n = len(counts), 100
    packed, scales, biases = experts(bits, G, E, n, k, seed=500 + bits)
    rhs = sorted_rows(counts)
    x = draw_x((rhs.size, 1, k), "bf16", seed=600 + k)
    banner(f"gather mfma grouped bits={bits} G={G} k={k} counts={counts}")
    got = run(x, "bf16", packed, scales, biases, G, bits, None, rhs, sorted_=True, path="gemv_mfma")
    check(orc, got, x, "bf16", packed, scales, biases, G, bits, np.arange(rhs.size, dtype=np.uint32), rhs,
          "gemv_mfma", grouped=True)
    got_b = run(x, "bf16", packed, scales, biases, G, bits, None, rhs, sorted_=False, path="gemv_mfma")
    if mfma_exact_codes(bits, G, grouped_rows_per_tile(rhs.size, E)) == mfma_exact_codes(bits, G, 1):
        # the grouped walk and the batched kernel compute each row the same way
        np.testing.assert_array_equal(got, got_b)
    else:
        # the batched kernel (one row per tile) takes the codes exactly, the grouped walk does not
        check(orc, got_b, x, "bf16", packed, scales, biases, G, bits, np.arange(rhs.size, dtype=np.uint32), rhs,
              "gemv_mfma")


def test_gather_grouped_rows_past_every_expert_are_nan(orc):
    E, n, k, G, bits = 3, 40, 512, 64, 4
    packed, scales, biases = experts(bits, G, E, n, k, seed=700)
    rhs = np.array([0, 0, 2, 2, 2, 3, 7, 7], np.uint32)  # the last three are past the experts
    x = draw_x((rhs.size, 1, k), "bf16", seed=701)
    banner("gather mfma grouped, rows past every expert")
    got = run(x, "bf16", packed, scales, biases, G, bits, None, rhs, sorted_=True, path="gemv_mfma")
    check(orc, got, x, "bf16", packed, scales, biases, G, bits, np.arange(rhs.size, dtype=np.uint32), rhs,
          "gemv_mfma", grouped=True)
    assert np.isnan(got[5:]).all() and np.isfinite(got[:5]).all()


# ---- grouped: the GEMM over each expert's rows (hundreds of rows per expert) ------------------------

def grouped_refs(orc, x, packed, scales, biases, G, bits, rhs):
    """Row r against expert rhs[r], each expert's rows at once: the oracle's product (gather_qmm's
    definition: the plain product per batch) and x . bf16(W)^T in float64 (the kernel's own
    arithmetic: weights rounded to bf16); NaN for rows past the experts."""
    E, n = packed.shape[0], packed.shape[1]
    xr = x.reshape(rhs.size, -1)
    ref = np.full((rhs.size, 1, n), np.nan)
    tight = np.full((rhs.size, 1, n), np.nan)
    xf = orc.bf16_to_f32(xr).astype(np.float64)
    for e in np.unique(rhs):
        if e >= E:
            continue
        rows = np.flatnonzero(rhs == e)
        ref[rows, 0, :] = orc.qmm(np.ascontiguousarray(xr[rows]), "bf16", packed[e], scales[e], biases[e], G, bits)
        w = orc.bf16_to_f32(orc.dequantize(packed[e], scales[e], biases[e], G, bits, out="bf16")).astype(np.float64)
        tight[rows, 0, :] = xf[rows] @ w.T
    return ref, tight


def check_grouped(orc, got, x, packed, scales, biases, G, bits, rhs):
    ref, tight = grouped_refs(orc, x, packed, scales, biases, G, bits, rhs)
    nan = rhs >= packed.shape[0]
    assert np.isnan(got[nan]).all(), "rows past every expert must be NaN"
    assert np.isfinite(got[~nan]).all()
    g2, r2, t2 = (a[~nan].reshape(-1, a.shape[-1]) for a in (got, ref, tight))
    if g2.size:
        assert orc.max_row_rel_err(g2, r2) <= TOL["bf16"]
        assert orc.max_row_rel_err(g2, t2) <= TIGHT["bf16"]


# Experts of several 128-row tiles (odd and even counts, so both blocks of an expert's tile column
# take tiles), of one row, empty ones, a ragged tile column (n = 300 of 256-column tiles), and rows
# past every expert; every width.
@pytest.mark.parametrize("bits,G,counts,past", [
    (4, 64, [0, 200, 129, 1, 300, 50], 3),
    (3, 32, [130, 0, 5], 0),
    (8, 128, [257], 2),
    (2, 64, [64, 64, 64, 64], 0),
    (5, 32, [10, 300], 1),
    (6, 128, [0, 0, 140], 0),
    (1, 32, [100, 30], 5),
])
def test_gather_grouped_gemm(orc, bits, G, counts, past):
    E, n, k = len(counts), 300, 1024
    packed, scales, biases = experts(bits, G, E, n, k, seed=900 + bits)
    rhs = np.concatenate([sorted_rows(counts), np.full(past, E + 2, np.uint32)]).astype(np.uint32)
    x = draw_x((rhs.size, 1, k), "bf16", seed=910 + bits)
    banner(f"gather grouped gemm bits={bits} G={G} counts={counts} past={past}")
    got = run(x, "bf16", packed, scales, biases, G, bits, None, rhs, sorted_=True, path="gemm")
    check_grouped(orc, got, x, packed, scales, biases, G, bits, rhs)


def test_gather_grouped_gemm_dispatch(orc):
    # experts averaging 32 rows or more: AUTO takes the grouped GEMM (the same bits as forced);
    # fewer: the matrix-core decode kernel's grouped walk
    E, n, k, G, bits = 4, 256, 2048, 64, 4
    packed, scales, biases = experts(bits, G, E, n, k, seed=930)
    for counts, kernel in (([40, 30, 50, 8], "gemm"), ([10, 30, 20, 8], "gemv_mfma")):
        rhs = sorted_rows(counts)
        x = draw_x((rhs.size, 1, k), "bf16", seed=931)
        banner(f"gather grouped dispatch counts={counts}")
        auto = run(x, "bf16", packed, scales, biases, G, bits, None, rhs, sorted_=True)
        forced = run(x, "bf16", packed, scales, biases, G, bits, None, rhs, sorted_=True, path=kernel)
        np.testing.assert_array_equal(auto, forced)
        check_grouped(orc, auto, x, packed, scales, biases, G, bits, rhs)
    # the GEMM needs the sorted promise with one row per batch
    with pytest.raises(qaff().QaffError, match="grouped GEMM"):
        run(x, "bf16", packed, scales, biases, G, bits, None, rhs, sorted_=False, path="gemm")


@pytest.mark.parametrize("path,x_dtype", [("gemv", "bf16"), ("gemv", "f32"), ("gemv_mfma", "bf16")])
def test_gather_batched_out_of_range_is_nan(orc, path, x_dtype):
    E, n, k, G, bits = 2, 70, 512, 32, 4
    packed, scales, biases = experts(bits, G, E, n, k, seed=710)
    x = draw_x((2, 3, k), x_dtype, seed=711)
    lhs = np.array([0, 2, 1, 1], np.uint32)
    rhs = np.array([1, 0, 5, 0], np.uint32)
    banner(f"gather out of range {path} {x_dtype}")
    got = run(x, x_dtype, packed, scales, biases, G, bits, lhs, rhs, path=path)
    check(orc, got, x, x_dtype, packed, scales, biases, G, bits, lhs, rhs, path)
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all()


def test_gather_auto_picks_a_tested_kernel(orc):
    E, n, k, G, bits = 8, 96, 1024, 64, 4
    packed, scales, biases = experts(bits, G, E, n, k, seed=720)
    rhs = sorted_rows([2, 1, 0, 3, 1, 1, 0, 2])
    x = draw_x((rhs.size, 1, k), "bf16", seed=721)
    banner("gather auto vs forced")
    # sorted, one row per batch, at least one row per expert on average: the grouped walk
    auto = run(x, "bf16", packed, scales, biases, G, bits, None, rhs, sorted_=True)
    forced = run(x, "bf16", packed, scales, biases, G, bits, None, rhs, sorted_=True, path="gemv_mfma")
    np.testing.assert_array_equal(auto, forced)
    # unsorted promise, m = 1: the VALU GEMV
    auto = run(x, "bf16", packed, scales, biases, G, bits, None, rhs)
    forced = run(x, "bf16", packed, scales, biases, G, bits, None, rhs, path="gemv")
    np.testing.assert_array_equal(auto, forced)


def test_gather_binding_broadcasts_and_defaults(orc):
    E, n, k, G, bits = 3, 50, 512, 32, 4
    packed, scales, biases = experts(bits, G, E, n, k, seed=730)
    x = draw_x((2, 2, k), "bf16", seed=731)
    lhs = np.array([[1], [0]], np.uint32)
    rhs = np.array([2, 0, 1], np.uint32)
    banner("gather broadcast")
    q = qaff()
    y = q.gather_qmm(dev_x(x, "bf16"), dev_u32(packed), dev_bf16(scales), dev_bf16(biases), G, bits,
                     lhs_indices=dev_u32(lhs), rhs_indices=dev_u32(rhs))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (2, 3, 2, n)
    ref = orc.gather_qmm(x, "bf16", packed, scales, biases, G, bits, lhs=lhs, rhs=rhs)
    assert orc.max_row_rel_err(host_f64(y).reshape(-1, n), ref.reshape(-1, n)) <= TOL["bf16"]
    # both defaults: batch i of x with expert i (three of each)
    x3 = draw_x((3, 1, k), "bf16", seed=732)
    y3 = q.gather_qmm(dev_x(x3, "bf16"), dev_u32(packed), dev_bf16(scales), dev_bf16(biases), G, bits)
    torch.cuda.synchronize()
    ref3 = orc.gather_qmm(x3, "bf16", packed, scales, biases, G, bits)
    assert orc.max_row_rel_err(host_f64(y3).reshape(-1, n), ref3.reshape(-1, n)) <= TOL["bf16"]
    # int64 indices are read as their uint32 value
    y4 = q.gather_qmm(dev_x(x, "bf16"), dev_u32(packed), dev_bf16(scales), dev_bf16(biases), G, bits,
                      lhs_indices=torch.from_numpy(lhs.astype(np.int64)).cuda(),
                      rhs_indices=torch.from_numpy(rhs.astype(np.int64)).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_f64(y4), host_f64(y))


def test_gather_empty(orc):
    packed, scales, biases = experts(4, 64, 2, 8, 512, seed=740)
    x = draw_x((1, 1, 512), "bf16", seed=741)   # one x batch: broadcasts against no batches
    banner("gather empty")
    y = qaff().gather_qmm(dev_x(x, "bf16"), dev_u32(packed), dev_bf16(scales), dev_bf16(biases), 64, 4,
                          rhs_indices=torch.zeros(0, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 1, 8)


# ---- the mixture-of-experts workload at full size -----------------------------------------------

@pytest.mark.parametrize("tokens", W.WORKLOADS["moe_4bit_g64_e128_768x2048"].ms)
def test_gather_moe_workload(orc, tokens):
    wl = W.WORKLOADS["moe_4bit_g64_e128_768x2048"]
    mi = W.moe_inputs(wl, tokens)
    banner(f"gather moe workload tokens={tokens} rows={mi.expert.size}")
    got = run(mi.x_rows, "bf16", mi.packed, mi.scales, mi.biases, wl.group_size, wl.bits, None, mi.expert,
              sorted_=True)
    grouped = mi.expert.size >= wl.experts
    check(orc, got, mi.x_rows, "bf16", mi.packed, mi.scales, mi.biases, wl.group_size, wl.bits,
          np.arange(mi.expert.size, dtype=np.uint32), mi.expert, "gemv_mfma" if grouped else "gemv", grouped=grouped)
    # the same rows through lhs indices (token of each row) into the unpermuted activations
    got2 = run(mi.x[:, None, :], "bf16", mi.packed, mi.scales, mi.biases, wl.group_size, wl.bits, mi.token,
               mi.expert)
    check(orc, got2, mi.x[:, None, :], "bf16", mi.packed, mi.scales, mi.biases, wl.group_size, wl.bits,
          mi.token, mi.expert, "gemv")


def test_qmm_with_a_batched_weight_broadcasts(orc):
    # nuvec_core quantized_matmul: batch dimensions of x and w broadcast when w has them
    E, n, k, G, bits = 4, 40, 512, 64, 4
    packed, scales, biases = experts(bits, G, E, n, k, seed=750)
    x = draw_x((2, 1, 3, k), "bf16", seed=751)
    banner("qmm batched weight")
    q = qaff()
    pw, sw, bw = dev_u32(packed), dev_bf16(scales), dev_bf16(biases)
    y = q.qmm(dev_x(x, "bf16"), pw, sw, bw, G, bits)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (2, E, 3, n)
    ref = orc.gather_qmm(x, "bf16", packed, scales, biases, G, bits)   # default indices, broadcast
    assert ref.shape == (2, E, 3, n)
    assert orc.max_row_rel_err(host_f64(y).reshape(-1, n), ref.reshape(-1, n)) <= TOL["bf16"]
    # a 2-D x takes the weight's batch; a 1-D x is a row vector and drops that row
    x2 = draw_x((3, k), "bf16", seed=752)
    y2 = q.qmm(dev_x(x2, "bf16"), pw, sw, bw, G, bits)
    x1 = x2[0]
    y1 = q.qmm(dev_x(x1, "bf16"), pw, sw, bw, G, bits)
    torch.cuda.synchronize()
    assert tuple(y2.shape) == (E, 3, n) and tuple(y1.shape) == (E, n)
    ref2 = orc.gather_qmm(x2[None], "bf16", packed, scales, biases, G, bits)
    assert orc.max_row_rel_err(host_f64(y2).reshape(-1, n), ref2.reshape(-1, n)) <= TOL["bf16"]
    ref1 = orc.gather_qmm(x1[None, None], "bf16", packed, scales, biases, G, bits)[:, 0, :]
    assert orc.max_row_rel_err(host_f64(y1), ref1) <= TOL["bf16"]


def test_gather_moe_prefill_workload(orc):
    # 2048 tokens, top-8 of 128 experts [768, 2048] (about 128 rows per expert): the grouped GEMM
    wl = W.WORKLOADS["moe_prefill_4bit_g64_e128_768x2048"]
    mi = W.moe_inputs(wl, wl.ms[0])
    lib = qaff()._lib.load()
    banner(f"gather moe prefill workload rows={mi.expert.size}")
    got = run(mi.x_rows, "bf16", mi.packed, mi.scales, mi.biases, wl.group_size, wl.bits, None, mi.expert,
              sorted_=True)
    check_grouped(orc, got, mi.x_rows, mi.packed, mi.scales, mi.biases, wl.group_size, wl.bits, mi.expert)
