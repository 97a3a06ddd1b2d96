"""float16 and float32 scales and biases, float16 x (x, scales and biases promote to one float
type), on the GPU against the CPU oracle through the C ABI (via the binding).

* dequantize: bit-exact (w = s * c, then + b, in float32 on both sides; bf16 and float16 outputs
  rounded to nearest even on both sides).
* qmm: per-row max relative error against the float64 oracle: 1e-4 for a float32 y (the kernel
  sums float32 products, like the VALU GEMV), 1e-3 for a float16 y (one rounding to 11
  significant bits, 2^-11 = 4.9e-4 of the row's largest value, plus float32 summation).
"""
import numpy as np
import pytest
import torch

import oracle as orc_mod
from gpu_util import banner, dev_u32
from quantized_matmul_mlx_amd import workloads as W

pytestmark = pytest.mark.gpu

TIGHT = {torch.float32: 1e-4, torch.float16: 1e-3, torch.bfloat16: 4e-3}
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


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


def scales_of(inp, sb, seed):
    """Scales and biases of the workload's ranges as host arrays of type sb (bit patterns for the
    16-bit types) and as device tensors of that type."""
    rng = np.random.default_rng(seed)
    s32 = rng.uniform(1e-3, 2e-2, inp.scales.shape).astype(np.float32)
    b32 = rng.uniform(-0.15, 0.0, inp.scales.shape).astype(np.float32)
    if sb == "f32":
        hs, hb = s32, b32
    elif sb == "f16":
        hs, hb = s32.astype(np.float16).view(np.uint16), b32.astype(np.float16).view(np.uint16)
    else:
        hs, hb = W.bf16_bits_from_f32(s32), W.bf16_bits_from_f32(b32)
    return hs, hb, to_dev(hs, sb), to_dev(hb, sb)


def to_dev(a, dtype):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).cuda()
    return t.view(TORCH[dtype])


def host(t):
    t = t.detach().cpu()
    return t.numpy() if t.dtype == torch.float32 else t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("sb", ["f16", "f32", "bf16"])
@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("bits,G", [(4, 64), (3, 32), (8, 128), (1, 32), (6, 64)])
def test_dequantize_typed_bit_exact(orc, sb, out, bits, G):
    inp = W.random_inputs(bits, G, 37, 3 * G, 0, seed=bits + G)
    hs, hb, ds, db = scales_of(inp, sb, seed=bits * G)
    banner(f"dequantize typed sb={sb} out={out} bits={bits} G={G}")
    got = qaff().dequantize(dev_u32(inp.packed), ds, db, G, bits, out_dtype=TORCH[out])
    torch.cuda.synchronize()
    ref = orc.dequantize_typed(inp.packed, hs, hb, sb, G, bits, out=out)
    np.testing.assert_array_equal(host(got).view(ref.dtype), ref)


@pytest.mark.parametrize("xt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("sb", ["f16", "f32"])
@pytest.mark.parametrize("bits,G", [(4, 64), (5, 32), (8, 128), (2, 64)])
@pytest.mark.parametrize("m", [1, 5])
def test_qmm_typed(orc, xt, sb, bits, G, m):
    n, k = 150, 20 * G // 2 * 2
    inp = W.random_inputs(bits, G, n, k, 0, seed=bits * 7 + G + m)
    hs, hb, ds, db = scales_of(inp, sb, seed=bits + G + m)
    x32 = np.random.default_rng(m + bits).standard_normal((m, k)).astype(np.float32)
    hx = x32 if xt == "f32" else (x32.astype(np.float16).view(np.uint16) if xt == "f16" else W.bf16_bits_from_f32(x32))
    banner(f"qmm typed x={xt} sb={sb} bits={bits} G={G} m={m}")
    y = qaff().qmm(to_dev(hx, xt), dev_u32(inp.packed), ds, db, G, bits)
    torch.cuda.synchronize()
    want = torch.float16 if (xt == "f16" and sb == "f16") else torch.float32
    assert y.dtype == want and tuple(y.shape) == (m, n)
    ref = orc.qmm_typed(hx, xt, inp.packed, hs, hb, sb, G, bits)
    got = y.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = orc.max_row_rel_err(got, ref)
    assert err <= TIGHT[want], f"max row rel err {err:.3e} > {TIGHT[want]}"


# float16 x with float16 scales and biases: the bf16 GEMV's layout in float16 (codes as 1024 + c,
# v_dot2_f32_f16). Every width; m = 1, 2, 3 and 8 (x-row tiles of 1, 2, 4 and 8 rows); K of one
# pass, and long rows (more than 4096 codes: the wider pass, with scales and biases through LDS when
# a row has an even number of groups, 4352 / 128 = 34 and 8192 / 32 = 256, and without at
# 4224 / 128 = 33).
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G,m,k", [(64, 1, 2048), (32, 2, 1024), (128, 3, 4352), (64, 8, 1024), (32, 1, 8192),
                                   (128, 1, 4224)])
def test_qmm_f16_gemv(orc, bits, G, m, k):
    n = 77
    inp = W.random_inputs(bits, G, n, k, 0, seed=bits * 11 + G + m + k)
    hs, hb, ds, db = scales_of(inp, "f16", seed=bits + G + m + k)
    x = np.random.default_rng(m + bits + k).standard_normal((m, k)).astype(np.float16)
    banner(f"qmm float16 gemv bits={bits} G={G} m={m} k={k}")
    y = qaff().qmm(to_dev(x.view(np.uint16), "f16"), dev_u32(inp.packed), ds, db, G, bits)
    torch.cuda.synchronize()
    assert y.dtype == torch.float16 and tuple(y.shape) == (m, n)
    ref = orc.qmm_typed(x.view(np.uint16), "f16", inp.packed, hs, hb, "f16", G, bits)
    got = y.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = orc.max_row_rel_err(got, ref)
    assert err <= TIGHT[torch.float16], f"max row rel err {err:.3e} > {TIGHT[torch.float16]}"


def test_f16_x_with_bf16_scales_promotes_to_f32(orc):
    inp = W.random_inputs(4, 64, 100, 512, 0, seed=5)
    x = np.random.default_rng(6).standard_normal((3, 512)).astype(np.float16)
    banner("qmm f16 x, bf16 scales")
    y = qaff().qmm(to_dev(x.view(np.uint16), "f16"), dev_u32(inp.packed), to_dev(inp.scales, "bf16"),
                   to_dev(inp.biases, "bf16"), 64, 4)
    torch.cuda.synchronize()
    assert y.dtype == torch.float32
    ref = orc.qmm_typed(x.view(np.uint16), "f16", inp.packed, inp.scales, inp.biases, "bf16", 64, 4)
    assert orc.max_row_rel_err(y.cpu().numpy().astype(np.float64), ref) <= TIGHT[torch.float32]


def test_bf16_only_operations_reject_other_scales(orc):
    inp = W.random_inputs(4, 64, 16, 128, 0, seed=7)
    hs, hb, ds, db = scales_of(inp, "f16", seed=8)
    q = qaff()
    banner("bf16-only operations reject float16 scales")
    with pytest.raises(TypeError):
        q.dequant_rows(dev_u32(inp.packed), ds, db, torch.zeros(2, dtype=torch.int32, device="cuda"), 64, 4)
    with pytest.raises(TypeError):
        q.gemv_silu_gate(torch.zeros((1, 128), dtype=torch.bfloat16, device="cuda"),
                         torch.zeros((1, 128), dtype=torch.bfloat16, device="cuda"), dev_u32(inp.packed), ds, db, 64, 4)
    with pytest.raises(TypeError):   # scales and biases of different types
        q.qmm(torch.zeros((1, 128), dtype=torch.bfloat16, device="cuda"), dev_u32(inp.packed), ds,
              to_dev(inp.biases, "bf16"), 64, 4)


# ---- the product without the transpose (W stored [k, n]), typed ----------------------------------

def typed_x(x32, xt):
    return x32 if xt == "f32" else (x32.astype(np.float16).view(np.uint16) if xt == "f16" else W.bf16_bits_from_f32(x32))


@pytest.mark.parametrize("xt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("sb", ["f16", "f32", "bf16"])
@pytest.mark.parametrize("bits,G", [(4, 64), (3, 32), (8, 128), (1, 32), (6, 64)])
def test_qmm_nt_typed(orc, xt, sb, bits, G):
    # k = 100 rows (not a multiple of the 16 row phases), n = 5 G (a ragged column tile), m = 3 (a
    # slice of 2 x rows and one of 1)
    k, n, m = 100, 5 * G, 3
    inp = W.random_inputs(bits, G, k, n, 0, seed=bits * 11 + G)      # a [k, n] weight: groups along n
    hs, hb, ds, db = scales_of(inp, sb, seed=bits + 3 * G)
    hx = typed_x(np.random.default_rng(bits + G).standard_normal((m, k)).astype(np.float32), xt)
    banner(f"qmm_nt typed x={xt} sb={sb} bits={bits} G={G}")
    y = qaff().qmm(to_dev(hx, xt), dev_u32(inp.packed), ds, db, G, bits, transpose=False)
    torch.cuda.synchronize()
    want = promoted(xt, sb)
    assert y.dtype == want and tuple(y.shape) == (m, n)
    ref = orc.qmm_nt_typed(hx, xt, inp.packed, hs, hb, sb, G, bits)
    got = y.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = orc.max_row_rel_err(got, ref)
    assert err <= TIGHT[want], f"max row rel err {err:.3e} > {TIGHT[want]}"


@pytest.mark.parametrize("sb", ["f16", "f32"])
def test_qmm_nt_typed_full_size(orc, sb):
    # a [4096, 4096] 4-bit g64 weight, x [2, 4096] float16: 32 K chunks per column tile
    k = n = 4096
    inp = W.random_inputs(4, 64, k, n, 0, seed=123)
    hs, hb, ds, db = scales_of(inp, sb, seed=124)
    hx = typed_x(np.random.default_rng(125).standard_normal((2, k)).astype(np.float32), "f16")
    banner(f"qmm_nt typed full size sb={sb}")
    y = qaff().qmm_nt(to_dev(hx, "f16"), dev_u32(inp.packed), ds, db, 64, 4)
    torch.cuda.synchronize()
    want = promoted("f16", sb)
    ref = orc.qmm_nt_typed(hx, "f16", inp.packed, hs, hb, sb, 64, 4)
    err = orc.max_row_rel_err(y.float().cpu().numpy().astype(np.float64), ref)
    assert err <= TIGHT[want], f"max row rel err {err:.3e} > {TIGHT[want]}"


@pytest.mark.parametrize("n", [320, 2048])
def test_qmm_nt_typed_float16_x_is_its_float32_copy(orc, n):
    # every operand is widened to float32 exactly as it is loaded, so a float16 x (the run-time
    # typed kernel) and the float32 x of the same values (the float32 kernel) give the same y, bit
    # for bit, with bf16 scales; a 1-D x is one row. n = 320 splits K, n = 2048 takes one thread
    # block per column block.
    k = 700
    inp = W.random_inputs(5, 32, k, n, 0, seed=130)
    x16 = np.random.default_rng(131).standard_normal((3, k)).astype(np.float16)
    p, s, b = dev_u32(inp.packed), to_dev(inp.scales, "bf16"), to_dev(inp.biases, "bf16")
    banner(f"qmm_nt typed float16 x against its float32 copy n={n}")
    y16 = qaff().qmm_nt(to_dev(x16.view(np.uint16), "f16"), p, s, b, 32, 5)
    y32 = qaff().qmm_nt(to_dev(x16.astype(np.float32), "f32"), p, s, b, 32, 5)
    y1 = qaff().qmm_nt(to_dev(x16[1].view(np.uint16), "f16"), p, s, b, 32, 5)
    torch.cuda.synchronize()
    assert y16.dtype == torch.float32 and tuple(y1.shape) == (n,)
    assert torch.equal(y16, y32) and torch.equal(y1, y32[1])
    ref = orc.qmm_nt_typed(x16.view(np.uint16), "f16", inp.packed, inp.scales, inp.biases, "bf16", 32, 5)
    assert orc.max_row_rel_err(host(y16).astype(np.float64), ref) <= TIGHT[torch.float32]


@pytest.mark.parametrize("bits,G", [(4, 64), (3, 32), (8, 128)])
def test_qmm_nt_float16_form_is_the_float32_one_rounded(orc, bits, G):
    # float16 x, scales and biases (the fixed float16 form, y float16) against float32 copies of the
    # same values (the run-time typed form, y float32): the same float32 sums, so y16 is y32
    # rounded to nearest even, bit for bit
    k, n, m = 700, 5 * G, 3
    inp = W.random_inputs(bits, G, k, n, 0, seed=150 + bits)
    hs, hb, ds, db = scales_of(inp, "f16", seed=151 + bits)
    x16 = np.random.default_rng(152 + bits).standard_normal((m, k)).astype(np.float16)
    p = dev_u32(inp.packed)
    banner(f"qmm_nt float16 form against float32 copies bits={bits} G={G}")
    y16 = qaff().qmm_nt(to_dev(x16.view(np.uint16), "f16"), p, ds, db, G, bits)
    y32 = qaff().qmm_nt(to_dev(x16.astype(np.float32), "f32"), p, ds.float(), db.float(), G, bits)
    torch.cuda.synchronize()
    assert y16.dtype == torch.float16 and y32.dtype == torch.float32
    assert torch.equal(y16, y32.half())


def test_qmm_nt_typed_rejects_the_static_scratch(orc):
    inp = W.random_inputs(4, 64, 64, 128, 0, seed=140)
    hs, hb, ds, db = scales_of(inp, "f16", seed=141)
    x = torch.zeros((1, 64), dtype=torch.float16, device="cuda")
    banner("qmm_nt typed rejects the static scratch")
    with pytest.raises(TypeError):
        qaff().qmm_nt(x, dev_u32(inp.packed), ds, db, 64, 4, out=torch.empty((1, 128), dtype=torch.float16,
                                                                          device="cuda"), static_scratch=True)


# ---- gathered products (nuvec_core gather_qmm: x, scales and biases promote to one type) ----------

def promoted(xt, sb):
    return TORCH[xt] if xt == sb else torch.float32


def typed_experts(bits, G, E, n, k, sb, seed):
    inp = W.random_inputs(bits, G, E * n, k, 0, seed=seed)
    hs, hb, ds, db = scales_of(inp, sb, seed=seed + 1)
    return (inp.packed.reshape(E, n, -1), hs.reshape(E, n, -1), hb.reshape(E, n, -1),
            ds.reshape(E, n, -1), db.reshape(E, n, -1))


def check_gather(orc, y, hx, xt, packed, hs, hb, sb, G, bits, lhs, rhs):
    want = promoted(xt, sb)
    assert y.dtype == want
    ref = orc.gather_qmm_typed(hx, xt, packed, hs, hb, sb, G, bits, lhs=lhs, rhs=rhs)
    got = y.float().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape
    nan = np.isnan(ref).all(axis=(1, 2))
    assert np.isnan(got[nan]).all() and np.isfinite(got[~nan]).all()
    err = orc.max_row_rel_err(got[~nan].reshape(-1, got.shape[-1]), ref[~nan].reshape(-1, ref.shape[-1]))
    assert err <= TIGHT[want], f"max row rel err {err:.3e} > {TIGHT[want]}"


@pytest.mark.parametrize("xt,sb", [("f16", "f16"), ("f16", "f32"), ("f32", "f16"), ("bf16", "f32"), ("f16", "bf16"),
                                   ("f32", "f32")])
@pytest.mark.parametrize("bits,G,m", [(4, 64, 1), (3, 32, 3), (8, 128, 2), (5, 64, 6)])
def test_gather_qmm_typed(orc, xt, sb, bits, G, m):
    # 5 experts of [150, 640]; batches past x (lhs 7) and past the experts (rhs 9) are NaN
    E, n, k = 5, 150, 640
    packed, hs, hb, ds, db = typed_experts(bits, G, E, n, k, sb, seed=60 + bits + G)
    x32 = np.random.default_rng(m + bits).standard_normal((4, m, k)).astype(np.float32)
    hx = x32 if xt == "f32" else (x32.astype(np.float16).view(np.uint16) if xt == "f16" else W.bf16_bits_from_f32(x32))
    lhs = np.array([3, 0, 0, 2, 1, 7, 3], np.uint32)
    rhs = np.array([4, 4, 1, 0, 9, 2, 3], np.uint32)
    banner(f"gather_qmm typed x={xt} sb={sb} bits={bits} G={G} m={m}")
    y = qaff().gather_qmm(to_dev(hx, xt), dev_u32(packed), ds, db, G, bits, lhs_indices=dev_u32(lhs),
                          rhs_indices=dev_u32(rhs))
    torch.cuda.synchronize()
    check_gather(orc, y, hx, xt, packed, hs, hb, sb, G, bits, lhs, rhs)


def test_gather_qmm_typed_unaligned_x_and_sorted_rows(orc):
    # x at a 2-byte offset takes the element-by-element kernel; sorted rows (one per batch, the
    # mixture-of-experts form) with float16 scales, the typed kernel
    from gpu_util import at_offset
    E, n, k, G, bits = 4, 96, 512, 64, 4
    packed, hs, hb, ds, db = typed_experts(bits, G, E, n, k, "f16", seed=70)
    rhs = np.repeat(np.arange(E, dtype=np.uint32), [3, 0, 5, 2])
    x = np.random.default_rng(71).standard_normal((rhs.size, 1, k)).astype(np.float16)
    hx = x.view(np.uint16)
    banner("gather_qmm typed, float16 x at an offset, sorted rows")
    xd = at_offset(to_dev(hx, "f16"))
    assert xd.data_ptr() % 16 != 0
    y = qaff().gather_qmm(xd, dev_u32(packed), ds, db, G, bits, rhs_indices=dev_u32(rhs), sorted_indices=True)
    torch.cuda.synchronize()
    check_gather(orc, y, hx, "f16", packed, hs, hb, "f16", G, bits, np.arange(rhs.size, dtype=np.uint32), rhs)
    y2 = qaff().gather_qmm(to_dev(hx, "f16"), dev_u32(packed), ds, db, G, bits, rhs_indices=dev_u32(rhs),
                           sorted_indices=True)
    torch.cuda.synchronize()
    check_gather(orc, y2, hx, "f16", packed, hs, hb, "f16", G, bits, np.arange(rhs.size, dtype=np.uint32), rhs)
    with pytest.raises(ValueError, match="automatic path"):
        qaff().gather_qmm(to_dev(hx, "f16"), dev_u32(packed), ds, db, G, bits, rhs_indices=dev_u32(rhs),
                          path="gemv_mfma")


# The grouped walk (16 rows or more per expert on average): experts of several row tiles, empty
# ones, one row, rows past every expert, and more than 1024 rows (the counting's search).
@pytest.mark.parametrize("xt,sb,counts,past", [
    ("f16", "f16", [39, 0, 1, 26, 14], 0),
    ("f16", "f32", [23, 33, 0, 0, 22], 3),
    ("f32", "f16", [130] * 8 + [0] * 8 + [7], 5),
])
def test_gather_qmm_typed_grouped(orc, xt, sb, counts, past):
    E, n, k, G, bits = len(counts), 70, 256, 64, 4
    packed, hs, hb, ds, db = typed_experts(bits, G, E, n, k, sb, seed=80 + E)
    rhs = np.concatenate([np.repeat(np.arange(E, dtype=np.uint32), counts),
                          np.full(past, E + 2, np.uint32)]).astype(np.uint32)
    x32 = np.random.default_rng(81).standard_normal((rhs.size, 1, k)).astype(np.float32)
    hx = x32 if xt == "f32" else x32.astype(np.float16).view(np.uint16)
    banner(f"gather_qmm typed grouped x={xt} sb={sb} rows={rhs.size} past={past}")
    y = qaff().gather_qmm(to_dev(hx, xt), dev_u32(packed), ds, db, G, bits, rhs_indices=dev_u32(rhs),
                          sorted_indices=True)
    torch.cuda.synchronize()
    check_gather(orc, y, hx, xt, packed, hs, hb, sb, G, bits, np.arange(rhs.size, dtype=np.uint32), rhs)
    # the batched walk (no promise) computes every row the same way
    y_b = qaff().gather_qmm(to_dev(hx, xt), dev_u32(packed), ds, db, G, bits, rhs_indices=dev_u32(rhs))
    torch.cuda.synchronize()
    a, b = host(y), host(y_b)
    np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  b.view(np.uint32) if b.dtype == np.float32 else b)


def test_gather_qmm_typed_moe_workload(orc):
    # the 64-token mixture-of-experts layer with float16 x, scales and biases
    wl = W.WORKLOADS["moe_4bit_g64_e128_768x2048"]
    mi = W.moe_inputs(wl, 64)
    to16 = lambda a: W.f32_from_bf16_bits(a).astype(np.float16).view(np.uint16)
    hs, hb, hx = to16(mi.scales), to16(mi.biases), to16(mi.x_rows)
    banner("gather_qmm typed moe 64 tokens")
    y = qaff().gather_qmm(to_dev(hx, "f16"), dev_u32(mi.packed), to_dev(hs, "f16"), to_dev(hb, "f16"),
                          wl.group_size, wl.bits, rhs_indices=dev_u32(mi.expert), sorted_indices=True)
    torch.cuda.synchronize()
    check_gather(orc, y, hx, "f16", mi.packed, hs, hb, "f16", wl.group_size, wl.bits,
                 np.arange(mi.expert.size, dtype=np.uint32), mi.expert)


# ---- float16 on the matrix cores ------------------------------------------------------------------
#
# A float16 x with float16 scales and biases takes the float16 forms of qaff_qmm's kernels under its
# rules: the matrix-core decode kernel from 3 rows (2 past 4096 codes), with exact 4-bit codes
# 1024 + c in bands of the operand rows where they apply and otherwise the weights rounded to
# float16; the GEMM past 16 rows, W rounded to float16. Against the float64 oracle at the float16
# bound above.

def f16_case(bits, G, n, k, m, seed):
    inp = W.random_inputs(bits, G, n, k, 0, seed=seed)
    hs, hb, ds, db = scales_of(inp, "f16", seed=seed + 1)
    x = np.random.default_rng(seed + 2).standard_normal((m, k)).astype(np.float16)
    return inp, hs, hb, ds, db, x


def check_f16_qmm(orc, y, x, inp, hs, hb, G, bits):
    assert y.dtype == torch.float16 and tuple(y.shape) == (x.shape[0], inp.wl.n)
    ref = orc.qmm_typed(x.view(np.uint16), "f16", inp.packed, hs, hb, "f16", G, bits)
    got = y.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    err = orc.max_row_rel_err(got, ref)
    assert err <= TIGHT[torch.float16], f"max row rel err {err:.3e} > {TIGHT[torch.float16]}"


# The decode kernel: K of one slice (512), several (1536, 2048, 4096), past 4096 (5120: 2 rows;
# 14336: several slices per wave); x rows rounded to 4, 8 and 16; ragged n.
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("m,n,k", [(3, 150, 512), (4, 77, 4096), (8, 150, 2048), (16, 40, 1536), (2, 40, 5120),
                                   (12, 33, 14336)])
def test_qmm_f16_matrix_core_decode(orc, bits, G, m, n, k):
    inp, hs, hb, ds, db, x = f16_case(bits, G, n, k, m, seed=bits * 5 + G + m + n + k)
    banner(f"qmm float16 matrix-core decode bits={bits} G={G} m={m} n={n} k={k}")
    y = qaff().qmm(to_dev(x.view(np.uint16), "f16"), dev_u32(inp.packed), ds, db, G, bits)
    torch.cuda.synchronize()
    check_f16_qmm(orc, y, x, inp, hs, hb, G, bits)


# The GEMM: ragged tiles in m and n, K of whole 1024-code chunks and K with a tail (1056 codes: the
# general variant). (Up to 128 rows where the decode kernel takes K run as 16-row slices instead.)
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("G,m,n,k", [(64, 140, 300, 1024), (128, 300, 520, 2048), (32, 130, 260, 1056),
                                     (32, 17, 300, 1056)])
def test_qmm_f16_gemm(orc, bits, G, m, n, k):
    inp, hs, hb, ds, db, x = f16_case(bits, G, n, k, m, seed=bits * 3 + G + m + k)
    banner(f"qmm float16 gemm bits={bits} G={G} m={m} n={n} k={k}")
    y = qaff().qmm(to_dev(x.view(np.uint16), "f16"), dev_u32(inp.packed), ds, db, G, bits)
    torch.cuda.synchronize()
    check_f16_qmm(orc, y, x, inp, hs, hb, G, bits)


# 17 to 128 float16 rows: 16-row slices of the float16 decode path, each equal to the slice run as a
# call of its own, bit for bit.
@pytest.mark.parametrize("bits,G,m,n,k", [(4, 64, 17, 300, 1024), (3, 32, 40, 150, 4096), (8, 128, 64, 96, 2048),
                                          (4, 64, 33, 150, 8192), (4, 64, 120, 300, 2048)])
def test_qmm_f16_decode_slices(orc, bits, G, m, n, k):
    inp, hs, hb, ds, db, x = f16_case(bits, G, n, k, m, seed=bits * 5 + G + m + k)
    banner(f"qmm float16 decode slices bits={bits} G={G} m={m} n={n} k={k}")
    xd, p = to_dev(x.view(np.uint16), "f16"), dev_u32(inp.packed)
    y = qaff().qmm(xd, p, ds, db, G, bits)
    parts = [qaff().qmm(xd[m0:m0 + 16], p, ds, db, G, bits) for m0 in range(0, m, 16)]
    torch.cuda.synchronize()
    check_f16_qmm(orc, y, x, inp, hs, hb, G, bits)
    assert torch.equal(y.view(torch.int16), torch.cat(parts).view(torch.int16))


# Gathered float16 products on the matrix cores: batched (x rows of 4 per batch; batches past x
# and past the experts are NaN), grouped by expert (sorted rows, one per batch, at least one per
# expert on average), and the grouped GEMM (32 or more per expert), with rows past every expert.
@pytest.mark.parametrize("bits,G", [(4, 64), (3, 32), (8, 128), (4, 128)])
def test_gather_qmm_f16_batched_matrix_cores(orc, bits, G):
    E, n, k, m = 5, 150, 1024, 4
    packed, hs, hb, ds, db = typed_experts(bits, G, E, n, k, "f16", seed=90 + bits + G)
    hx = np.random.default_rng(bits + G).standard_normal((4, m, k)).astype(np.float16).view(np.uint16)
    lhs = np.array([3, 0, 0, 2, 1, 7, 3], np.uint32)
    rhs = np.array([4, 4, 1, 0, 9, 2, 3], np.uint32)
    banner(f"gather_qmm float16 batched matrix cores bits={bits} G={G}")
    y = qaff().gather_qmm(to_dev(hx, "f16"), dev_u32(packed), ds, db, G, bits, lhs_indices=dev_u32(lhs),
                          rhs_indices=dev_u32(rhs))
    torch.cuda.synchronize()
    check_gather(orc, y, hx, "f16", packed, hs, hb, "f16", G, bits, lhs, rhs)


@pytest.mark.parametrize("bits,G,counts,past", [(4, 64, [3, 0, 1, 7, 5], 2), (3, 32, [2, 9, 0, 4], 0),
                                                (4, 64, [40, 40, 40, 0, 90], 3), (8, 128, [70, 0, 33, 61], 1)])
def test_gather_qmm_f16_grouped_matrix_cores(orc, bits, G, counts, past):
    E, n, k = len(counts), 70, 1024
    packed, hs, hb, ds, db = typed_experts(bits, G, E, n, k, "f16", seed=95 + E + bits)
    rhs = np.concatenate([np.repeat(np.arange(E, dtype=np.uint32), counts),
                          np.full(past, E + 2, np.uint32)]).astype(np.uint32)
    hx = np.random.default_rng(96 + bits).standard_normal((rhs.size, 1, k)).astype(np.float16).view(np.uint16)
    banner(f"gather_qmm float16 grouped matrix cores bits={bits} G={G} rows={rhs.size} past={past}")
    y = qaff().gather_qmm(to_dev(hx, "f16"), dev_u32(packed), ds, db, G, bits, rhs_indices=dev_u32(rhs),
                          sorted_indices=True)
    torch.cuda.synchronize()
    check_gather(orc, y, hx, "f16", packed, hs, hb, "f16", G, bits, np.arange(rhs.size, dtype=np.uint32), rhs)
