"""The C ABI on the CPU: the library loads, exports every symbol include/qaff.h declares, and
rejects bad arguments on the host (no GPU is touched: every case here fails validation or is a
no-op that returns before any HIP call)."""
import ctypes
import os
import re

import pytest

from quantized_matmul_mlx_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, INVALID, UNSUPPORTED = _lib.QAFF_OK, _lib.QAFF_ERR_INVALID_ARGUMENT, _lib.QAFF_ERR_UNSUPPORTED
F32, BF16 = _lib.QAFF_F32, _lib.QAFF_BF16

# fake, never dereferenced device addresses (validation fails or the call is a no-op first)
A16 = ctypes.c_void_p(0x10000)
A4 = ctypes.c_void_p(0x10004)
A2 = ctypes.c_void_p(0x10002)
A1 = ctypes.c_void_p(0x10001)
NULL = None


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from quantized_matmul_mlx_amd import build
        build.build()
    return _lib.load()


def header_functions():
    text = open(os.path.join(ROOT, "include", "qaff.h")).read()
    return sorted(set(re.findall(r"\b(qaff_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), f"{name} is declared in qaff.h but not exported"


def test_bench_aids_export_every_declared_symbol(lib):
    # the benchmark's measurement aids: include/qaff_bench.h against libqaff_bench.so
    text = open(os.path.join(ROOT, "include", "qaff_bench.h")).read()
    declared = sorted(set(re.findall(r"\b(qaff_bench_[a-z_0-9]+)\s*\(", text)))
    assert declared == ["qaff_bench_read", "qaff_bench_read_store", "qaff_bench_stamp", "qaff_bench_wall_clock_khz"]
    aux = ctypes.CDLL(os.path.join(ROOT, "quantized_matmul_mlx_amd", "libqaff_bench.so"))
    for name in declared:
        assert hasattr(aux, name), f"{name} is declared in qaff_bench.h but not exported"
    # argument checks on the host (fake addresses, never dereferenced)
    aux.qaff_bench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    aux.qaff_bench_read.restype = ctypes.c_int
    assert aux.qaff_bench_read(A16, 100, 4, 0, 0, A16, NULL) != 0      # not a multiple of 16 bytes
    assert aux.qaff_bench_read(A4, 64, 4, 0, 0, A16, NULL) != 0        # misaligned source
    assert aux.qaff_bench_read(A16, 64, 3, 0, 0, A16, NULL) != 0       # unsupported shape
    assert aux.qaff_bench_read(NULL, 64, 4, 0, 0, A16, NULL) != 0
    aux.qaff_bench_read_store.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]
    aux.qaff_bench_read_store.restype = ctypes.c_int
    assert aux.qaff_bench_read_store(A16, 64, 4, 0, A16, 0, NULL) != 0   # no output elements
    assert aux.qaff_bench_read_store(A16, 64, 4, 0, A1, 8, NULL) != 0    # misaligned output
    assert aux.qaff_bench_read_store(A16, 64, 5, 0, A16, 8, NULL) != 0   # unsupported shape


def test_product_library_does_not_link_the_bench_aids(lib):
    import subprocess
    out = subprocess.run(["nm", "-D", _lib.LIB_PATH], capture_output=True, text=True).stdout
    assert "qaff_bench_" not in out


def test_version_and_status_strings(lib):
    assert lib.qaff_abi_version() == _lib.ABI_VERSION
    assert lib.qaff_status_string(OK) == b"QAFF_OK"
    assert lib.qaff_status_string(INVALID) == b"QAFF_ERR_INVALID_ARGUMENT"
    assert lib.qaff_status_string(UNSUPPORTED) == b"QAFF_ERR_UNSUPPORTED"
    assert lib.qaff_status_string(_lib.QAFF_ERR_DEVICE) == b"QAFF_ERR_DEVICE"
    assert lib.qaff_gemv_max_m() >= 1
    assert 1 <= lib.qaff_gemv_mfma_min_m() <= lib.qaff_gemv_max_m()


def dq(lib, rows=4, cols=64, G=32, bits=4, packed=A16, scales=A16, biases=A16, out=A16, dt=F32):
    return lib.qaff_dequantize(packed, scales, biases, rows, cols, G, bits, out, dt, NULL)


def qmm(lib, m=1, n=4, k=64, G=32, bits=4, x=A16, xdt=BF16, packed=A16, scales=A16, biases=A16,
        y=A16, path=0):
    return lib.qaff_qmm_ex(x, xdt, m, packed, scales, biases, n, k, G, bits, y, NULL, path)


def rows(lib, table_rows=8, cols=64, G=32, bits=4, idx=A16, n_idx=2, out=A16, dt=F32,
         packed=A16, scales=A16, biases=A16):
    return lib.qaff_dequant_rows(packed, scales, biases, table_rows, cols, G, bits, idx, n_idx, out,
                                 dt, NULL)


@pytest.mark.parametrize("bits", [0, 7, 9, 16, -4])
def test_unsupported_bit_widths(lib, bits):
    assert dq(lib, bits=bits) == UNSUPPORTED
    assert b"bits" in lib.qaff_last_error()
    assert qmm(lib, bits=bits) == UNSUPPORTED
    assert rows(lib, bits=bits) == UNSUPPORTED


@pytest.mark.parametrize("G", [0, 8, 16, 48, 256, -32])
def test_bad_group_sizes(lib, G):
    assert dq(lib, G=G, cols=256) == INVALID
    assert b"group size" in lib.qaff_last_error()
    assert qmm(lib, G=G, k=256) == INVALID
    assert rows(lib, G=G, cols=256) == INVALID


def test_cols_not_multiple_of_group(lib):
    assert dq(lib, cols=96, G=64) == INVALID
    assert qmm(lib, k=96, G=64) == INVALID
    assert rows(lib, cols=160, G=128) == INVALID


def test_negative_sizes(lib):
    assert dq(lib, rows=-1) == INVALID
    assert dq(lib, cols=-32) == INVALID
    assert qmm(lib, m=-1) == INVALID
    assert qmm(lib, n=-1) == INVALID
    assert qmm(lib, k=-64) == INVALID
    assert rows(lib, table_rows=-1) == INVALID
    assert rows(lib, n_idx=-1) == INVALID


def test_rows_of_2_pow_32_bits_or_more(lib):
    # the kernels address within a row's code stream in 32 bits: cols * bits must stay below 2^32
    for bits in (1, 3, 4, 8):
        top = (2**32 - 1) // bits // 128 * 128          # the longest row that fits, in whole groups
        over = top + 128
        assert dq(lib, cols=over, G=128, bits=bits) == UNSUPPORTED
        assert b"2^32 bits" in lib.qaff_last_error()
        assert qmm(lib, k=over, G=128, bits=bits) == UNSUPPORTED
        assert rows(lib, cols=over, G=128, bits=bits) == UNSUPPORTED
        # at the limit the weight itself passes; this call then stops at its null output
        assert dq(lib, cols=top, G=128, bits=bits, out=NULL) == INVALID
        assert b"null output" in lib.qaff_last_error()
    assert dq(lib, cols=2**40, G=128) == UNSUPPORTED      # no overflow in the check itself


def test_null_pointers(lib):
    assert dq(lib, packed=NULL) == INVALID
    assert dq(lib, scales=NULL) == INVALID
    assert dq(lib, biases=NULL) == INVALID
    assert dq(lib, out=NULL) == INVALID
    assert qmm(lib, x=NULL) == INVALID
    assert qmm(lib, y=NULL) == INVALID
    assert qmm(lib, packed=NULL) == INVALID
    assert rows(lib, idx=NULL) == INVALID
    assert rows(lib, out=NULL) == INVALID


def test_misaligned_pointers(lib):
    assert dq(lib, packed=A2) == INVALID and b"4-byte" in lib.qaff_last_error()
    assert dq(lib, scales=A1) == INVALID
    assert dq(lib, out=A2) == INVALID and b"element size" in lib.qaff_last_error()   # float32 out at 2 bytes
    assert dq(lib, out=A1, dt=BF16) == INVALID
    assert qmm(lib, y=A1) == INVALID
    assert qmm(lib, x=A1) == INVALID
    assert qmm(lib, xdt=F32, x=A2) == INVALID                 # a float32 x at 2 bytes
    # an element-aligned x that is not 16-byte aligned takes the element-by-element kernel, which
    # the MFMA paths do not have
    assert qmm(lib, x=A2, k=512, path=3) == UNSUPPORTED and b"16-byte" in lib.qaff_last_error()
    assert qmm(lib, x=A2, m=20, path=2) == UNSUPPORTED
    assert rows(lib, idx=A2) == INVALID


def test_dtype_and_path_checks(lib):
    assert dq(lib, dt=7) == INVALID
    assert qmm(lib, xdt=5) == INVALID
    assert qmm(lib, path=9) == INVALID
    assert qmm(lib, xdt=F32, path=2) == UNSUPPORTED      # the MFMA GEMM takes bf16 x only
    assert b"bf16" in lib.qaff_last_error()
    assert qmm(lib, xdt=F32, path=3) == UNSUPPORTED      # so does the matrix-core decode kernel
    # the matrix-core decode kernel: k a multiple of 512 up to 32768, m <= 16, 4-byte scale words
    assert qmm(lib, k=64, path=3) == UNSUPPORTED
    assert b"matrix-core decode" in lib.qaff_last_error()
    assert qmm(lib, k=32768 + 512, path=3) == UNSUPPORTED
    assert qmm(lib, m=17, k=512, path=3) == UNSUPPORTED
    assert qmm(lib, k=512, scales=A2, path=3) == UNSUPPORTED
    assert rows(lib, dt=-1) == INVALID


def test_empty_outputs_are_no_ops(lib):
    # nothing to write: OK, even with null buffers, and no HIP call is made
    assert dq(lib, rows=0, packed=NULL, scales=NULL, biases=NULL, out=NULL) == OK
    assert dq(lib, cols=0, packed=NULL, scales=NULL, biases=NULL, out=NULL) == OK
    assert qmm(lib, m=0, x=NULL, y=NULL) == OK
    assert qmm(lib, n=0, x=NULL, y=NULL, packed=NULL, scales=NULL, biases=NULL) == OK
    assert rows(lib, n_idx=0, idx=NULL, out=NULL) == OK
    assert lib.qaff_last_error() == b""


def test_error_text_is_per_call(lib):
    assert dq(lib, bits=7) == UNSUPPORTED
    assert lib.qaff_last_error() != b""
    assert qmm(lib, m=0) == OK
    assert lib.qaff_last_error() == b""


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()


def gate_up(lib, m=1, n=4, k=64, G=32, bits=4, x=A16, gy=A16, uy=A16, gp=A16, up=A16):
    return lib.qaff_gemv_gate_up(x, m, gp, A16, A16, up, A16, A16, n, k, G, bits, gy, uy, NULL)


def silu(lib, m=1, n=4, k=64, G=32, bits=4, gate=A16, upv=A16, resid=NULL, y=A16):
    return lib.qaff_gemv_silu_gate(gate, upv, m, A16, A16, A16, n, k, G, bits, resid, y, NULL)


def test_fused_decode_checks(lib):
    assert gate_up(lib, m=17) == UNSUPPORTED                 # decode products: m <= 16
    assert b"m <= 16" in lib.qaff_last_error()
    assert silu(lib, m=17) == UNSUPPORTED
    assert gate_up(lib, bits=7) == UNSUPPORTED
    assert silu(lib, G=48) == INVALID
    assert gate_up(lib, up=NULL) == INVALID                  # the second weight is checked too
    assert gate_up(lib, uy=NULL) == INVALID
    assert gate_up(lib, x=A1) == INVALID
    assert gate_up(lib, gy=A1) == INVALID
    assert silu(lib, gate=A1) == INVALID
    assert silu(lib, y=A1) == INVALID
    assert silu(lib, y=NULL) == INVALID
    assert silu(lib, resid=A1) == INVALID                    # a residual must be 2-byte aligned
    assert gate_up(lib, m=-1) == INVALID
    # nothing to write
    assert gate_up(lib, m=0, x=NULL, gy=NULL, uy=NULL) == OK
    assert silu(lib, n=0, gate=NULL, upv=NULL, y=NULL) == OK


def gather(lib, xb=2, m=1, wb=3, n=4, k=512, G=64, bits=4, lhs=NULL, rhs=A16, batch=2, sorted_=0, x=A16,
           y=A16, dtype=BF16, path=0, packed=A16, scales=A16):
    return lib.qaff_gather_qmm_ex(x, dtype, xb, m, packed, scales, A16, wb, n, k, G, bits, lhs, rhs, batch,
                                  sorted_, y, NULL, path)


def test_gather_qmm_checks(lib):
    assert gather(lib, xb=-1) == INVALID
    assert gather(lib, batch=-1) == INVALID
    assert gather(lib, bits=7) == UNSUPPORTED
    assert gather(lib, G=48) == INVALID
    assert gather(lib, packed=NULL) == INVALID                # the stacked weight is checked
    assert gather(lib, lhs=NULL, batch=3) == INVALID          # no lhs: batch <= x batches
    assert b"lhs" in lib.qaff_last_error()
    assert gather(lib, rhs=NULL, batch=4) == INVALID          # no rhs: batch <= weight batches
    assert gather(lib, rhs=A2) == INVALID                     # indices are 4-byte aligned
    assert gather(lib, lhs=A2) == INVALID
    assert gather(lib, path=2) == UNSUPPORTED                 # the grouped GEMM needs sorted rows
    assert gather(lib, path=9) == INVALID
    assert gather(lib, path=3, dtype=F32) == UNSUPPORTED      # the matrix-core kernel takes bf16
    assert gather(lib, path=3, k=320, G=64) == UNSUPPORTED    # ... and k a multiple of 512
    assert gather(lib, path=3, scales=A2) == UNSUPPORTED      # ... and 4-byte aligned scales
    assert gather(lib, y=NULL) == INVALID
    assert gather(lib, y=A1) == INVALID
    assert gather(lib, x=A1) == INVALID
    assert gather(lib, x=A2, path=3) == UNSUPPORTED            # the matrix-core kernel: 16-byte x
    assert gather(lib, xb=1 << 32) == UNSUPPORTED
    # nothing to write
    assert gather(lib, batch=0, x=NULL, y=NULL) == OK
    assert gather(lib, m=0, x=NULL, y=NULL) == OK
    assert gather(lib, n=0, x=NULL, y=NULL) == OK


def quant(lib, rows=2, cols=64, G=32, bits=4, w=A16, packed=A16, scales=A16, biases=A16, dtype=BF16):
    return lib.qaff_quantize(w, dtype, rows, cols, G, bits, packed, scales, biases, NULL)


def test_quantize_checks(lib):
    assert quant(lib, bits=7) == UNSUPPORTED
    assert quant(lib, G=48) == INVALID
    assert quant(lib, cols=48) == INVALID                     # not a multiple of the group size
    assert quant(lib, rows=-1) == INVALID
    assert quant(lib, packed=NULL) == INVALID
    assert quant(lib, scales=A1) == INVALID
    assert quant(lib, w=NULL) == INVALID
    assert quant(lib, w=A1) == INVALID                        # w aligned to its element size
    assert quant(lib, w=A2, dtype=F32) == INVALID
    assert quant(lib, dtype=7) == INVALID
    assert quant(lib, rows=0, w=NULL, packed=NULL, scales=NULL, biases=NULL) == OK


def qnt(lib, m=1, k=64, n=64, G=32, bits=4, x=A16, y=A16, ws=A16, wsb=1 << 20, dtype=BF16):
    return lib.qaff_qmm_nt(x, dtype, m, A16, A16, A16, k, n, G, bits, ws, wsb, y, NULL)


def test_qmm_nt_checks(lib):
    assert lib.qaff_qmm_nt_workspace_size(1, 4096, 4096, 4) > 0
    assert lib.qaff_qmm_nt_workspace_size(0, 4096, 4096, 4) == 0
    assert qnt(lib, bits=7) == UNSUPPORTED
    assert qnt(lib, n=48) == INVALID                         # groups run along n
    assert qnt(lib, m=-1) == INVALID
    assert qnt(lib, y=NULL) == INVALID
    assert qnt(lib, x=A1) == INVALID
    assert qnt(lib, y=A2, dtype=F32) == INVALID
    assert qnt(lib, ws=NULL) == INVALID                      # the workspace is required ...
    assert b"workspace" in lib.qaff_last_error()
    assert qnt(lib, wsb=4) == INVALID                        # ... and must be large enough
    assert qnt(lib, ws=A4) == INVALID                        # ... and 16-byte aligned
    assert qnt(lib, m=0, x=NULL, y=NULL, ws=NULL) == OK


def test_qmm_nt_typed_checks(lib):
    F16 = _lib.QAFF_F16
    q = lambda xt=F16, sb=F16, m=1, x=A16, y=A16, scales=A16, ws=A16, wsb=1 << 20, bits=4: lib.qaff_qmm_nt_typed(
        x, xt, m, A16, scales, A16, sb, 64, 64, 32, bits, ws, wsb, y, NULL)
    assert q(xt=5) == INVALID and q(sb=3) == INVALID
    assert q(bits=7) == UNSUPPORTED
    assert q(sb=F32, scales=A2) == INVALID                   # float32 scales are 4-byte aligned
    assert q(sb=BF16, y=A2) == INVALID                       # float16 x with bf16 scales: float32 y
    assert q(xt=F32, x=A2) == INVALID
    assert q(y=NULL) == INVALID
    assert q(ws=NULL) == INVALID and b"workspace" in lib.qaff_last_error()
    assert q(wsb=4) == INVALID
    assert q(m=0, x=NULL, y=NULL, ws=NULL) == OK
    # the plain entry point keeps its types: float16 x is not one of them
    assert qnt(lib, dtype=F16) == INVALID


def qws(lib, m=128, n=4096, k=14336, G=128, bits=4, x=A16, y=A16, ws=A16, wsb=1 << 26):
    return lib.qaff_qmm_ws(x, BF16, m, A16, A16, A16, n, k, G, bits, ws, wsb, y, NULL)


def test_qmm_ws_checks(lib):
    size = lambda m, n=4096, k=14336: lib.qaff_qmm_workspace_size(m, n, k, 128, 4)
    assert size(16, k=4096) == 0 and size(16) == 0           # the matrix-core decode kernel's range
    far = 33792                                              # past it (above 32768), from 8 rows:
    assert size(7, k=far) == 0 and size(8, k=far) > 0 and size(16, k=far) > 0  # the split GEMM
    assert size(17) > 0 and size(128) > 0 and size(1024) > 0  # few GEMM tiles: K splits
    assert size(17, k=4096) == 0 and size(32, k=4096) == 0      # ... except small weights at up to 32
    assert size(33, k=4096) > 0 and size(17, n=8192, k=4096) > 0  # rows: 16-row decode slices there
    assert size(2048) == 0                                   # a tile per compute unit already
    assert size(128, k=14336 + 64) > 0                       # K with a tail splits its whole chunks too
    assert size(128, k=1024) == 0                            # a single chunk of K
    assert size(128, k=1024 + 64) == 0                       # ... also with a tail
    assert size(128, k=960) == 0                             # no whole chunk
    assert qws(lib, ws=NULL) == INVALID                      # a workspace is needed here ...
    assert b"workspace" in lib.qaff_last_error()
    assert qws(lib, wsb=4) == INVALID                        # ... large enough
    assert qws(lib, ws=A4) == INVALID                        # ... and 16-byte aligned
    assert qws(lib, m=0, x=NULL, y=NULL, ws=NULL) == OK
    assert qws(lib, bits=7) == UNSUPPORTED


def test_typed_checks(lib):
    F16 = _lib.QAFF_F16
    assert lib.qaff_promote_dtype(F16, F16) == F16
    assert lib.qaff_promote_dtype(BF16, BF16) == BF16
    assert lib.qaff_promote_dtype(BF16, F16) == F32
    assert lib.qaff_promote_dtype(F32, F16) == F32
    dq_t = lambda sb=F16, out=F32, scales=A16, o=A16, bits=4: lib.qaff_dequantize_typed(
        A16, scales, A16, sb, 2, 64, 32, bits, o, out, NULL)
    assert dq_t(sb=7) == INVALID
    assert dq_t(out=9) == INVALID
    assert dq_t(bits=7) == UNSUPPORTED
    assert dq_t(sb=F32, scales=A2) == INVALID               # float32 scales are 4-byte aligned
    assert dq_t(o=NULL) == INVALID
    q_t = lambda xt=F16, sb=F16, x=A16, y=A16, scales=A16: lib.qaff_qmm_typed(
        x, xt, 1, A16, scales, A16, sb, 4, 64, 32, 4, y, NULL)
    assert q_t(xt=5) == INVALID
    assert q_t(sb=F32, scales=A2) == INVALID
    assert q_t(y=NULL) == INVALID
    assert q_t(x=A1) == INVALID
    assert q_t(xt=F32, x=A2) == INVALID
    assert dq_t(o=A2) == INVALID                              # a float32 output at 2 bytes
    # the old entry points keep their types: float16 is not one of them
    assert lib.qaff_qmm(A16, F16, 1, A16, A16, A16, 4, 64, 32, 4, A16, NULL) == INVALID


def test_qmm_nt_static_rejects_on_the_host(lib):
    # past the static scratch (8 MiB of partial sums): UNSUPPORTED, before any device call
    assert lib.qaff_qmm_nt_static_max_bytes() == 8 << 20
    m, k, n = 2, 128 * 300, 4096
    assert lib.qaff_qmm_nt_workspace_size(m, k, n, 4) > lib.qaff_qmm_nt_static_max_bytes()
    assert lib.qaff_qmm_nt_static(A16, BF16, m, A16, A16, A16, k, n, 64, 4, A16, NULL) == UNSUPPORTED
    assert b"static scratch" in lib.qaff_last_error()
    # the workspace entry point's own checks apply
    assert lib.qaff_qmm_nt_static(A16, BF16, 1, A16, A16, A16, 64, 48, 32, 4, A16, NULL) == INVALID  # n % G
    assert lib.qaff_qmm_nt_static(A16, BF16, 1, A16, A16, A16, 64, 64, 32, 7, A16, NULL) == UNSUPPORTED
    assert lib.qaff_qmm_nt_static(A16, BF16, 0, A16, A16, A16, 64, 64, 32, 4, A16, NULL) == OK      # m = 0
