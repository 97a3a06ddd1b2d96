"""CPU oracle for grouped affine dequantization and the quantized matmul (MLX layout).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library never imports it, and the two share no
code: this is a ctypes wrapper over ``oracle.c`` (plain C, built with gcc, no HIP).

Every function takes and returns host numpy arrays. bf16 values travel as ``uint16`` bit
patterns. What each function computes, and the page passage it follows, is documented in
``oracle.c``:

* ``unpack_codes`` / ``pack_codes`` -- the row's little-endian bit stream, one bit at a time
  (nuvec_core ``quantized.rs`` module documentation; rlx-moshi ``mlx_dequant.rs``, doc comment of
  ``dequantize_affine``).
* ``dequantize`` -- ``w = scale * code + bias`` per group, float32 product then float32 sum
  (rlx-moshi ``dequantize_affine``; spark_runtime ``mlx_int8.rs`` module formula), optionally
  rounded to bf16 (nearest, ties to even).
* ``dequant_rows`` -- the gathered-row lookup (maya2_mlx ``quant.py``, ``rows``).
* ``qmm`` -- ``x . dequantize(W)^T`` summed in double precision (nuvec_core ``quantized_matmul``;
  maya2_mlx ``mm``).
* ``qmm_nt`` -- ``x . dequantize(W)`` for a weight stored [k, n] (nuvec_core ``quantized_matmul``
  without the transpose).
* ``gather_qmm`` -- output batch i is ``x[lhs[i]] . dequantize(W[rhs[i]])^T`` (nuvec_core
  ``gather_qmm`` and ``gather_indices``).
* ``silu_gate`` / ``silu_gate_qmm`` -- the fused decode products' activation and product
  (spark_runtime ``gemv_silu_gate``).
* ``dequantize_typed`` / ``qmm_typed`` -- the same with float16, bfloat16 or float32 scales, biases
  and x (nuvec_core: x, scales and biases promote to one float type); ``f16_to_f32`` /
  ``f32_to_f16`` -- IEEE binary16 widening and round-to-nearest-even narrowing, by hand.
* ``quantize`` -- w -> packed codes, bf16 scales and biases: bias = group min, scale =
  (max - min) / (2^bits - 1), code = round((w - bias) / scale) clamped (nuvec_core module
  documentation and ``quantize``; rlx-moshi: bias = group min).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (always recompiles)."""
    cmd = ["gcc", *CFLAGS, "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    global _lib
    _lib = None
    return _LIB


_lib = None

_u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_int = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    lib.orc_version.restype = _int
    lib.orc_unpack_codes.argtypes = [_u32p, _i64, _i64, _int, _u8p]
    lib.orc_pack_codes.argtypes = [_u8p, _i64, _i64, _int, _u32p]
    lib.orc_bf16_to_f32.argtypes = [_u16p, _i64, _f32p]
    lib.orc_f32_to_bf16.argtypes = [_f32p, _i64, _u16p]
    lib.orc_dequantize.argtypes = [_u32p, _u16p, _u16p, _i64, _i64, _i64, _int, _f32p, _int]
    lib.orc_dequant_rows.argtypes = [_u32p, _u16p, _u16p, _i64, _i64, _i64, _int, _u32p, _i64,
                                     _f32p, _int]
    lib.orc_qmm.argtypes = [ctypes.c_void_p, _int, _i64, _u32p, _u16p, _u16p, _i64, _i64, _i64,
                            _int, _f64p, _int]
    lib.orc_gather_qmm.argtypes = [ctypes.c_void_p, _int, _i64, _i64, _u32p, _u16p, _u16p, _i64, _i64, _i64,
                                   _i64, _int, ctypes.c_void_p, ctypes.c_void_p, _i64, _f64p, _int]
    lib.orc_f16_to_f32.argtypes = [_u16p, _i64, _f32p]
    lib.orc_f32_to_f16.argtypes = [_f32p, _i64, _u16p]
    lib.orc_dequantize_typed.argtypes = [_u32p, ctypes.c_void_p, ctypes.c_void_p, _int, _i64, _i64, _i64, _int, _f32p]
    lib.orc_qmm_typed.argtypes = [ctypes.c_void_p, _int, _i64, _u32p, ctypes.c_void_p, ctypes.c_void_p, _int, _i64, _i64,
                                  _i64, _int, _f64p]
    lib.orc_qmm_nt.argtypes = [ctypes.c_void_p, _int, _i64, _u32p, _u16p, _u16p, _i64, _i64, _i64, _int, _f64p]
    lib.orc_qmm_nt_typed.argtypes = [ctypes.c_void_p, _int, _i64, _u32p, ctypes.c_void_p, ctypes.c_void_p, _int, _i64,
                                     _i64, _i64, _int, _f64p]
    lib.orc_quantize.argtypes = [ctypes.c_void_p, _int, _i64, _i64, _i64, _int, _u32p, _u16p, _u16p]
    lib.orc_quantize_typed.argtypes = [ctypes.c_void_p, _int, _i64, _i64, _i64, _int, _u32p, ctypes.c_void_p,
                                       ctypes.c_void_p, _int]
    lib.orc_gather_qmm_typed.argtypes = [ctypes.c_void_p, _int, _i64, _i64, _u32p, ctypes.c_void_p, ctypes.c_void_p,
                                         _int, _i64, _i64, _i64, _i64, _int, ctypes.c_void_p, ctypes.c_void_p, _i64,
                                         _f64p]
    lib.orc_silu_gate.argtypes = [_u16p, _u16p, _i64, _f64p]
    lib.orc_silu_gate_qmm.argtypes = [_u16p, _u16p, ctypes.c_void_p, _i64, _u32p, _u16p, _u16p, _i64,
                                      _i64, _i64, _int, _f64p, _int]
    for name in ("orc_unpack_codes", "orc_pack_codes", "orc_dequantize", "orc_dequant_rows",
                 "orc_qmm", "orc_silu_gate_qmm", "orc_gather_qmm", "orc_quantize", "orc_qmm_nt",
                 "orc_dequantize_typed", "orc_qmm_typed", "orc_quantize_typed", "orc_gather_qmm_typed",
                 "orc_qmm_nt_typed"):
        getattr(lib, name).restype = _int
    for name in ("orc_bf16_to_f32", "orc_f32_to_bf16", "orc_silu_gate", "orc_f16_to_f32", "orc_f32_to_f16"):
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid parameters (rc={rc})")


def unpack_codes(packed: np.ndarray, cols: int, bits: int) -> np.ndarray:
    packed = _c(np.atleast_2d(packed), np.uint32)
    rows = packed.shape[0]
    out = np.empty((rows, cols), np.uint8)
    _check(_load().orc_unpack_codes(packed, rows, cols, bits, out), "unpack_codes")
    return out


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = _c(np.atleast_2d(codes), np.uint8)
    rows, cols = codes.shape
    if (cols * bits) % 32:
        raise ValueError("cols * bits must be a multiple of 32")
    out = np.empty((rows, cols * bits // 32), np.uint32)
    _check(_load().orc_pack_codes(codes, rows, cols, bits, out), "pack_codes")
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    _load().orc_bf16_to_f32(h.reshape(-1), h.size, out.reshape(-1))
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().orc_f32_to_bf16(a.reshape(-1), a.size, out.reshape(-1))
    return out


def dequantize(packed, scales, biases, group_size: int, bits: int, out: str = "f32",
               cols: int | None = None, threads: int | None = None) -> np.ndarray:
    """Dense [rows, cols] float32 (``out="f32"``) or bf16 bits (``out="bf16"``)."""
    packed = _c(np.atleast_2d(packed), np.uint32)
    scales = _c(np.atleast_2d(scales), np.uint16)
    biases = _c(np.atleast_2d(biases), np.uint16)
    rows = packed.shape[0]
    cols = packed.shape[1] * 32 // bits if cols is None else cols
    res = np.empty((rows, cols), np.float32)
    _check(_load().orc_dequantize(packed, scales, biases, rows, cols, group_size, bits, res,
                                  threads or default_threads()), "dequantize")
    if out == "f32":
        return res
    if out == "bf16":
        return f32_to_bf16(res)
    raise ValueError(out)


def dequant_rows(packed, scales, biases, indices, group_size: int, bits: int, out: str = "f32",
                 threads: int | None = None) -> np.ndarray:
    packed = _c(packed, np.uint32)
    scales = _c(scales, np.uint16)
    biases = _c(biases, np.uint16)
    idx = _c(indices, np.uint32).reshape(-1)
    rows = packed.shape[0]
    cols = packed.shape[1] * 32 // bits
    res = np.empty((idx.size, cols), np.float32)
    _check(_load().orc_dequant_rows(packed, scales, biases, rows, cols, group_size, bits, idx,
                                    idx.size, res, threads or default_threads()), "dequant_rows")
    if out == "f32":
        return res
    if out == "bf16":
        return f32_to_bf16(res)
    raise ValueError(out)


def qmm(x, x_dtype: str, packed, scales, biases, group_size: int, bits: int,
        threads: int | None = None) -> np.ndarray:
    """y = x . dequantize(W)^T in float64, shape [m, n]. ``x_dtype`` is "f32" (x float32) or
    "bf16" (x uint16 bit patterns)."""
    packed = _c(packed, np.uint32)
    scales = _c(scales, np.uint16)
    biases = _c(biases, np.uint16)
    if x_dtype == "bf16":
        xa = _c(np.atleast_2d(x), np.uint16)
    elif x_dtype == "f32":
        xa = _c(np.atleast_2d(x), np.float32)
    else:
        raise ValueError(x_dtype)
    m, k = xa.shape
    n = packed.shape[0]
    if packed.shape[1] * 32 != k * bits:
        raise ValueError("x columns do not match the packed width")
    out = np.empty((m, n), np.float64)
    _check(_load().orc_qmm(xa.ctypes.data, 1 if x_dtype == "bf16" else 0, m, packed, scales, biases,
                           n, k, group_size, bits, out, threads or default_threads()), "qmm")
    return out


def qmm_nt(x, x_dtype: str, packed, scales, biases, group_size: int, bits: int) -> np.ndarray:
    """y = x . dequantize(W) in float64, shape [m, n], for W stored [k, n]: packed
    [k, n*bits/32], scales and biases [k, n/G]."""
    packed = _c(np.atleast_2d(packed), np.uint32)
    scales = _c(np.atleast_2d(scales), np.uint16)
    biases = _c(np.atleast_2d(biases), np.uint16)
    if x_dtype == "bf16":
        xa = _c(np.atleast_2d(x), np.uint16)
    elif x_dtype == "f32":
        xa = _c(np.atleast_2d(x), np.float32)
    else:
        raise ValueError(x_dtype)
    m, k = xa.shape
    if packed.shape[0] != k:
        raise ValueError("x columns do not match the weight's rows")
    n = packed.shape[1] * 32 // bits
    out = np.empty((m, n), np.float64)
    _check(_load().orc_qmm_nt(xa.ctypes.data, 1 if x_dtype == "bf16" else 0, m, packed, scales, biases, k, n,
                              group_size, bits, out), "qmm_nt")
    return out


def silu_gate(gate, up) -> np.ndarray:
    """h = silu(gate) * up in float64 (spark_runtime ``gemv_silu_gate``'s activation); gate and up
    are bf16 bit patterns of one shape."""
    gate = _c(gate, np.uint16)
    up = _c(up, np.uint16)
    if gate.shape != up.shape:
        raise ValueError("gate and up differ in shape")
    out = np.empty(gate.shape, np.float64)
    _load().orc_silu_gate(gate, up, gate.size, out)
    return out


def silu_gate_qmm(gate, up, resid, packed, scales, biases, group_size: int, bits: int,
                  threads: int | None = None) -> np.ndarray:
    """y = (silu(gate) * up) . dequantize(W)^T (+ resid) in float64, shape [m, n]
    (spark_runtime ``gemv_silu_gate`` / ``gemv_silu_gate_resid``). gate, up [m, k] and resid
    [m, n] (or None) are bf16 bit patterns."""
    packed = _c(packed, np.uint32)
    scales = _c(scales, np.uint16)
    biases = _c(biases, np.uint16)
    gate = _c(np.atleast_2d(gate), np.uint16)
    up = _c(np.atleast_2d(up), np.uint16)
    if gate.shape != up.shape:
        raise ValueError("gate and up differ in shape")
    m, k = gate.shape
    n = packed.shape[0]
    if packed.shape[1] * 32 != k * bits:
        raise ValueError("gate columns do not match the packed width")
    r = None
    if resid is not None:
        r = _c(np.atleast_2d(resid), np.uint16)
        if r.shape != (m, n):
            raise ValueError("resid must be [m, n]")
    out = np.empty((m, n), np.float64)
    _check(_load().orc_silu_gate_qmm(gate, up, r.ctypes.data if r is not None else None, m, packed, scales,
                                     biases, n, k, group_size, bits, out, threads or default_threads()),
           "silu_gate_qmm")
    return out


def gather_indices(x_batch_shape, w_batch_shape, lhs=None, rhs=None):
    """nuvec_core ``gather_indices``: the two index arrays as uint32, each defaulting to every batch
    of its operand in order (shaped like that operand's batch dimensions), broadcast together.
    Returns (lhs, rhs) flattened, and the broadcast batch shape."""
    def one(batch_shape, given):
        if given is None:
            count = int(np.prod(batch_shape, dtype=np.int64))
            return np.arange(count, dtype=np.uint32).reshape(batch_shape)
        given = np.asarray(given)
        if given.dtype.kind not in "iu":
            raise ValueError("indices must be integers")
        return given.astype(np.uint32)
    lhs_a, rhs_a = one(tuple(x_batch_shape), lhs), one(tuple(w_batch_shape), rhs)
    shape = np.broadcast_shapes(lhs_a.shape, rhs_a.shape)
    return (np.ascontiguousarray(np.broadcast_to(lhs_a, shape)).reshape(-1),
            np.ascontiguousarray(np.broadcast_to(rhs_a, shape)).reshape(-1), shape)


def gather_qmm(x, x_dtype: str, packed, scales, biases, group_size: int, bits: int, lhs=None, rhs=None,
               threads: int | None = None) -> np.ndarray:
    """nuvec_core ``gather_qmm`` with the transpose: x is [..., m, k] (float32, or bf16 bit
    patterns with ``x_dtype="bf16"``), packed [..., n, k*bits/32] and scales, biases [..., n, k/G];
    output batch i is ``x[lhs[i]] . dequantize(W[rhs[i]])^T`` in float64, shape
    broadcast(batch) + [m, n]. An index past its operand gives a NaN batch."""
    if x_dtype == "bf16":
        xa = _c(x, np.uint16)
    elif x_dtype == "f32":
        xa = _c(x, np.float32)
    else:
        raise ValueError(x_dtype)
    packed = _c(packed, np.uint32)
    scales = _c(scales, np.uint16)
    biases = _c(biases, np.uint16)
    if xa.ndim < 2 or packed.ndim < 2 or scales.shape != biases.shape:
        raise ValueError("x must be [..., m, k] and w [..., n, k*bits/32]")
    m, k = xa.shape[-2:]
    n = packed.shape[-2]
    if packed.shape[-1] * 32 != k * bits:
        raise ValueError("x columns do not match the packed width")
    li, ri, shape = gather_indices(xa.shape[:-2], packed.shape[:-2], lhs, rhs)
    xb = int(np.prod(xa.shape[:-2], dtype=np.int64))
    wb = int(np.prod(packed.shape[:-2], dtype=np.int64))
    out = np.empty((li.size, m, n), np.float64)
    _check(_load().orc_gather_qmm(xa.ctypes.data, 1 if x_dtype == "bf16" else 0, xb, m,
                                  packed.reshape(-1), scales.reshape(-1), biases.reshape(-1), wb, n, k,
                                  group_size, bits, li.ctypes.data, ri.ctypes.data, li.size, out,
                                  threads or default_threads()), "gather_qmm")
    return out.reshape(tuple(shape) + (m, n))


def quantize(w, w_dtype: str, group_size: int, bits: int, sb_dtype: str = "bf16"):
    """(packed uint32 [rows, cols*bits/32], scales [rows, cols/G], biases [rows, cols/G]) of a
    [rows, cols] weight given as float32 (``w_dtype="f32"``) or bf16 / float16 bit patterns
    ("bf16", "f16"); scales and biases in ``sb_dtype`` (float32, or bf16 / float16 bit patterns;
    nuvec_core's rule is w's own dtype)."""
    wa = _typed(np.atleast_2d(w), w_dtype)
    if w_dtype not in DTYPES or sb_dtype not in DTYPES:
        raise ValueError((w_dtype, sb_dtype))
    rows, cols = wa.shape
    if group_size <= 0 or cols % group_size or (cols * bits) % 32:
        raise ValueError("cols must be a multiple of the group size")
    packed = np.empty((rows, cols * bits // 32), np.uint32)
    sbt = np.float32 if sb_dtype == "f32" else np.uint16
    sc = np.empty((rows, cols // group_size), sbt)
    bi = np.empty((rows, cols // group_size), sbt)
    _check(_load().orc_quantize_typed(wa.ctypes.data, DTYPES[w_dtype], rows, cols, group_size, bits, packed,
                                      sc.ctypes.data, bi.ctypes.data, DTYPES[sb_dtype]), "quantize")
    return packed, sc, bi


DTYPES = {"f32": 0, "bf16": 1, "f16": 2}


def f16_to_f32(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    _load().orc_f16_to_f32(h.reshape(-1), h.size, out.reshape(-1))
    return out


def f32_to_f16(a: np.ndarray) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    _load().orc_f32_to_f16(a.reshape(-1), a.size, out.reshape(-1))
    return out


def _typed(a, dtype):
    """float32 array for "f32", uint16 bit patterns for "bf16" / "f16"."""
    return _c(a, np.float32 if dtype == "f32" else np.uint16)


def dequantize_typed(packed, scales, biases, sb_dtype: str, group_size: int, bits: int, out: str = "f32"):
    """Dense [rows, cols] from scales and biases of dtype ``sb_dtype`` ("f32", "bf16", "f16"): w = s*c
    then + b in float32, returned as float32 or rounded to "bf16" / "f16" (bit patterns)."""
    packed = _c(np.atleast_2d(packed), np.uint32)
    sc, bi = _typed(np.atleast_2d(scales), sb_dtype), _typed(np.atleast_2d(biases), sb_dtype)
    rows, cols = packed.shape[0], packed.shape[1] * 32 // bits
    res = np.empty((rows, cols), np.float32)
    _check(_load().orc_dequantize_typed(packed, sc.ctypes.data, bi.ctypes.data, DTYPES[sb_dtype], rows, cols,
                                        group_size, bits, res), "dequantize_typed")
    if out == "f32":
        return res
    if out == "bf16":
        return f32_to_bf16(res)
    if out == "f16":
        return f32_to_f16(res)
    raise ValueError(out)


def qmm_typed(x, x_dtype: str, packed, scales, biases, sb_dtype: str, group_size: int, bits: int) -> np.ndarray:
    """y = x . dequantize(W)^T in float64 with x and the scales/biases of any of the three types."""
    xa = _typed(np.atleast_2d(x), x_dtype)
    packed = _c(packed, np.uint32)
    sc, bi = _typed(scales, sb_dtype), _typed(biases, sb_dtype)
    m, k = xa.shape
    n = packed.shape[0]
    out = np.empty((m, n), np.float64)
    _check(_load().orc_qmm_typed(xa.ctypes.data, DTYPES[x_dtype], m, packed, sc.ctypes.data, bi.ctypes.data,
                                 DTYPES[sb_dtype], n, k, group_size, bits, out), "qmm_typed")
    return out


def qmm_nt_typed(x, x_dtype: str, packed, scales, biases, sb_dtype: str, group_size: int, bits: int) -> np.ndarray:
    """y = x . dequantize(W) in float64 for W stored [k, n] (packed [k, n*bits/32], scales and biases
    [k, n/G]), with x and the scales/biases of any of the three types."""
    xa = _typed(np.atleast_2d(x), x_dtype)
    packed = _c(np.atleast_2d(packed), np.uint32)
    sc, bi = _typed(np.atleast_2d(scales), sb_dtype), _typed(np.atleast_2d(biases), sb_dtype)
    m, k = xa.shape
    if packed.shape[0] != k:
        raise ValueError("x columns do not match the weight's rows")
    n = packed.shape[1] * 32 // bits
    out = np.empty((m, n), np.float64)
    _check(_load().orc_qmm_nt_typed(xa.ctypes.data, DTYPES[x_dtype], m, packed, sc.ctypes.data, bi.ctypes.data,
                                    DTYPES[sb_dtype], k, n, group_size, bits, out), "qmm_nt_typed")
    return out


def gather_qmm_typed(x, x_dtype: str, packed, scales, biases, sb_dtype: str, group_size: int, bits: int,
                     lhs=None, rhs=None) -> np.ndarray:
    """gather_qmm with x and the scales/biases of any of the three types: output batch i is
    qmm_typed of x batch lhs[i] against weight batch rhs[i] in float64 (NaN past either operand),
    shape broadcast(batch) + [m, n]."""
    xa = _typed(x, x_dtype)
    packed = _c(packed, np.uint32)
    sc, bi = _typed(scales, sb_dtype), _typed(biases, sb_dtype)
    if xa.ndim < 2 or packed.ndim < 2 or sc.shape != bi.shape:
        raise ValueError("x must be [..., m, k] and w [..., n, k*bits/32]")
    m, k = xa.shape[-2:]
    n = packed.shape[-2]
    if packed.shape[-1] * 32 != k * bits:
        raise ValueError("x columns do not match the packed width")
    li, ri, shape = gather_indices(xa.shape[:-2], packed.shape[:-2], lhs, rhs)
    xb = int(np.prod(xa.shape[:-2], dtype=np.int64))
    wb = int(np.prod(packed.shape[:-2], dtype=np.int64))
    out = np.empty((li.size, m, n), np.float64)
    _check(_load().orc_gather_qmm_typed(xa.ctypes.data, DTYPES[x_dtype], xb, m, packed.reshape(-1), sc.ctypes.data,
                                        bi.ctypes.data, DTYPES[sb_dtype], wb, n, k, group_size, bits, li.ctypes.data,
                                        ri.ctypes.data, li.size, out), "gather_qmm_typed")
    return out.reshape(tuple(shape) + (m, n))


def max_row_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """The matmul comparison: for each output row, the largest |y - ref| divided by the largest
    |ref| of that row (the absolute error where that row of ref is all zero); the result is the
    worst row. Elementwise relative error is meaningless for sums that can land near zero."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    if y.shape != ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {ref.shape}")
    if y.size == 0:
        return 0.0
    err = np.abs(y - ref).max(axis=-1)
    scale = np.abs(ref).max(axis=-1)
    rel = np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), err)
    return float(rel.max())
