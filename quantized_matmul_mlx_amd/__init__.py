"""qaff: MLX-layout grouped affine dequantization and quantized matmul on AMD MI355X (gfx950).

Thin binding over the C ABI of ``include/qaff.h`` (``libqaff.so``, hand-written HIP kernels). This
layer only marshals arguments: it checks devices, dtypes and contiguity, then passes raw device
pointers and the current HIP stream. Every step of the computation runs in the library's kernels;
if the library is missing, calls raise.

Weights use the MLX layout: ``packed`` uint32 (or int32) [n, k*bits/32] holding each row as a
little-endian bit stream of codes; ``scales`` and ``biases`` bf16 [n, k/group_size] (int16/uint16
bit views are accepted too). A weight is ``scale * code + bias`` of its group.

    y = qmm(x, packed, scales, biases, group_size, bits)   # x . dequantize(W)^T, W never dense
    w = dequantize(packed, scales, biases, group_size, bits, out_dtype=torch.bfloat16)
    packed, scales, biases = quantize(w, group_size, bits)   # bias = group min, bf16 scales
    e = dequant_rows(packed, scales, biases, idx, group_size, bits)   # embedding lookup
    g, u = gemv_gate_up(x, gate_w, up_w, group_size, bits)           # two projections, x read once
    y = gemv_silu_gate(g, u, packed, scales, biases, group_size, bits, resid=r)  # W . (silu(g) * u) + r
    y = gather_qmm(x, packed, scales, biases, group_size, bits, rhs_indices=experts,
                   sorted_indices=True)                     # batch i: x[i] . dequantize(W[experts[i]])^T
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import QaffError

__all__ = ["quantize", "dequantize", "qmm", "qmm_nt", "dequant_rows", "gemv_gate_up", "gemv_silu_gate", "gather_qmm", "QWeight",
           "QaffError", "gemv_max_m", "gemv_mfma_min_m"]

_PACKED_DTYPES = (torch.int32, torch.uint32)
_BF16_BITS_DTYPES = (torch.bfloat16, torch.int16, torch.uint16)
_INDEX_DTYPES = (torch.int32, torch.uint32)
_GATHER_INDEX_DTYPES = (torch.int32, torch.uint32, torch.int64)
_OUT_DTYPES = {torch.float32: _lib.QAFF_F32, torch.bfloat16: _lib.QAFF_BF16}
# every float type the typed entry points take (x, scales and biases, outputs)
_ANY_DTYPES = {torch.float32: _lib.QAFF_F32, torch.bfloat16: _lib.QAFF_BF16, torch.float16: _lib.QAFF_F16}
_FROM_CODE = {v: k for k, v in _ANY_DTYPES.items()}
_SCALE_DTYPES = _BF16_BITS_DTYPES + (torch.float16, torch.float32)


def _sb_code(scales):
    """dtype code of the scales: float16 and float32 tensors as such, anything else bf16 bits."""
    return _ANY_DTYPES.get(scales.dtype, _lib.QAFF_BF16) if scales.dtype in (torch.float16, torch.float32) \
        else _lib.QAFF_BF16


def _need(t, name, dtypes, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _weights(packed, scales, biases, group_size, bits, typed=False):
    """Checks a weight; returns (device, rows, cols). Only ``typed`` callers (qmm, qmm_nt,
    gather_qmm, dequantize) take float16 or float32 scales and biases; the other operations read
    bf16 ones."""
    _need(packed, "packed", _PACKED_DTYPES)
    dev = packed.device
    _need(scales, "scales", _SCALE_DTYPES, dev)
    _need(biases, "biases", _SCALE_DTYPES, dev)
    if _sb_code(scales) != _sb_code(biases):
        raise TypeError(f"scales ({scales.dtype}) and biases ({biases.dtype}) differ in type")
    if not typed and _sb_code(scales) != _lib.QAFF_BF16:
        raise TypeError(f"this operation reads bf16 scales and biases, got {scales.dtype} "
                        "(float16 and float32 scales are taken by qmm, qmm_nt, gather_qmm and dequantize)")
    if packed.dim() != 2 or scales.dim() != 2 or biases.dim() != 2:
        raise ValueError("packed, scales and biases must be 2-D")
    rows, words = packed.shape
    if (words * 32) % bits:
        raise ValueError(f"packed width {words} is not a whole number of {bits}-bit codes")
    cols = words * 32 // bits
    if group_size <= 0 or cols % group_size:
        raise ValueError(f"{cols} columns are not a multiple of the group size {group_size}")
    want = (rows, cols // group_size)
    if tuple(scales.shape) != want or tuple(biases.shape) != want:
        raise ValueError(f"scales/biases must be {list(want)}, got {list(scales.shape)} and "
                         f"{list(biases.shape)}")
    return dev, rows, cols


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else None


def gemv_max_m() -> int:
    """Largest number of x rows the automatic dispatch sends to the decode path for a bf16 x."""
    return int(_lib.load().qaff_gemv_max_m())


def gemv_mfma_min_m(k: int = 0) -> int:
    """Smallest number of bf16 x rows the automatic dispatch sends to the matrix-core decode
    kernel (for the shapes it takes) at a K of k codes: the library's figure up to 4096, 2 above
    (the rule qaff.h states for qaff_gemv_mfma_min_m)."""
    return 2 if k > 4096 else int(_lib.load().qaff_gemv_mfma_min_m())


def dequantize(packed, scales, biases, group_size: int, bits: int, out_dtype=torch.float32,
               out=None):
    """Dense ``[rows, cols]`` weights (rlx-moshi ``dequantize_affine``; maya2_mlx ``QW.dense``).
    Scales and biases may be bf16, float16 or float32, and the output float32, bf16 or float16."""
    lib = _lib.load()
    dev, rows, cols = _weights(packed, scales, biases, group_size, bits, typed=True)
    if out_dtype not in _ANY_DTYPES:
        raise TypeError(f"out_dtype must be float32, bfloat16 or float16, got {out_dtype}")
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=dev)
    else:
        _need(out, "out", (out_dtype,), dev)
        if tuple(out.shape) != (rows, cols):
            raise ValueError(f"out must be [{rows}, {cols}]")
    with torch.cuda.device(dev):
        _lib.check(lib.qaff_dequantize_typed(_p(packed), _p(scales), _p(biases), _sb_code(scales), rows, cols,
                                             group_size, bits, _p(out), _ANY_DTYPES[out_dtype], _stream(dev)))
    return out


def quantize(w, group_size: int, bits: int, scales_dtype=None):
    """Quantizes the last axis of a float32, bf16 or float16 weight ``[..., cols]`` (nuvec_core
    ``quantize``): returns packed uint32 ``[..., cols*bits/32]`` (as int32), and scales and biases
    ``[..., cols/group_size]`` in ``scales_dtype`` (default: w's dtype, nuvec_core's rule; bf16 is
    what the products other than the ``*_typed`` ones read); bias = group minimum, scale =
    (max - min) / (2^bits - 1)."""
    lib = _lib.load()
    _need(w, "w", tuple(_ANY_DTYPES))
    sdt = w.dtype if scales_dtype is None else scales_dtype
    if sdt not in _ANY_DTYPES:
        raise TypeError(f"scales_dtype must be float32, bfloat16 or float16, got {sdt}")
    dev = w.device
    if w.dim() < 1:
        raise ValueError("w must have at least one dimension")
    cols = w.shape[-1]
    lead = tuple(w.shape[:-1])
    rows = math.prod(lead)
    if group_size <= 0 or cols % group_size:
        raise ValueError(f"{cols} columns are not a multiple of the group size {group_size}")
    packed = torch.empty(lead + (cols * bits // 32,), dtype=torch.int32, device=dev)
    scales = torch.empty(lead + (cols // group_size,), dtype=sdt, device=dev)
    biases = torch.empty(lead + (cols // group_size,), dtype=sdt, device=dev)
    with torch.cuda.device(dev):
        _lib.check(lib.qaff_quantize_typed(_p(w), _ANY_DTYPES[w.dtype], rows, cols, group_size, bits, _p(packed),
                                           _p(scales), _p(biases), _ANY_DTYPES[sdt], _stream(dev)))
    return packed, scales, biases


def qmm_nt(x, packed, scales, biases, group_size: int, bits: int, out=None, static_scratch: bool = False):
    """``x . dequantize(W)`` for a weight stored ``[k, n]`` (nuvec_core ``quantized_matmul`` with
    ``transpose=False``): packed ``[k, n*bits/32]``, scales and biases ``[k, n/group_size]``;
    x ``[..., k]`` (1-D: one row); the result has shape ``[..., n]``.
    x float32 or bf16 with bf16 scales: the result has x's dtype. x may also be float16 and the
    scales and biases float16 or float32 (``qaff_qmm_nt_typed``): x, scales and biases then promote
    to one type (float32 unless they agree), which is the result's type.
    The call's float32 K-chunk partial sums go to a workspace tensor allocated here, or with
    ``static_scratch`` (and ``out`` given; float32 or bf16 x, bf16 scales) to the library's
    per-device scratch array (``qaff_qmm_nt_static``): the call then allocates nothing."""
    lib = _lib.load()
    dev, k, n = _weights(packed, scales, biases, group_size, bits, typed=True)
    _need(x, "x", tuple(_ANY_DTYPES), dev)
    if x.shape[-1] != k:
        raise ValueError(f"x has {x.shape[-1]} columns, the weight {k} rows")
    sb = _sb_code(scales)
    typed = sb != _lib.QAFF_BF16 or x.dtype == torch.float16
    yt = _FROM_CODE[int(lib.qaff_promote_dtype(_ANY_DTYPES[x.dtype], sb))]
    lead = tuple(x.shape[:-1])
    m = math.prod(lead)
    if out is None:
        out = torch.empty(lead + (n,), dtype=yt, device=dev)
    else:
        _need(out, "out", (yt,), dev)
        if tuple(out.shape) != lead + (n,):
            raise ValueError(f"out must be {list(lead + (n,))}")
    if static_scratch:
        if typed:
            raise TypeError("the static scratch takes float32 or bf16 x with bf16 scales and biases")
        with torch.cuda.device(dev):
            _lib.check(lib.qaff_qmm_nt_static(_p(x), _OUT_DTYPES[x.dtype], m, _p(packed), _p(scales), _p(biases), k,
                                              n, group_size, bits, _p(out), _stream(dev)))
        return out
    nbytes = int(lib.qaff_qmm_nt_workspace_size(m, k, n, bits))
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    with torch.cuda.device(dev):
        if typed:
            _lib.check(lib.qaff_qmm_nt_typed(_p(x), _ANY_DTYPES[x.dtype], m, _p(packed), _p(scales), _p(biases), sb,
                                             k, n, group_size, bits, _p(ws), ws.numel(), _p(out), _stream(dev)))
        else:
            _lib.check(lib.qaff_qmm_nt(_p(x), _OUT_DTYPES[x.dtype], m, _p(packed), _p(scales), _p(biases), k, n,
                                       group_size, bits, _p(ws), ws.numel(), _p(out), _stream(dev)))
    return out


def qmm(x, packed, scales, biases, group_size: int, bits: int, path: str = "auto", out=None,
        transpose: bool = True):
    """``x . dequantize(W)^T`` (nuvec_core ``quantized_matmul`` with transpose; maya2_mlx ``mm``).

    x is float32 or bf16 ``[..., k]`` (a 1-D x is one row); the result has x's dtype and shape
    ``[..., n]``. ``path`` forces a kernel ("gemv", "gemv_mfma" or "gemm") for tests and
    benchmarks.

    A weight with batch dimensions (packed ``[..., n, k*bits/32]``) multiplies x ``[..., m, k]``
    batch by batch, the batch dimensions of both broadcast together (a 2-D x takes the weight's
    batch; a 1-D x is a row vector and the result drops that row): the gathered product with
    its default indices.

    ``transpose=False`` computes ``x . dequantize(W)`` for a weight stored ``[k, n]``
    (``qmm_nt``).

    x may also be float16, and the scales and biases float16 or float32: x, scales and biases then
    promote to one type (float32 unless they agree), which is y's type. A float16 x with float16
    scales and biases runs on the float16 forms of the kernels above, chosen as for bf16; other
    mixes on a typed VALU kernel. Either way the library picks the kernel (path 'auto')."""
    if not transpose:
        if path != "auto":
            raise ValueError("the product without the transpose has one kernel: path 'auto'")
        return qmm_nt(x, packed, scales, biases, group_size, bits, out=out)
    if isinstance(packed, torch.Tensor) and packed.dim() > 2:
        if path == "gemm":
            raise ValueError("a batched weight runs on the gathered kernels: path 'auto', 'gemv' or 'gemv_mfma'")
        vector = isinstance(x, torch.Tensor) and x.dim() == 1
        y = gather_qmm(x[None] if vector else x, packed, scales, biases, group_size, bits, path=path, out=out)
        return y.squeeze(-2) if vector else y
    lib = _lib.load()
    dev, n, k = _weights(packed, scales, biases, group_size, bits, typed=True)
    _need(x, "x", tuple(_ANY_DTYPES), dev)
    if x.shape[-1] != k:
        raise ValueError(f"x has {x.shape[-1]} columns, the weight {k}")
    if path not in _lib.PATHS:
        raise ValueError(f"path must be one of {tuple(_lib.PATHS)}")
    sb = _sb_code(scales)
    if sb != _lib.QAFF_BF16 or x.dtype == torch.float16:
        # x, scales and biases promote to one type (float32 unless they agree); the library picks
        # the kernel
        if path != "auto":
            raise ValueError("float16 x or non-bf16 scales take the automatic path: path 'auto'")
        lead = tuple(x.shape[:-1])
        m = math.prod(lead)
        yt = _FROM_CODE[int(lib.qaff_promote_dtype(_ANY_DTYPES[x.dtype], sb))]
        if out is None:
            out = torch.empty(lead + (n,), dtype=yt, device=dev)
        else:
            _need(out, "out", (yt,), dev)
            if tuple(out.shape) != lead + (n,):
                raise ValueError(f"out must be {list(lead + (n,))}")
        with torch.cuda.device(dev):
            _lib.check(lib.qaff_qmm_typed(_p(x), _ANY_DTYPES[x.dtype], m, _p(packed), _p(scales), _p(biases), sb, n,
                                          k, group_size, bits, _p(out), _stream(dev)))
        return out
    lead = tuple(x.shape[:-1])
    m = math.prod(lead)
    x2 = x.reshape(m, k)
    if out is None:
        out = torch.empty(lead + (n,), dtype=x.dtype, device=dev)
    else:
        _need(out, "out", (x.dtype,), dev)
        if tuple(out.shape) != lead + (n,):
            raise ValueError(f"out must be {list(lead + (n,))}")
    # the automatic path of a bf16 x may split K through a workspace (few tiles of the GEMM)
    nbytes = int(lib.qaff_qmm_workspace_size(m, n, k, group_size, bits)) if (
        path == "auto" and x.dtype == torch.bfloat16) else 0
    with torch.cuda.device(dev):
        if nbytes > 0:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            _lib.check(lib.qaff_qmm_ws(_p(x2), _OUT_DTYPES[x.dtype], m, _p(packed), _p(scales), _p(biases), n, k,
                                       group_size, bits, _p(ws), ws.numel(), _p(out), _stream(dev)))
        else:
            _lib.check(lib.qaff_qmm_ex(_p(x2), _OUT_DTYPES[x.dtype], m, _p(packed), _p(scales),
                                       _p(biases), n, k, group_size, bits, _p(out), _stream(dev),
                                       _lib.PATHS[path]))
    return out


def dequant_rows(packed, scales, biases, indices, group_size: int, bits: int,
                 out_dtype=torch.float32, out=None):
    """Dequantized rows ``indices`` of a quantized table (maya2_mlx ``rows``). Indices are int32
    or uint32 and are read as uint32; an index past the table gives a row of NaNs."""
    lib = _lib.load()
    dev, rows, cols = _weights(packed, scales, biases, group_size, bits)
    _need(indices, "indices", _INDEX_DTYPES, dev)
    idx = indices.reshape(-1)
    if out_dtype not in _OUT_DTYPES:
        raise TypeError(f"out_dtype must be float32 or bfloat16, got {out_dtype}")
    shape = tuple(indices.shape) + (cols,)
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=dev)
    else:
        _need(out, "out", (out_dtype,), dev)
        if tuple(out.shape) != shape:
            raise ValueError(f"out must be {list(shape)}")
    with torch.cuda.device(dev):
        _lib.check(lib.qaff_dequant_rows(_p(packed), _p(scales), _p(biases), rows, cols, group_size,
                                         bits, _p(idx), idx.numel(), _p(out),
                                         _OUT_DTYPES[out_dtype], _stream(dev)))
    return out


class QWeight:
    """A quantized ``[out, in]`` weight (maya2_mlx ``QW``): packed codes, scales, biases, bits and
    group size. The caller owns the tensors."""

    __slots__ = ("q", "scales", "biases", "bits", "group_size", "shape")

    def __init__(self, q, scales, biases, bits: int, group_size: int):
        self.q, self.scales, self.biases = q, scales, biases
        self.bits, self.group_size = int(bits), int(group_size)
        _, rows, cols = _weights(q, scales, biases, self.group_size, self.bits, typed=True)
        self.shape = (rows, cols)

    def dense(self, dtype=torch.float32):
        return dequantize(self.q, self.scales, self.biases, self.group_size, self.bits, dtype)

    def mm(self, x, path: str = "auto"):
        """x @ W.T"""
        return qmm(x, self.q, self.scales, self.biases, self.group_size, self.bits, path)

    def rows(self, idx, dtype=torch.float32):
        return dequant_rows(self.q, self.scales, self.biases, idx, self.group_size, self.bits, dtype)


def _rows_2d(t, name, k, dev):
    """A bf16 [..., k] decode input as [m, k] (a 1-D input is one row) and its leading shape."""
    _need(t, name, (torch.bfloat16,), dev)
    if t.shape[-1] != k:
        raise ValueError(f"{name} has {t.shape[-1]} columns, the weight {k}")
    lead = tuple(t.shape[:-1])
    return t.reshape(math.prod(lead), k), lead


def gemv_gate_up(x, gate_w, up_w, group_size: int, bits: int):
    """Both projections of one bf16 x in one launch (spark_runtime ``gemv_gate_up``): returns
    ``(x . dequantize(gate)^T, x . dequantize(up)^T)``. ``gate_w`` and ``up_w`` are
    ``(packed, scales, biases)`` of the same shape; at most 16 rows of x."""
    lib = _lib.load()
    dev, n, k = _weights(*gate_w, group_size, bits)
    dev2, n2, k2 = _weights(*up_w, group_size, bits)
    if (dev2, n2, k2) != (dev, n, k):
        raise ValueError("gate and up weights differ in device or shape")
    x2, lead = _rows_2d(x, "x", k, dev)
    gy = torch.empty(lead + (n,), dtype=torch.bfloat16, device=dev)
    uy = torch.empty(lead + (n,), dtype=torch.bfloat16, device=dev)
    with torch.cuda.device(dev):
        _lib.check(lib.qaff_gemv_gate_up(_p(x2), x2.shape[0], _p(gate_w[0]), _p(gate_w[1]), _p(gate_w[2]),
                                         _p(up_w[0]), _p(up_w[1]), _p(up_w[2]), n, k, group_size, bits,
                                         _p(gy), _p(uy), _stream(dev)))
    return gy, uy


def gemv_silu_gate(gate, up, packed, scales, biases, group_size: int, bits: int, resid=None):
    """``(silu(gate) * up) . dequantize(W)^T (+ resid)`` in one launch (spark_runtime
    ``gemv_silu_gate`` / ``gemv_silu_gate_resid``); gate and up bf16 ``[..., k]`` (at most 16
    rows), resid bf16 ``[..., n]`` or None; the result is bf16 ``[..., n]``."""
    lib = _lib.load()
    dev, n, k = _weights(packed, scales, biases, group_size, bits)
    g2, lead = _rows_2d(gate, "gate", k, dev)
    u2, lead_u = _rows_2d(up, "up", k, dev)
    if lead_u != lead:
        raise ValueError("gate and up differ in shape")
    r2 = None
    if resid is not None:
        _need(resid, "resid", (torch.bfloat16,), dev)
        if tuple(resid.shape) != lead + (n,):
            raise ValueError(f"resid must be {list(lead + (n,))}")
        r2 = resid
    y = torch.empty(lead + (n,), dtype=torch.bfloat16, device=dev)
    with torch.cuda.device(dev):
        _lib.check(lib.qaff_gemv_silu_gate(_p(g2), _p(u2), g2.shape[0], _p(packed), _p(scales), _p(biases),
                                           n, k, group_size, bits, _p(r2), _p(y), _stream(dev)))
    return y


def _batch_indices(given, batch_shape, name, dev):
    """One operand's indices of a gathered product (nuvec_core ``gather_indices``): the given
    integer tensor, or every batch of the operand in order (None stands for that while its shape is
    the broadcast one)."""
    if given is None:
        return None, tuple(batch_shape)
    _need(given, name, _GATHER_INDEX_DTYPES, dev)
    return given, tuple(given.shape)


def _expand_indices(t, own_shape, shape, dev):
    """Indices as a contiguous int32/uint32 tensor of the broadcast shape (argument marshalling:
    a default becomes an explicit arange only when it has to broadcast)."""
    if t is None:
        if own_shape == shape:
            return None
        t = torch.arange(math.prod(own_shape), dtype=torch.int32, device=dev).reshape(own_shape)
    elif t.dtype == torch.int64:
        t = t.to(torch.int32)  # the low 32 bits: the same uint32 value as a cast of the integer
    if tuple(t.shape) != shape:
        t = t.expand(shape)
    return t.contiguous()


def gather_qmm(x, packed, scales, biases, group_size: int, bits: int, lhs_indices=None, rhs_indices=None,
               sorted_indices: bool = False, path: str = "auto", out=None):
    """Quantized products of gathered batches (nuvec_core ``gather_qmm`` with the transpose):
    output batch i is ``x[lhs[i]] . dequantize(W[rhs[i]])^T`` over the flattened batch dimensions
    of x ``[..., m, k]`` and of the weight (packed ``[..., n, k*bits/32]``, scales and biases
    ``[..., n, k/group_size]``). Indices are integer tensors that broadcast together, each
    defaulting to every batch of its operand; an index past its operand gives a NaN batch.
    ``sorted_indices`` promises that ``rhs_indices`` is sorted (rows grouped by expert), which lets
    the kernel read each expert's weights once. The result has shape ``broadcast(batch) + [m, n]``.

    x is float32, bf16 or float16 and the scales and biases bf16, float16 or float32: they promote
    to one type (float32 unless they agree), which is the result's type. A float16 x or scales
    other than bf16 take the automatic path: the float16 forms of the bf16 kernels where x, scales
    and biases are all float16, a typed VALU kernel otherwise (path 'auto')."""
    lib = _lib.load()
    _need(packed, "packed", _PACKED_DTYPES)
    dev = packed.device
    if packed.dim() < 2 or scales.dim() < 2 or tuple(scales.shape[:-2]) != tuple(packed.shape[:-2]):
        raise ValueError("packed must be [..., n, k*bits/32] and scales, biases [..., n, k/group_size]")
    if tuple(biases.shape) != tuple(scales.shape):
        raise ValueError("scales and biases differ in shape")
    w_batch = tuple(packed.shape[:-2])
    wb = math.prod(w_batch)
    n = packed.shape[-2]
    _, _, k = _weights(packed.reshape(-1, packed.shape[-1]), scales.reshape(-1, scales.shape[-1]),
                       biases.reshape(-1, biases.shape[-1]), group_size, bits, typed=True)
    _need(x, "x", tuple(_ANY_DTYPES), dev)
    sb = _sb_code(scales)
    typed = sb != _lib.QAFF_BF16 or x.dtype == torch.float16
    yt = _FROM_CODE[int(lib.qaff_promote_dtype(_ANY_DTYPES[x.dtype], sb))]
    if x.dim() < 2:
        raise ValueError("x must be [..., m, k]")
    m = x.shape[-2]
    if x.shape[-1] != k:
        raise ValueError(f"x has {x.shape[-1]} columns, the weight {k}")
    if path not in ("auto", "gemv", "gemv_mfma", "gemm"):
        raise ValueError("path must be 'auto', 'gemv', 'gemv_mfma' or 'gemm'")
    if typed and path != "auto":
        raise ValueError("float16 x or non-bf16 scales take the automatic path: path 'auto'")
    x_batch = tuple(x.shape[:-2])
    lhs, lhs_shape = _batch_indices(lhs_indices, x_batch, "lhs_indices", dev)
    rhs, rhs_shape = _batch_indices(rhs_indices, w_batch, "rhs_indices", dev)
    shape = tuple(torch.broadcast_shapes(lhs_shape, rhs_shape))
    lhs = _expand_indices(lhs, lhs_shape, shape, dev)
    rhs = _expand_indices(rhs, rhs_shape, shape, dev)
    batch = math.prod(shape)
    want = shape + (m, n)
    if out is None:
        out = torch.empty(want, dtype=yt, device=dev)
    else:
        _need(out, "out", (yt,), dev)
        if tuple(out.shape) != want:
            raise ValueError(f"out must be {list(want)}")
    with torch.cuda.device(dev):
        if typed:
            _lib.check(lib.qaff_gather_qmm_typed(_p(x), _ANY_DTYPES[x.dtype], math.prod(x_batch), m, _p(packed),
                                                 _p(scales), _p(biases), sb, wb, n, k, group_size, bits, _p(lhs),
                                                 _p(rhs), batch, 1 if sorted_indices else 0, _p(out), _stream(dev)))
        else:
            _lib.check(lib.qaff_gather_qmm_ex(_p(x), _OUT_DTYPES[x.dtype], math.prod(x_batch), m, _p(packed),
                                              _p(scales), _p(biases), wb, n, k, group_size, bits, _p(lhs),
                                              _p(rhs), batch, 1 if sorted_indices else 0, _p(out), _stream(dev),
                                              _lib.PATHS[path]))
    return out
