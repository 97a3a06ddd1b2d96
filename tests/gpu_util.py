"""Helpers for the GPU tests: move seeded numpy inputs to the device and results back. No method
arithmetic here: bf16 values move as bit patterns."""
import sys

import numpy as np
import torch


def banner(msg):
    """Names the case on stdout before a GPU step, so a run that dies still says where."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev_u32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint32).view(np.int32)).cuda()


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def dev_x(x, x_dtype):
    if x_dtype == "bf16":
        return dev_bf16(x)
    if x_dtype == "f16":   # float16 bit patterns
        return torch.from_numpy(np.ascontiguousarray(x, np.uint16).view(np.int16)).cuda().view(torch.float16)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def dev_weights(inp):
    return dev_u32(inp.packed), dev_bf16(inp.scales), dev_bf16(inp.biases)


def host_bits(t):
    """bf16 or float16 tensor -> uint16 bit patterns; float32 tensor -> float32 array."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def host_f64(t):
    t = t.detach().cpu()
    return t.float().numpy().astype(np.float64)


def at_offset(t, elements=1):
    """A contiguous copy of t that starts `elements` elements past a fresh allocation (2 bytes for
    bf16: not 4- or 16-byte aligned)."""
    flat = t.reshape(-1)
    big = torch.empty(flat.numel() + elements, dtype=t.dtype, device=t.device)
    view = big[elements:]
    view.copy_(flat)
    return view.view(t.shape)


def mfma_rows_per_tile(rows):
    """x rows per tile of the matrix-core decode and gathered kernels: rows rounded up to 4, 8 or 16."""
    return 4 if rows <= 4 else 8 if rows <= 8 else 16


def mfma_exact_codes(bits, G, rows):
    """Whether those kernels multiply 4-bit codes exactly (scale and bias applied to each group's
    sums, weights never rounded to bf16): a chunk's 4 >> log2(G / 32) groups each take a band of
    the tile's rows among the 16 operand rows. Their own arithmetic is then the float32 oracle."""
    return bits == 4 and (4 >> {32: 0, 64: 1, 128: 2}[G]) * mfma_rows_per_tile(rows) <= 16


def grouped_rows_per_tile(batch, experts):
    """The grouped walk's rows per tile: twice the mean rows per expert, rounded up."""
    return (2 * batch + experts - 1) // max(experts, 1)
