"""Test inputs for quantize: groups whose values sit within a few float32 ulps of the rounding
boundaries bias + (k + 1/2) * scale, with minima of very different magnitudes so that w - bias is
often not a float32. Input construction only: the scale and bias here are the roundings of the
group's float32 statistics to the scales' type (torch's bf16 conversion, numpy's float16 one, or
float32 as is), so that the values land near the boundaries the quantizer will use."""
import numpy as np
import torch


def bf16_rne(v):
    """float32 -> bf16 bits (round to nearest even) through torch's conversion."""
    t = torch.tensor(np.asarray(v, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_value(v):
    """The float32 value of the bf16 rounding of v."""
    return (bf16_rne(v).astype(np.uint32) << 16).view(np.float32)


def f16_value(v):
    """The float32 value of the float16 rounding of v (numpy's conversion, round to nearest even)."""
    return np.asarray(v, np.float32).astype(np.float16).astype(np.float32)


def f32_value(v):
    return np.asarray(v, np.float32)


def near_tie_groups(rows, groups, G, bits, seed, w_type=np.float32, stored=bf16_value):
    """Groups of w_type values (float32 or float16) near the boundaries of the scale and bias as
    `stored` (the float32 value of the scales' type: bf16_value, f16_value or f32_value) keeps
    them."""
    rng = np.random.default_rng(seed)
    top = 2 ** bits - 1
    lo_exp = -40 if w_type == np.float32 else -10
    w = np.zeros((rows, groups * G), w_type)
    for r in range(rows):
        for g in range(groups):
            lo = w_type(rng.choice([-1.0, 1.0]) * 2.0 ** rng.integers(lo_exp, 2) * rng.uniform(0.5, 1.0))
            hi = w_type(lo + abs(lo) * rng.uniform(0.5, 8.0) + rng.uniform(0.0, 1.0))
            s = float(stored([(np.float32(hi) - np.float32(lo)) / np.float32(top)])[0])
            b = float(stored([np.float32(lo)])[0])
            vals = []
            for _ in range(G - 2):
                v = w_type(b + (rng.integers(0, top + 1) + 0.5) * s)
                for _ in range(abs(int(rng.integers(-2, 3)))):
                    v = np.nextafter(v, w_type(np.inf) if rng.random() < 0.5 else w_type(-np.inf))
                vals.append(min(max(v, lo), hi))
            w[r, g * G:(g + 1) * G] = rng.permutation(np.array([lo, hi] + vals, w_type))
    return w


def tie_example():
    """A 4-bit group of 32 (min 2^-100, max 0.9375, so scale 0.0625 and bias 2^-100) holding
    3.5 * 0.0625 and 5.5 * 0.0625: their exact quotients fall just below the ties."""
    w = np.full((1, 32), 0.5, np.float32)
    w[0, 0], w[0, 1], w[0, 2], w[0, 3] = np.float32(2.0 ** -100), 0.9375, 0.21875, 0.34375
    return w
