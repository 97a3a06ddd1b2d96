/* The quantize kernel's fast decision, emulated in float32 on the CPU (test infrastructure).
 * For each value: t = fma(v - bias, 1/scale, 1/2), code = floor(t) clamped to [0, top], unless
 * t's fraction lies within 2^-12 of an integer (or is NaN): then the value is flagged "near" and
 * the kernel decides it with its exact test instead. A scale of 0 gives code 0.
 * Compiled without contraction, so each operation rounds once, as the kernel's do. */
#include <math.h>
#include <stdint.h>

void fast_decisions(const float* w, int64_t rows, int64_t cols, int32_t group, const float* scales,
                    const float* biases, int32_t top, int32_t* code, uint8_t* near) {
    const int64_t gpr = cols / group;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < cols; ++j) {
            const float s = scales[r * gpr + j / group];
            const float b = biases[r * gpr + j / group];
            const float rcp = s != 0.0f ? 1.0f / s : 0.0f;
            const float d = w[r * cols + j] - b;
            const float t = fmaf(d, rcp, 0.5f);
            const float c0 = floorf(t);
            const float fr = (t - c0) - 0.5f;
            const int is_near = !(fabsf(fr) < 0.5f - 0x1p-12f);
            float c = fminf(fmaxf(c0, 0.0f), (float)top);
            if (s == 0.0f) c = 0.0f;
            code[r * cols + j] = (int32_t)c;
            near[r * cols + j] = (uint8_t)(is_near && s != 0.0f);
        }
}
