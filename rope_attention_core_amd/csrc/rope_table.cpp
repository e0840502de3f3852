// Host-side FP32 RoPE table (sa3attn_rope_table, declared in include/sa3attn.h).
//
// The cos/sin values are computed on the host and handed to the kernel as a frozen
// FP32 table, with no trigonometry inside the attention core (sa3_trt README,
// section "DiT precision", the fp8 tier's baked FP32 RoPE table). Each entry is one
// rounding of the double-precision value: fp32(cos(fp64(m) * theta_i)) with
// theta_i = base^(-2 i / D) as the double nearest the real value. Evaluating the
// angle in a narrow type is what broke the retired bf16 tier (same section): at
// ~4155 rad a bf16 angle has 32 rad spacing.

#include <cmath>

#include "sa3attn.h"

extern "C" int sa3attn_rope_table(float *cos_out, float *sin_out, int L, int D, double base) {
    if (!cos_out || !sin_out) return SA3_ERR_NULL;
    if (L < 1 || D < 2 || (D & 1)) return SA3_ERR_SHAPE;
    if (!std::isfinite(base) || !(base > 0.0)) return SA3_ERR_ARG;
    const int half = D / 2;
    for (int i = 0; i < half; ++i) {
        // theta_i rounded once to double from an extended-precision power: a plain
        // double pow() may be off by one unit in the last place for some i, which
        // shifts the FP32 entries at large positions.
        const double theta = (double)powl((long double)base, -2.0L * (long double)i / (long double)D);
        for (int m = 0; m < L; ++m) {
            const double phi = (double)m * theta;
            cos_out[(size_t)m * half + i] = (float)std::cos(phi);
            sin_out[(size_t)m * half + i] = (float)std::sin(phi);
        }
    }
    return SA3_OK;
}
