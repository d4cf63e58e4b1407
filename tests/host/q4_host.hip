// Host build of the int4 activation code (q4 in csrc/common.hpp, the function every int4
// quantizer kernel calls), driven by tests/test_q4_host.py: for each scale it compares q4
// with the plain definition, rint(fl32(x / s)) clipped to [-8, 7], over every finite bf16 x
// with |x| <= a, and over fp32 x placed on and around each quotient k + 1/2.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "../../ternary_weight_quantized_bitlinear_amd/csrc/common.hpp"

static uint32_t q4_plain(float x, float s) {
    volatile float q = x / s;  // one IEEE division, rounded to nearest even
    float v = rintf(q);
    v = fminf(fmaxf(v, -8.0f), 7.0f);
    return (uint32_t)((int)v) & 0xFu;
}

static float f32(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

// counts[0]: values compared, counts[1]: mismatches, counts[2]: values whose t fell in the
// exact-division band
extern "C" void host_q4_check(const float *amax, int n, uint64_t *counts) {
    counts[0] = counts[1] = counts[2] = 0;
    for (int i = 0; i < n; ++i) {
        const float a = amax[i];
        const float s = a / 7.0f;
        const float r = bl::q4_recip(s);
        auto check = [&](float x) {
            if (!(fabsf(x) <= a)) return;
            ++counts[0];
            if (bl::q4(x, s, r) != q4_plain(x, s)) ++counts[1];
            const float t = x * r, v = rintf(t);
            if (!(fabsf(fabsf(t - v) - 0.5f) >= 0x1p-18f)) ++counts[2];
        };
        for (uint32_t b = 0; b < 65536; ++b) check(f32(b << 16));
        for (int k = -8; k < 8; ++k) {
            const float h = f32(0);
            (void)h;
            // x near (k + 1/2) s: the fp32 neighbours of the product, 64 ulps each way
            float x = (float)((k + 0.5) * (double)s);
            for (int u = 0; u < 64; ++u) x = nextafterf(x, -INFINITY);
            for (int u = 0; u < 129; ++u) {
                check(x);
                x = nextafterf(x, INFINITY);
            }
        }
    }
}
