// Host build of the layer norm's exact-moment helpers (the same header the kernels
// include), driven by tests/test_moments_host.py against exact rational sums.  It runs
// the kernels' algorithm on one row: the anchor is the row's largest biased exponent; the
// row's 8-element groups are dealt to 256 threads as the kernels deal them; per thread,
// S1's window terms go into an int64 and the squares into SqAcc, both flushed into
// 128-bit sums every 128 steps; the values below the window go into exponent bins.  No
// value below the window: mom_window_stats; otherwise mom_bins_stats.
#include <stdint.h>

#include "../../ternary_weight_quantized_bitlinear_amd/csrc/exact_moments.hpp"

extern "C" void host_moments(const uint16_t *x, int64_t K, double *s1_out, double *d_out,
                             int *slow) {
    constexpr int kThreads = 256;
    int E = 1;
    for (int64_t k = 0; k < K; ++k) E = E > bl::sq_exp(x[k]) ? E : bl::sq_exp(x[k]);
    bl::u128 s2 = 0;
    bl::i128 s1 = 0;
    int64_t bins1[256] = {0};
    uint64_t bins2[256] = {0};
    bool spill = false;
    for (int t = 0; t < kThreads; ++t) {
        bl::SqAcc part;
        bl::u128 acc2 = 0;
        bl::i128 acc1 = 0;
        int64_t p1 = 0;
        int steps = 0;
        for (int64_t g = t; 8 * g < K; g += kThreads) {
            for (int j = 0; j < 8 && 8 * g + j < K; ++j) {
                const uint16_t b = x[8 * g + j];
                if (bl::sq_acc_step(b, E, part)) {
                    spill = true;
                    const int e = bl::sq_exp(b);
                    const int64_t m = (b & 0x7F) | (e ? 0x80 : 0);
                    bins1[e ? e : 1] += (b & 0x8000) ? -m : m;
                    bins2[e ? e : 1] += (uint64_t)(m * m);
                }
                p1 += bl::mom_s1_term(b, E);
            }
            steps += 8;
            if (steps % bl::kSqAccSteps == 0) {
                bl::sq_acc_flush(part, acc2);
                acc1 += p1;
                p1 = 0;
            }
        }
        bl::sq_acc_flush(part, acc2);
        acc1 += p1;
        s2 += acc2;
        s1 += acc1;
    }
    *slow = spill ? 1 : 0;
    if (!spill) {
        bl::mom_window_stats(s2, s1, E, K, s1_out, d_out);
        return;
    }
    uint32_t work[3 * bl::kMomLimbs];
    bl::mom_bins_stats(s2, s1, E, bins1, bins2, K, work, s1_out, d_out);
}
