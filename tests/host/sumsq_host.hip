// Host build of the RMS norm's exact sum-of-squares helpers (the same header the kernels
// include), driven by tests/test_sumsq_host.py against exact rational sums.  It runs the
// kernels' algorithm on one row: the row's 8-element groups are dealt to 256 threads in
// four waves of 64 as the kernels deal them; each wave takes its largest exponent as its
// anchor and sums its squares in its window; the wave sums are combined exactly
// (sq_round_anchored), or, when a value lies below its wave's window or the anchors lie
// far apart, everything is summed again at the row's largest exponent with exponent bins
// for the values below the window (sq_round_with_bins).
#include <stdint.h>

#include "../../ternary_weight_quantized_bitlinear_amd/csrc/exact_sumsq.hpp"

extern "C" double host_sumsq(const uint16_t *x, int64_t K, int *slow) {
    constexpr int kThreads = 256, kWaves = 4;
    int Ew[kWaves] = {0, 0, 0, 0};
    for (int64_t k = 0; k < K; ++k) {
        const int w = (int)(((k / 8) % kThreads) / 64);
        Ew[w] = Ew[w] > bl::sq_exp(x[k]) ? Ew[w] : bl::sq_exp(x[k]);
    }
    int Erow = 1;
    for (int w = 0; w < kWaves; ++w) {
        Ew[w] = Ew[w] > 1 ? Ew[w] : 1;
        Erow = Erow > Ew[w] ? Erow : Ew[w];
    }
    // per lane (thread), as the kernels run it: partial sums flushed every 128 steps
    bl::u128 sums[kWaves] = {0, 0, 0, 0};
    bool spill = false;
    for (int t = 0; t < kThreads; ++t) {
        const int w = t / 64;
        bl::SqAcc part;
        bl::u128 acc = 0;
        int steps = 0;
        for (int64_t g = t; 8 * g < K; g += kThreads) {
            for (int j = 0; j < 8 && 8 * g + j < K; ++j) spill |= bl::sq_acc_step(x[8 * g + j], Ew[w], part);
            steps += 8;
            if (steps % bl::kSqAccSteps == 0) bl::sq_acc_flush(part, acc);
        }
        bl::sq_acc_flush(part, acc);
        sums[w] += acc;
    }
    double S = 0.0;
    if (!spill && Ew[0] == Ew[1] && Ew[1] == Ew[2] && Ew[2] == Ew[3]) {
        *slow = 0;
        return bl::sq_round(sums[0] + sums[1] + sums[2] + sums[3], 2 * Ew[0] - 268 - bl::kSqFrac);
    }
    if (!spill && bl::sq_round_anchored(sums, Ew, kWaves, &S)) {
        *slow = 0;
        return S;
    }
    *slow = 1;
    bl::u128 acc2 = 0;
    uint64_t bins[256] = {0};
    for (int64_t k = 0; k < K; ++k) {
        uint32_t sq;
        int bin;
        if (!bl::sq_window_add(x[k], Erow, acc2, &sq, &bin)) bins[bin] += sq;
    }
    uint32_t big[bl::kSqLimbs];
    return bl::sq_round_with_bins(acc2, Erow, bins, big);
}
