// Host build of the RMS norm's exact sum-of-squares helpers (the same header the kernels
// include), driven by tests/test_sumsq_host.py against exact rational sums.  It runs the
// kernel's algorithm on one row: the row's largest exponent, the window sum, the bins
// for values below the window, then the fast or the slow rounding.
#include <stdint.h>

#include "../../ternary_weight_quantized_bitlinear_amd/csrc/exact_sumsq.hpp"

extern "C" double host_sumsq(const uint16_t *x, int64_t K, int *slow) {
    int E = 1;
    for (int64_t k = 0; k < K; ++k) E = E > bl::sq_exp(x[k]) ? E : bl::sq_exp(x[k]);
    bl::u128 acc = 0;
    uint64_t bins[256] = {0};
    int spill = 0;
    for (int64_t k = 0; k < K; ++k) {
        uint32_t sq;
        int bin;
        if (!bl::sq_window_add(x[k], E, acc, &sq, &bin)) {
            bins[bin] += sq;
            spill = 1;
        }
    }
    *slow = spill;
    if (!spill) return bl::sq_round(acc, 2 * E - 268 - bl::kSqFrac);
    uint32_t big[bl::kSqLimbs];
    return bl::sq_round_with_bins(acc, E, bins, big);
}
