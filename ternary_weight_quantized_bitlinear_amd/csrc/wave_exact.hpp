// Exact integer reductions across a wave (the norm kernels' window sums, "BitNet 2B4T
// Guide", "3. Sub-Layer Normalization (SubLN)").  Device code only.
#pragma once

#include "common.hpp"
#include "exact_sumsq.hpp"

namespace bl {

__device__ __forceinline__ int wave_max_int(int v) {
    v = max(v, dpp_mov<kDppQuadXor1>(0, v));
    v = max(v, dpp_mov<kDppQuadXor2>(0, v));
    v = max(v, dpp_mov<kDppHalfMirror>(0, v));
    v = max(v, dpp_mov<kDppMirror>(0, v));
    v = max(v, dpp_mov<kDppBcast15, 0xA>(0, v));
    v = max(v, dpp_mov<kDppBcast31, 0xC>(0, v));
    return __builtin_amdgcn_readlane(v, 63);
}

// The sum over the wave of each lane's 128-bit integer, exact modulo 2^128: six 24-bit
// digits, each summed with DPP lane moves (64 digits stay below 2^30), then recombined
// with carries.
__device__ __forceinline__ u128 wave_sum_u128(u128 v) {
    u128 total = 0;
#pragma unroll
    for (int d = 0; d < 6; ++d) {
        const int digit = (int)((uint32_t)(v >> (24 * d)) & 0xFFFFFFu);
        total += (u128)(uint32_t)wave_sum(digit) << (24 * d);
    }
    return total;
}

}  // namespace bl
