// Register bitonic sort of 64-bit selection keys across one wave, shared by the merge
// and the two-stage fine selection: lane l holds elements EPL*l .. EPL*l + EPL-1 of a
// 64*EPL-key network (EPL = 2^LE); strides below EPL compare within a lane, larger ones
// exchange with lane l ^ (stride / EPL).  Padding keys are 0, below every real key.
#pragma once

#include "si_common.hpp"

namespace si {

// 64-bit lane exchange: partner lane ^ m (DPP within a quad for m = 1, 2)
template <int M>
__device__ __forceinline__ uint64_t xor_lane64(uint64_t v) {
    if constexpr (M == 1 || M == 2) {
        constexpr int C = M == 1 ? kDppQuadSwap1 : kDppQuadSwap2;
        const uint32_t lo = dpp<C>(0u, (uint32_t)v), hi = dpp<C>(0u, (uint32_t)(v >> 32));
        return ((uint64_t)hi << 32) | lo;
    } else {
        return __shfl_xor(v, M);
    }
}

// One bitonic stage: blocks of 2^S elements, compare distance 2^T, LE = log2(EPL).
// A block sorts descending when bit S of its element index is 0 (the whole network's
// block always); bit S >= LE of the index EPL*lane + e is lane bit S - LE.
template <int LE, int S, int T>
__device__ __forceinline__ void bitonic_stage(uint64_t (&x)[1 << LE], int lane) {
    constexpr int EPL = 1 << LE, LN = LE + 6;   // log2 of the network size
    const bool desc_lane = S == LN || ((lane >> (S >= LE ? S - LE : 0)) & 1) == 0;
    if constexpr (T >= LE) {
        constexpr int M = 1 << (T - LE);
        // the lane with the lower index keeps the larger key in a descending block
        const bool keep_max = ((lane & M) == 0) == desc_lane;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const uint64_t p = xor_lane64<M>(x[e]);
            x[e] = (x[e] > p) == keep_max ? x[e] : p;
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            if (e & (1 << T)) continue;
            const int e2 = e | (1 << T);
            const bool desc = S >= LE ? desc_lane : ((e >> S) & 1) == 0;
            const bool swap = (x[e] > x[e2]) != desc;
            const uint64_t a = x[e], b = x[e2];
            x[e] = swap ? b : a;
            x[e2] = swap ? a : b;
        }
    }
}

template <int LE, int S, int T>
__device__ __forceinline__ void bitonic_merge_steps(uint64_t (&x)[1 << LE], int lane) {
    bitonic_stage<LE, S, T>(x, lane);
    if constexpr (T > 0) bitonic_merge_steps<LE, S, T - 1>(x, lane);
}

template <int LE, int S>
__device__ __forceinline__ void bitonic_blocks(uint64_t (&x)[1 << LE], int lane) {
    bitonic_merge_steps<LE, S, S - 1>(x, lane);
    if constexpr (S < LE + 6) bitonic_blocks<LE, S + 1>(x, lane);
}

// Sorts the 64*EPL keys x (element EPL*lane + e in x[e]) into descending order.
template <int LE>
__device__ __forceinline__ void sort_desc(uint64_t (&x)[1 << LE]) {
    bitonic_blocks<LE, 1>(x, lane_id());
}

// Writes one output row: the first n (<= k) of the sorted keys x (element EPL*lane + e
// in x[e]) as (index, score), then -1 / -inf up to k.  oi / os point at the row.
template <int LE>
__device__ __forceinline__ void write_sorted_keys(int32_t* oi_row, float* os_row, int k,
                                                  const uint64_t (&x)[1 << LE], int n, int lane) {
    constexpr int EPL = 1 << LE;
    int32_t* oi = oi_row + EPL * lane;
    float* os = os_row + EPL * lane;
    if (EPL * lane + EPL <= k && (k & 3) == 0) {
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
            int32_t vi[4];
            float vs[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool real = EPL * lane + e + j < n;
                vi[j] = real ? key_index(x[e + j]) : -1;
                vs[j] = real ? key_score(x[e + j]) : -__builtin_inff();
            }
            *reinterpret_cast<u32x4*>(oi + e) =
                u32x4{(uint32_t)vi[0], (uint32_t)vi[1], (uint32_t)vi[2], (uint32_t)vi[3]};
            *reinterpret_cast<u32x4*>(os + e) =
                u32x4{__float_as_uint(vs[0]), __float_as_uint(vs[1]), __float_as_uint(vs[2]),
                      __float_as_uint(vs[3])};
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            if (EPL * lane + e < k) {
                const bool real = EPL * lane + e < n;
                oi[e] = real ? key_index(x[e]) : -1;
                os[e] = real ? key_score(x[e]) : -__builtin_inff();
            }
        }
    }
}

}  // namespace si
