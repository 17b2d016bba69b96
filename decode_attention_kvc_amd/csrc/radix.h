// Block-wide exact k-selection on 32-bit keys and ordered flag scans, for a
// workgroup of NT threads (a multiple of the 64-wide wave).
//
// radix_select finds the k-th smallest key with four passes of 8-bit digits
// (LDS histograms, most significant digit first); rows equal to that key
// are taken in ascending row order, so "the k smallest, ties to the lower
// row" is decided exactly.  block_scan_flag gives each thread the number of
// set flags before it in thread order.  Every thread of the workgroup must
// call both (they contain barriers).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace kvc {

template <int NT>
struct RadixSmem {
    uint32_t hist[256];
    uint32_t wave_tot[NT / WAVE];
    uint32_t bcast[4];
};

// Exclusive prefix count of `flag` over the block in thread order; returns
// this thread's offset and writes the block total to *total.
template <int NT>
__device__ __forceinline__ uint32_t block_scan_flag(bool flag, RadixSmem<NT>& sm,
                                                    uint32_t* total) {
    constexpr int NWV = NT / WAVE;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const unsigned long long bal = __ballot(flag);
    const uint32_t before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) sm.wave_tot[wave] = __popcll(bal);
    __syncthreads();
    uint32_t off = 0, tot = 0;
    for (int w = 0; w < NWV; ++w) {
        const uint32_t c = sm.wave_tot[w];
        off += (w < wave) ? c : 0u;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return off + before;
}

// Exclusive prefix sum of v over the block in thread order; returns this
// thread's offset and writes the block total to *total.
template <int NT>
__device__ __forceinline__ uint32_t block_scan_u32(uint32_t v, RadixSmem<NT>& sm, uint32_t* total) {
    constexpr int NWV = NT / WAVE;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == WAVE - 1) sm.wave_tot[wave] = incl;
    __syncthreads();
    uint32_t off = 0, tot = 0;
    for (int w = 0; w < NWV; ++w) {
        const uint32_t c = sm.wave_tot[w];
        off += (w < wave) ? c : 0u;
        tot += c;
    }
    __syncthreads();
    *total = tot;
    return off + incl - v;
}

// k-th smallest (1-based) of key(t), t < n.  Returns the key; *take gets how
// many rows equal to it belong to the k smallest (lowest rows first).
template <int NT, typename KeyFn>
__device__ uint32_t radix_select(int n, uint32_t k, KeyFn key, RadixSmem<NT>& sm, uint32_t* take) {
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += NT) sm.hist[i] = 0;
        __syncthreads();
        for (int t = tid; t < n; t += NT) {
            const uint32_t u = key(t);
            if ((u & mask) == prefix) atomicAdd(&sm.hist[(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < WAVE) {
            // lane owns bins 4*lane .. 4*lane+3
            uint32_t c[4], s = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                c[e] = sm.hist[4 * tid + e];
                s += c[e];
            }
            // inclusive scan of s across the wave
            uint32_t incl = s;
#pragma unroll
            for (int o = 1; o < WAVE; o <<= 1) {
                const uint32_t y = __shfl_up(incl, o);
                if (tid >= o) incl += y;
            }
            uint32_t run = incl - s;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (run < k && k <= run + c[e]) {
                    sm.bcast[0] = 4 * tid + e;
                    sm.bcast[1] = run;
                }
                run += c[e];
            }
        }
        __syncthreads();
        const uint32_t bin = sm.bcast[0], below = sm.bcast[1];
        __syncthreads();
        k -= below;
        prefix |= bin << shift;
        mask |= 255u << shift;
    }
    *take = k;
    return prefix;
}

}  // namespace kvc
