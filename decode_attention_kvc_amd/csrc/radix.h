// Block-wide exact k-selection on 32-bit keys and ordered flag scans, for a
// workgroup of NT threads (a multiple of the 64-wide wave).
//
// radix_select finds the k-th smallest key with four passes of 8-bit digits
// (LDS histograms, most significant digit first); rows equal to that key
// are taken in ascending row order, so "the k smallest, ties to the lower
// row" is decided exactly.  Keys that share their leading digit (floats of
// one magnitude) all land in a few bins, and LDS atomics on one address are
// serialised, so the histogram can be held in NC copies (lane l counts in
// copy l % NC; copies are padded so that one bin of two copies sits in two
// banks), which divides that serialisation by NC.  block_scan_flag gives
// each thread the number of set flags before it in thread order.  Every
// thread of the workgroup must call both (they contain barriers).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace kvc {

template <int NT, int NC = 1>
struct RadixSmem {
    static constexpr int PITCH = NC == 1 ? 256 : 257;
    uint32_t hist[NC * PITCH];
    uint32_t wave_tot[NT / WAVE];
    uint32_t bcast[4];
};

// Exclusive prefix count of `flag` over the block in thread order; returns
// this thread's offset and writes the block total to *total.
template <int NT, int NC>
__device__ __forceinline__ uint32_t block_scan_flag(bool flag, RadixSmem<NT, NC>& sm,
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
template <int NT, int NC>
__device__ __forceinline__ uint32_t block_scan_u32(uint32_t v, RadixSmem<NT, NC>& sm,
                                                   uint32_t* total) {
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
template <int NT, int NC, typename KeyFn>
__device__ uint32_t radix_select(int n, uint32_t k, KeyFn key, RadixSmem<NT, NC>& sm,
                                 uint32_t* take) {
    constexpr int PITCH = RadixSmem<NT, NC>::PITCH;
    const int tid = threadIdx.x;
    uint32_t* hist = sm.hist + (tid % NC) * PITCH;
    uint32_t prefix = 0, mask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < NC * PITCH; i += NT) sm.hist[i] = 0;
        __syncthreads();
        for (int t = tid; t < n; t += NT) {
            const uint32_t u = key(t);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < WAVE) {
            // lane owns bins 4*lane .. 4*lane+3 (summed over the copies)
            uint32_t c[4], s = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                c[e] = 0;
#pragma unroll
                for (int cp = 0; cp < NC; ++cp) c[e] += sm.hist[cp * PITCH + 4 * tid + e];
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
