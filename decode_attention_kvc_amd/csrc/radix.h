// Block-wide exact k-selection on 32-bit keys and ordered flag scans, for a
// workgroup of NT threads (a multiple of the 64-wide wave).
//
// radix_select finds the k smallest keys with passes of 8-bit digits (LDS
// histograms, most significant digit first, the first one counted by the
// caller while it stores the keys), stopping as soon as the bin that holds
// the k-th key is taken whole; rows tied in the last bin are taken in
// ascending row order, so "the k smallest, ties to the lower row" is decided
// exactly.  Keys that share their leading digit (floats of
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

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (plain
// VALU work, no LDS round trip): shifts by 1, 2, 4, 8 inside each 16-lane
// row, then the last lane of row 0 into rows 1 and 3 and the last lane of
// row 1 into rows 2 and 3.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += dpp_u32<0x111, 0xF>(v);   // row_shr:1
    v += dpp_u32<0x112, 0xF>(v);   // row_shr:2
    v += dpp_u32<0x114, 0xF>(v);   // row_shr:4
    v += dpp_u32<0x118, 0xF>(v);   // row_shr:8
    v += dpp_u32<0x142, 0xA>(v);   // row_bcast:15
    v += dpp_u32<0x143, 0xC>(v);   // row_bcast:31
    return v;
}

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
    const uint32_t incl = wave_incl_scan(v);
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

// The k smallest (1-based k) of key(t), t < n, ties to the lower row, as a
// masked prefix: key u is among them when (u & mask) < prefix, or when
// (u & mask) == prefix and it is among the first *take such rows in row
// order (*cnt such rows exist; take == cnt keeps them all).  The caller has
// counted every key's top 8 bits into sm.hist (copy tid % NC) and
// synchronised; further 8-bit digits are counted here only while the bin
// holding the k-th key is not kept whole, so keys of spread magnitudes
// resolve in one or two passes instead of four.  Returns the prefix.
template <int NT, int NC, typename KeyFn>
__device__ uint32_t radix_select(int n, uint32_t k, KeyFn key, RadixSmem<NT, NC>& sm,
                                 uint32_t* mask_out, uint32_t* take, uint32_t* cnt_out) {
    constexpr int PITCH = RadixSmem<NT, NC>::PITCH;
    const int tid = threadIdx.x;
    uint32_t* hist = sm.hist + (tid % NC) * PITCH;
    uint32_t prefix = 0, mask = 0, cnt = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (shift != 24) {
            // the previous scan read the histogram before the last barrier
            for (int i = tid; i < NC * PITCH; i += NT) sm.hist[i] = 0;
            __syncthreads();
#pragma unroll 4
            for (int t = tid; t < n; t += NT) {
                const uint32_t u = key(t);
                if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
            }
            __syncthreads();
        }
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
            const uint32_t incl = wave_incl_scan(s);
            uint32_t run = incl - s;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (run < k && k <= run + c[e]) {
                    sm.bcast[0] = 4 * tid + e;
                    sm.bcast[1] = run;
                    sm.bcast[2] = c[e];
                }
                run += c[e];
            }
        }
        __syncthreads();
        const uint32_t bin = sm.bcast[0], below = sm.bcast[1];
        cnt = sm.bcast[2];
        k -= below;
        prefix |= bin << shift;
        mask |= 255u << shift;
        // bcast is written again only after two more barriers
        if (cnt == k) break;
    }
    *mask_out = mask;
    *take = k;
    *cnt_out = cnt;
    return prefix;
}

}  // namespace kvc
