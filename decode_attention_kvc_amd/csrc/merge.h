// Merge of the split-K partials of a decode attention launch, shared by the
// bf16 and int8 kernels: by a merge kernel, or by the last workgroup of each
// slab to finish (COH).
//
// A work item is (query row, 8 channels).  With at most four splits a thread
// folds all of an item's splits with running log-sum-exp weights (all of its
// reads issued together).  With more, SG threads share an item when the slab
// has fewer items than threads, each folding every SG-th split with running
// weights (one pass of independent reads); the split groups' (max, sum, acc)
// meet once in LDS, rescaled to the largest maximum and added in a fixed
// order.
#pragma once
#include "common.h"
#include "kvc_internal.h"

namespace kvc {

constexpr float MERGE_LOG2E = 1.4426950408889634f;

// Partial stores and loads of the launches whose last workgroup per slab
// merges (COH): buffer accesses with the agent-scope cache policy (sc1),
// written through to and read from the device's coherence point.
constexpr int CPOL_SC1 = 16;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const float* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0x7fffffff, 0x00020000);
}

template <bool COH>
__device__ __forceinline__ f32x4 ld_part4(const float* a, __amdgpu_buffer_rsrc_t r,
                                          const float* base) {
    if constexpr (COH) {
        const int off = (int)((a - base) * 4);
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL_SC1));
    } else {
        return *reinterpret_cast<const f32x4*>(a);
    }
}

template <bool COH>
__device__ __forceinline__ void ld_ml(const float* a, __amdgpu_buffer_rsrc_t r, const float* base,
                                      float& m, float& l) {
    if constexpr (COH) {
        // two word loads (the compiler pairs them into one 8-byte load)
        const int off = (int)((a - base) * 4);
        m = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CPOL_SC1));
        l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off + 4, 0, CPOL_SC1));
    } else {
        m = a[0];
        l = a[1];
    }
}

template <int NTH, bool COH>
__device__ void combine_rows(const AttnLaunch& p, int j, int b, int r0, int rpb, float* red) {
    const int tid = threadIdx.x;
    const int slab = b * p.hkv + j;
    const int nsplit = p.nsplit, rp = p.rp;
    const size_t slabs = (size_t)p.nb * p.hkv;
    const float* acc = p.part + (size_t)slab * nsplit * rp * D;
    const float* ml = p.part + slabs * nsplit * rp * D + (size_t)slab * nsplit * rp * 2;
    const __amdgpu_buffer_rsrc_t rsrc = part_rsrc(p.part);
    const int items = min(rpb, p.rows - r0) * (D / 8);
    if (items <= 0) return;
    if (nsplit <= 4) {
        for (int idx = tid; idx < items; idx += NTH) {
            const int r = r0 + idx / (D / 8), d0 = (idx % (D / 8)) * 8;
            float M = -INFINITY, L = 0.f, o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll 4
            for (int sp = 0; sp < nsplit; ++sp) {
                float ms, ls;
                ld_ml<COH>(ml + ((size_t)sp * rp + r) * 2, rsrc, p.part, ms, ls);
                const float* a = acc + ((size_t)sp * rp + r) * D + d0;
                const f32x4 a0 = ld_part4<COH>(a, rsrc, p.part);
                const f32x4 a1 = ld_part4<COH>(a + 4, rsrc, p.part);
                // Branch-free, so that the loads of every unrolled split
                // are issued together: a split with no visible row (its
                // accumulators unwritten) is passed over by selects.
                const bool live = ms != -INFINITY;
                const float mn = fmaxf(M, ms);
                const float fo = exp2f((M - mn) * MERGE_LOG2E);   // 0 on the first live split
                const float fs = exp2f((ms - mn) * MERGE_LOG2E);
                L = live ? L * fo + ls * fs : L;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[e] = live ? o[e] * fo + a0[e] * fs : o[e];
                    o[4 + e] = live ? o[4 + e] * fo + a1[e] * fs : o[4 + e];
                }
                M = live ? mn : M;
            }
            const float inv = L > 0.f ? 1.f / L : 0.f;   // no split saw a row: zeros
            const int qi = r / p.g, h = j * p.g + r % p.g;
            float* dst = p.out + p.out_off[qi] + ((size_t)b * p.hq + h) * D + d0;
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[e] = o[e] * inv;
            if (d0 == 0 && p.lse)
                p.lse[p.lse_off[qi] + (size_t)b * p.hq + h] = L > 0.f ? M + logf(L) : -INFINITY;
        }
        return;
    }
    const int SG = max(1, min(nsplit, NTH / items));    // split groups per item
    const int per = SG == 1 ? NTH : items;              // items per block pass
    for (int i0 = 0; i0 < items; i0 += per) {
        const int sg = tid / per, item = i0 + tid % per;
        const bool act = sg < SG && item < items;
        const int r = act ? r0 + item / (D / 8) : 0, d0 = act ? (item % (D / 8)) * 8 : 0;
        // This thread's splits (every SG-th), folded with running weights;
        // the loads of four splits are issued together.
        float M = -INFINITY, L = 0.f, o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
        if (act) {
#pragma unroll 8
            for (int sp = sg; sp < nsplit; sp += SG) {
                float ms, ls;
                ld_ml<COH>(ml + ((size_t)sp * rp + r) * 2, rsrc, p.part, ms, ls);
                const float* a = acc + ((size_t)sp * rp + r) * D + d0;
                const f32x4 a0 = ld_part4<COH>(a, rsrc, p.part);
                const f32x4 a1 = ld_part4<COH>(a + 4, rsrc, p.part);
                // Branch-free, so that the loads of every unrolled split
                // are issued together: a split with no visible row (its
                // accumulators unwritten) is passed over by selects.
                const bool live = ms != -INFINITY;
                const float mn = fmaxf(M, ms);
                const float fo = exp2f((M - mn) * MERGE_LOG2E);   // 0 on the first live split
                const float fs = exp2f((ms - mn) * MERGE_LOG2E);
                L = live ? L * fo + ls * fs : L;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[e] = live ? o[e] * fo + a0[e] * fs : o[e];
                    o[4 + e] = live ? o[4 + e] * fo + a1[e] * fs : o[4 + e];
                }
                M = live ? mn : M;
            }
        }
        if (SG > 1) {
            // The split groups of an item meet in LDS once: group 0 rescales
            // every group's sums to the largest maximum and adds them in
            // group order.
#pragma unroll
            for (int e = 0; e < 8; ++e) red[tid * 10 + e] = o[e];
            red[tid * 10 + 8] = L;
            red[tid * 10 + 9] = M;
            __syncthreads();
            if (act && sg == 0) {
                float Mx = M;
                for (int s2 = 1; s2 < SG; ++s2) Mx = fmaxf(Mx, red[(s2 * per + tid % per) * 10 + 9]);
                if (Mx != -INFINITY) {
                    const float f0 = exp2f((M - Mx) * MERGE_LOG2E);
                    L *= f0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] *= f0;
                    for (int s2 = 1; s2 < SG; ++s2) {
                        const float* q2 = red + (s2 * per + tid % per) * 10;
                        const float f = exp2f((q2[9] - Mx) * MERGE_LOG2E);   // empty group: 0
#pragma unroll
                        for (int e = 0; e < 8; ++e) o[e] = fmaf(f, q2[e], o[e]);
                        L = fmaf(f, q2[8], L);
                    }
                }
                M = Mx;
            }
            __syncthreads();
        }
        if (act && sg == 0) {
            const float inv = L > 0.f ? 1.f / L : 0.f;   // no split saw a row: zeros
            const int qi = r / p.g, h = j * p.g + r % p.g;
            float* dst = p.out + p.out_off[qi] + ((size_t)b * p.hq + h) * D + d0;
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[e] = o[e] * inv;
            if (d0 == 0 && p.lse)
                p.lse[p.lse_off[qi] + (size_t)b * p.hq + h] = L > 0.f ? M + logf(L) : -INFINITY;
        }
    }
}

// Counted arrival of a workgroup whose partial is written; true in the last
// workgroup of the slab to arrive, which then merges every partial.  The
// partial stores are complete (vmcnt 0) before the workgroup counts itself
// in, and the last workgroup reads them with agent-scope loads: no L2
// writeback or invalidation is needed, since no partial passes through a
// non-coherent cache line.  The last workgroup returns the counter to zero
// for the next launch on the workspace.
__device__ __forceinline__ bool arrive_last(unsigned* ctr, int nsplit) {
    __shared__ int last;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned old =
            __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = old == (unsigned)nsplit - 1;
        if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return last;
}

// A workgroup's partial rows of a launch whose last workgroup merges: the
// accumulators (EPT floats from channel d0) and the (max, sum) pair of row r,
// written through to the coherence point.
template <int EPT>
__device__ __forceinline__ void store_part_coh(const AttnLaunch& p, float* part_acc,
                                               float* part_ml, int r, int d0, const float* o,
                                               float M, float L) {
    const __amdgpu_buffer_rsrc_t rs = part_rsrc(p.part);
    const int off = (int)((part_acc + (size_t)r * D + d0 - p.part) * 4);
#pragma unroll
    for (int e = 0; e < EPT; e += 4)
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]}), rs, off + 4 * e, 0,
            CPOL_SC1);
    if (d0 == 0)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, f32x2{M, L}), rs,
                                              (int)((part_ml + r * 2 - p.part) * 4), 0, CPOL_SC1);
}

}  // namespace kvc
