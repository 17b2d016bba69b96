// Compaction of the surviving KV rows of one slot into another cache.
//
// VASE summary (gist.science 2606.03928), §1: eviction discards the dropped
// key/value pairs for good, which is what gives the cache its fixed
// footprint.  dst row i <- src row kept[i] for every slab of the slot, K in
// [t][d] rows and V in 32-token channel-major tiles, out of place.
//
// One workgroup (256 threads) per 256 kept rows of a slab.  K rows are
// copied with 16-byte accesses, 16 (bf16) or 32 (fp32) lanes per row.  For V
// each thread owns one kept row and walks the 128 channels; the source
// indices are ascending, so a wave's reads of one channel fall in a few
// tiles.  An index outside [0, src t_len) produces a zero row instead
// of an out-of-bounds read.
#include "common.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int CROWS = 256;

template <typename E>
__global__ __launch_bounds__(256) void compact_kernel(CompactLaunch p) {
    constexpr int VEC = 16 / sizeof(E);     // elements per 16-byte access
    constexpr int CPR = D / VEC;            // 16-byte chunks per K row
    const int slab = blockIdx.z * p.hkv + blockIdx.y;
    const int i0 = blockIdx.x * CROWS;
    const int tid = threadIdx.x;
    const int32_t* kept = p.kept + (size_t)slab * p.n_keep;
    const E* sk = reinterpret_cast<const E*>(p.sk) + (size_t)slab * p.src_t_cap * D;
    const E* sv = reinterpret_cast<const E*>(p.sv) + (size_t)slab * p.src_t_cap * D;
    E* dk = reinterpret_cast<E*>(p.dk) + (size_t)slab * p.dst_t_cap * D;
    E* dv = reinterpret_cast<E*>(p.dv) + (size_t)slab * p.dst_t_cap * D;
    const int rows = min(CROWS, p.n_keep - i0);

    __shared__ int32_t src_row[CROWS];
    for (int x = tid; x < rows; x += blockDim.x) {
        const int32_t r = kept[i0 + x];
        src_row[x] = (r >= 0 && r < p.src_t_len) ? r : -1;
    }
    __syncthreads();

    // K rows
    for (int x = tid; x < rows * CPR; x += blockDim.x) {
        const int i = x / CPR, c = x % CPR;
        const int32_t r = src_row[i];
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (r >= 0) v = load_stream16(sk + (size_t)r * D + c * VEC);
        *reinterpret_cast<u32x4*>(dk + (size_t)(i0 + i) * D + c * VEC) = v;
    }
    // V columns
    if (tid < rows) {
        const int32_t r = src_row[tid];
        for (int d = 0; d < D; ++d) {
            E v = E(0);
            if (r >= 0) v = sv[vt_off(r, d)];
            dv[vt_off(i0 + tid, d)] = v;
        }
    }
}

}  // namespace

hipError_t launch_compact(const CompactLaunch& p, hipStream_t st) {
    const dim3 grid((p.n_keep + CROWS - 1) / CROWS, p.hkv, p.nb);
    if (p.elem == 4)
        hipLaunchKernelGGL(compact_kernel<float>, grid, dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL(compact_kernel<uint16_t>, grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace kvc
