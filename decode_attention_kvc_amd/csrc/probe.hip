// Read-bandwidth probe: streams a device buffer once with the access
// pattern of the decode attention kernel, without its arithmetic, and folds
// the words into a checksum.  It measures the read rate that this part
// sustains for a pure stream, the ceiling against which the HBM-bound
// kernels' rate is judged (the 8 TB/s of the data sheet is the interface's
// peak, not a rate any kernel reaches).
//
// Pattern: PROBE_BLOCKS workgroups of four waves, one contiguous range of
// the buffer each (the decode attention's launch shape); the waves take the
// range's 32 KB tiles round-robin (32 16-byte non-temporal loads per lane)
// with two tiles in flight per wave.  A range's ragged end is read one
// 16-byte word per lane.  Measured over 4 GiB: 7.1 TB/s with this shape,
// 6.9-7.1 TB/s for 256 to 2048 workgroups of 2 to 16 waves with 8 to 32
// loads per lane and tile, 5.6 TB/s for a grid-stride loop of single 16-byte
// loads; over 2 GiB the launch's start and drain take ~7% more per byte.
#include "common.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int PROBE_WAVES = 4;
constexpr int PROBE_THREADS = PROBE_WAVES * WAVE;
constexpr int TILE_LOADS = 32;                  // 16-byte loads per lane and tile
constexpr int TILE_WORDS = TILE_LOADS * WAVE;   // 16-byte words per tile (32 KB)

struct ProbeTile {
    u32x4 v[TILE_LOADS];
};

__device__ __forceinline__ void probe_load(ProbeTile& t, const u32x4* p, int lane) {
#pragma unroll
    for (int u = 0; u < TILE_LOADS; ++u) t.v[u] = __builtin_nontemporal_load(p + u * WAVE + lane);
}

__device__ __forceinline__ uint32_t probe_fold(const ProbeTile& t) {
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < TILE_LOADS; ++u) x ^= t.v[u][0] ^ t.v[u][1] ^ t.v[u][2] ^ t.v[u][3];
    return x;
}

__global__ __launch_bounds__(PROBE_THREADS) void read_probe_kernel(const u32x4* buf, size_t n16,
                                                                   uint32_t* out) {
    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    // this workgroup's range [r0, r1) of 16-byte words, whole tiles first
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t r0 = min(n16, (size_t)blockIdx.x * per), r1 = min(n16, r0 + per);
    const size_t ntile = (r1 - r0) / TILE_WORDS;
    const u32x4* base = buf + r0;
    uint32_t acc = 0;
    // tiles wave, wave + 4, ...: two in flight (the next tile's loads are
    // issued before the current one is folded)
    const size_t n = (size_t)wave < ntile ? (ntile - wave + PROBE_WAVES - 1) / PROBE_WAVES : 0;
    if (n > 0) {
        ProbeTile A, B;
        auto at = [&](size_t k) { return base + (wave + k * PROBE_WAVES) * TILE_WORDS; };
        probe_load(A, at(0), lane);
        size_t k = 0;
        for (; k + 2 < n; k += 2) {
            probe_load(B, at(k + 1), lane);
            acc ^= probe_fold(A);
            probe_load(A, at(k + 2), lane);
            acc ^= probe_fold(B);
        }
        if (k + 1 < n) {
            probe_load(B, at(k + 1), lane);
            acc ^= probe_fold(A);
            acc ^= probe_fold(B);
        } else {
            acc ^= probe_fold(A);
        }
    }
    for (size_t i = r0 + ntile * TILE_WORDS + threadIdx.x; i < r1; i += PROBE_THREADS) {
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    // workgroup XOR: across each wave by shuffles, then the waves in LDS
    for (int m = 1; m < WAVE; m <<= 1) acc ^= __shfl_xor(acc, m);
    __shared__ uint32_t wx[PROBE_WAVES];
    if (lane == 0) wx[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (int w = 0; w < PROBE_WAVES; ++w) x ^= wx[w];
        out[blockIdx.x] = x;
    }
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t st) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(PROBE_BLOCKS), dim3(PROBE_THREADS), 0, st,
                       static_cast<const u32x4*>(buf), bytes / 16, out);
    return hipGetLastError();
}

}  // namespace kvc
