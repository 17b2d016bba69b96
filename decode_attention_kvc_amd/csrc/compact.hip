// Compaction of the surviving KV rows of one slot into another cache.
//
// VASE summary (gist.science 2606.03928), §1: eviction discards the dropped
// key/value pairs for good, which is what gives the cache its fixed
// footprint.  dst row i <- src row kept[i] for every slab of the slot, K in
// [t][d] rows and V in 32-token channel-major tiles, out of place.
//
// One workgroup (256 threads) per 64 kept rows of a slab.
//  * K rows are copied with 16-byte accesses (16 lanes per bf16 row).
//  * V: the destination rows are taken in rounds of whole destination tiles.
//    A round covers as many destination tiles as keep the source rows they
//    need within the three staged source tiles; those source tiles are
//    loaded into LDS with coalesced 16-byte loads, and each (destination
//    tile, channel, 8-row group) is assembled from LDS and written with one
//    16-byte store.  With the kept rows ascending and dense (a steady-state
//    eviction keeps ~98% of the rows) the workgroup's two destination tiles
//    come from at most three source tiles: one round, its loads issued with
//    the K loads; sparse selections (a long prompt compressed 4x) take one
//    round per destination tile.  The small staging area (30 KB for bf16)
//    lets five workgroups share a CU, which is what keeps enough loads in
//    flight: 64-row workgroups with 31 KB of staging ran the steady pass in
//    230 us per Llama-3.1-8B-shaped slot, against 296 us for 256-row
//    workgroups with 62 KB (two per CU) and 287 us for 64 rows with 42 KB.
// Indices outside [0, src t_len) give zero rows; a row whose source tile is
// not staged (only possible for indices out of ascending order) is read
// straight from global memory, so no input can make an access leave the
// slab.
// Ragged batches: sequence b is read from source entry phys_src(b) and
// written to destination entry phys_dst(b); it keeps min(T_b, n_keep) rows
// (n_keep is the stride of `kept`), and indices at or past T_b give zero
// rows.
#include "common.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

constexpr int CROWS = 64;                 // destination rows per workgroup

template <typename E>
struct Stage {
    static constexpr int VEC = 16 / sizeof(E);         // elements per 16 bytes
    static constexpr int PITCH = VT + VEC;             // padded channel row (16-byte aligned)
    static constexpr int TILE = D * PITCH;             // elements per staged tile
    static constexpr int NT = 3;                       // staged source tiles
};

template <typename E>
__global__ __launch_bounds__(256) void compact_kernel(CompactLaunch p) {
    using S = Stage<E>;
    constexpr int VEC = S::VEC;
    constexpr int CPR = D / VEC;            // 16-byte chunks per K row
    // Contiguous runs of (row block, head, batch) blocks per XCD:
    // neighbouring row blocks of a slab share a boundary source tile of V,
    // and on one XCD its second read finds the tile in that XCD's L2.
    const BlockXYZ blk = xcd_run_block(true);
    const int bx = blk.x, by = blk.y, b = blk.z;
    const int slab = b * p.hkv + by;
    const int i0 = bx * CROWS;
    const int tid = threadIdx.x;
    const int sphys = seq_phys(p.src_sm, b), dphys = seq_phys(p.dst_sm, b);
    const int src_t_len = seq_rows(p.src_sm, b, sphys);
    const int rows = min(CROWS, min(src_t_len, p.n_keep) - i0);
    if (dphys < 0 || rows <= 0) return;          // whole workgroup
    const int32_t* kept = p.kept ? p.kept + (size_t)slab * p.n_keep : nullptr;
    const size_t scs = (size_t)sphys * p.hkv + by, dcs = (size_t)dphys * p.hkv + by;
    const E* sk = reinterpret_cast<const E*>(p.sk) + scs * p.src_t_cap * D;
    const E* sv = reinterpret_cast<const E*>(p.sv) + scs * p.src_t_cap * D;
    E* dk = reinterpret_cast<E*>(p.dk) + dcs * p.dst_t_cap * D;
    E* dv = reinterpret_cast<E*>(p.dv) + dcs * p.dst_t_cap * D;
    const int src_tiles = (src_t_len + VT - 1) / VT;

    __shared__ int32_t src_row[CROWS];
    __shared__ __align__(16) E stage[S::NT * S::TILE];
    for (int x = tid; x < CROWS; x += blockDim.x) {
        int32_t r = -1;
        if (x < rows) {
            r = kept ? kept[i0 + x] : i0 + x;
            if (r < 0 || r >= src_t_len) r = -1;
        }
        src_row[x] = r;
    }
    __syncthreads();

    // V rounds: every thread derives the same round boundaries from
    // src_row, so the loop and its barriers are uniform across the
    // workgroup.
    const int ntile = (rows + VT - 1) / VT;
    auto first_tile = [&](int a, int b) {       // source tile of the first valid row in [a, b)
        for (int x = a; x < b; ++x)
            if (src_row[x] >= 0) return src_row[x] / VT;
        return -1;
    };
    auto last_tile = [&](int a, int b) {
        for (int x = b - 1; x >= a; --x)
            if (src_row[x] >= 0) return src_row[x] / VT;
        return -1;
    };
    // Round starting at destination tile k: staged source tiles [lo, lo+n_st)
    // serve destination tiles [k, k_end).
    auto plan_round = [&](int k, int& lo, int& n_st, int& k_end) {
        lo = first_tile(k * VT, min(rows, (k + 1) * VT));
        int hi = last_tile(k * VT, min(rows, (k + 1) * VT));
        k_end = k + 1;
        if (lo >= 0) {
            while (k_end < ntile) {
                const int h2 = last_tile(k_end * VT, min(rows, (k_end + 1) * VT));
                if (h2 >= 0 && h2 - lo + 1 > S::NT) break;
                if (h2 > hi) hi = h2;
                ++k_end;
            }
        }
        n_st = (lo >= 0 && hi >= lo) ? min(hi - lo + 1, S::NT) : 0;
    };
    constexpr int CH_PER_TILE = D * VT / VEC;          // 16-byte chunks per source tile
    constexpr int SLOADS = (S::NT * CH_PER_TILE + 255) / 256;   // staging loads per thread
    auto stage_load = [&](int lo, int n_st, u32x4* reg) {
#pragma unroll
        for (int u = 0; u < SLOADS; ++u) {
            const int x = tid + 256 * u;
            const int tl = x / CH_PER_TILE, c = x % CH_PER_TILE;
            const int d = c / (VT / VEC), q = c % (VT / VEC);
            if (tl < n_st && lo + tl < src_tiles)
                reg[u] = load_stream16(sv + (size_t)(lo + tl) * D * VT + d * VT + q * VEC);
        }
    };
    auto stage_store = [&](int lo, int n_st, const u32x4* reg) {
#pragma unroll
        for (int u = 0; u < SLOADS; ++u) {
            const int x = tid + 256 * u;
            const int tl = x / CH_PER_TILE, c = x % CH_PER_TILE;
            const int d = c / (VT / VEC), q = c % (VT / VEC);
            if (tl < n_st && lo + tl < src_tiles)
                *reinterpret_cast<u32x4*>(&stage[tl * S::TILE + d * S::PITCH + q * VEC]) = reg[u];
        }
    };

    // K rows and the first V round's staging loads are all issued before
    // any of them is used: one memory round trip for the common case.
    constexpr int KLOADS = CROWS * CPR / 256;           // K chunks per thread
    u32x4 kreg[KLOADS];
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
        const int x = tid + 256 * u;
        const int i = x / CPR, c = x % CPR;
        const int32_t r = i < rows ? src_row[i] : -1;
        kreg[u] = u32x4{0u, 0u, 0u, 0u};
        if (r >= 0) kreg[u] = load_stream16(sk + (size_t)r * D + c * VEC);
    }
    int lo, n_st, k_end;
    plan_round(0, lo, n_st, k_end);
    u32x4 sreg[SLOADS];
    stage_load(lo, n_st, sreg);
#pragma unroll
    for (int u = 0; u < KLOADS; ++u) {
        const int x = tid + 256 * u;
        const int i = x / CPR, c = x % CPR;
        if (i < rows) *reinterpret_cast<u32x4*>(dk + (size_t)(i0 + i) * D + c * VEC) = kreg[u];
    }

    int k = 0;
    while (k < ntile) {
        if (k > 0) {
            plan_round(k, lo, n_st, k_end);
            stage_load(lo, n_st, sreg);
        }
        stage_store(lo, n_st, sreg);
        __syncthreads();
        // assemble destination tiles [k, k_end)
        constexpr int GROUPS = VT / VEC;                // 16-byte groups per channel row
        const int items = (k_end - k) * D * GROUPS;
        for (int x = tid; x < items; x += blockDim.x) {
            const int q = x % GROUPS, d = (x / GROUPS) % D, kk = k + x / (GROUPS * D);
            const int base = kk * VT + q * VEC;         // first destination row of the group
            union {
                E e[VEC];
                u32x4 v;
            } vals;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int i = base + e;
                E v = E(0);
                if (i < rows) {
                    const int32_t r = src_row[i];
                    if (r >= 0) {
                        const int tl = r / VT - lo;
                        if (tl >= 0 && tl < n_st) v = stage[tl * S::TILE + d * S::PITCH + (r % VT)];
                        else v = sv[vt_off(r, d)];
                    }
                }
                vals.e[e] = v;
            }
            const int di = i0 + base;                   // destination row of vals.e[0]
            if (base + VEC <= rows) {
                *reinterpret_cast<u32x4*>(dv + vt_off(di, d)) = vals.v;
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e)
                    if (base + e < rows) dv[vt_off(di + e, d)] = vals.e[e];
            }
        }
        __syncthreads();
        k = k_end;
    }
}

// Compaction from a source whose values are [t][D] rows (a prefill's
// layout) into the tiled layout.  A workgroup gathers its 64 kept rows of K
// and of V with 16-byte loads (only the kept rows are read: no source tile is
// fetched whole), writes the K rows, stages the V rows in LDS and writes
// them out as the destination's channel-major 32-token tiles with 16-byte
// stores.  Indices outside [0, src t_len) give zero rows, as above.
template <typename E>
__global__ __launch_bounds__(256) void compact_rows_kernel(CompactLaunch p) {
    constexpr int VEC = 16 / sizeof(E);
    constexpr int CPR = D / VEC;                // 16-byte chunks per row
    constexpr int PITCH = D + VEC;              // staged row pitch, 16-byte aligned
    constexpr int LOADS = CROWS * CPR / 256;    // chunks per thread, for K and for V
    const BlockXYZ blk = xcd_run_block(true);
    const int bx = blk.x, by = blk.y, b = blk.z;
    const int slab = b * p.hkv + by;
    const int i0 = bx * CROWS;
    const int tid = threadIdx.x;
    const int sphys = seq_phys(p.src_sm, b), dphys = seq_phys(p.dst_sm, b);
    const int src_t_len = seq_rows(p.src_sm, b, sphys);
    const int rows = min(CROWS, min(src_t_len, p.n_keep) - i0);
    if (dphys < 0 || rows <= 0) return;          // whole workgroup
    const int32_t* kept = p.kept ? p.kept + (size_t)slab * p.n_keep : nullptr;
    const size_t scs = (size_t)sphys * p.hkv + by, dcs = (size_t)dphys * p.hkv + by;
    const E* sk = reinterpret_cast<const E*>(p.sk) + scs * p.src_t_cap * D;
    const E* sv = reinterpret_cast<const E*>(p.sv) + scs * p.src_t_cap * D;
    E* dk = reinterpret_cast<E*>(p.dk) + dcs * p.dst_t_cap * D;
    E* dv = reinterpret_cast<E*>(p.dv) + dcs * p.dst_t_cap * D;

    __shared__ int32_t src_row[CROWS];
    __shared__ __align__(16) E stage[CROWS * PITCH];
    for (int x = tid; x < CROWS; x += blockDim.x) {
        int32_t r = -1;
        if (x < rows) {
            r = kept ? kept[i0 + x] : i0 + x;
            if (r < 0 || r >= src_t_len) r = -1;
        }
        src_row[x] = r;
    }
    __syncthreads();

    // every load of the block in flight at once
    u32x4 kreg[LOADS], vreg[LOADS];
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
        const int x = tid + 256 * u;
        const int i = x / CPR, c = x % CPR;
        const int32_t r = src_row[i];               // -1 past `rows`
        kreg[u] = vreg[u] = u32x4{0u, 0u, 0u, 0u};
        if (r >= 0) {
            kreg[u] = load_stream16(sk + (size_t)r * D + c * VEC);
            vreg[u] = load_stream16(sv + (size_t)r * D + c * VEC);
        }
    }
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
        const int x = tid + 256 * u;
        const int i = x / CPR, c = x % CPR;
        if (i < rows) *reinterpret_cast<u32x4*>(dk + (size_t)(i0 + i) * D + c * VEC) = kreg[u];
        *reinterpret_cast<u32x4*>(&stage[i * PITCH + c * VEC]) = vreg[u];
    }
    __syncthreads();

    // destination tiles: channel d of tile kk holds rows kk*32 .. kk*32+31,
    // written VEC rows per 16-byte store
    constexpr int GROUPS = VT / VEC;
    const int ntile = (rows + VT - 1) / VT;
    const int items = ntile * D * GROUPS;
    for (int x = tid; x < items; x += blockDim.x) {
        const int q = x % GROUPS, d = (x / GROUPS) % D, kk = x / (GROUPS * D);
        const int base = kk * VT + q * VEC;             // first block row of the group
        union {
            E e[VEC];
            u32x4 v;
        } vals;
#pragma unroll
        for (int e = 0; e < VEC; ++e) vals.e[e] = stage[(base + e) * PITCH + d];
        const int di = i0 + base;
        if (base + VEC <= rows) {
            *reinterpret_cast<u32x4*>(dv + vt_off(di, d)) = vals.v;
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if (base + e < rows) dv[vt_off(di + e, d)] = vals.e[e];
        }
    }
}

}  // namespace

hipError_t launch_compact(const CompactLaunch& p, hipStream_t st) {
    const dim3 grid((p.n_keep + CROWS - 1) / CROWS, p.hkv, p.nb);
    if (p.src_rows) {
        if (p.elem == 4)
            hipLaunchKernelGGL(compact_rows_kernel<float>, grid, dim3(256), 0, st, p);
        else
            hipLaunchKernelGGL(compact_rows_kernel<uint16_t>, grid, dim3(256), 0, st, p);
    } else if (p.elem == 4) {
        hipLaunchKernelGGL(compact_kernel<float>, grid, dim3(256), 0, st, p);
    } else {
        hipLaunchKernelGGL(compact_kernel<uint16_t>, grid, dim3(256), 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace kvc
