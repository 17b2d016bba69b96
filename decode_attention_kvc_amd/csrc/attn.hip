// Grouped-query decode attention over leader KV slots (split-K flash decode).
//
// Stochastic KV Routing (aitrends.kr article on R-CLA), inference and
// implementation paragraphs: every layer reads the KV of its nearest earlier
// leader, and only leaders store new rows.  One launch serves every q-layer
// that reads one slot, so a leader's slab streams from HBM once for all of
// its followers when the caller groups them.
//
// Work decomposition: grid (split, kv head, batch).  A workgroup of four
// waves owns one contiguous range of 32-row tiles of one slab; its waves take
// the tiles round-robin.  Per tile a wave
//   * loads 32 K rows ([t][d], 8 KB) and the matching 32-token V tile
//     ([d][32], 8 KB) straight from HBM into VGPRs with 16-byte loads,
//   * forms S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (query rows on the N
//     side, up to 16 per tile-column block),
//   * runs the online softmax in registers (the MFMA output layout puts one
//     query row per lane column, so the row max needs two cross-lane steps),
//   * forms O^T += V^T P^T with the same MFMA, P split into a bf16 high part
//     and a bf16 residual so the product keeps ~16 bits of P.
// The K-row order inside a tile is permuted so that the S^T fragment a lane
// holds is exactly its P^T operand fragment for the V^T product: no data
// movement between the two products.
// The four waves merge through LDS; each workgroup writes one partial
// (m, l, acc) per query row, and each slab's partials are merged with
// log-sum-exp weights into out / lse (merge.h): by the last workgroup of the
// slab to finish when each of its threads folds at most eight splits
// (partials written through to the device's coherence point, an arrival
// count, no cache writeback), else by a second, small kernel.  When a launch
// has one split per slab the workgroup normalises its rows itself.
//
// Ragged batches: sequence b reads rows [0, rows(b)) of cache entry phys(b);
// the launch is planned for the longest sequence and the splits past a
// sequence's end leave at once (an empty partial that the merge skips).  A
// sequence without rows gets a zero output and lse = -inf.
#include <type_traits>

#include "common.h"
#include "kvc_internal.h"
#include "merge.h"

namespace kvc {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float M_FLOOR = -1e30f;      // below any logit of a finite cache

struct TileRegs {
    u32x4 k[2][4];   // K rows: [column block c][d chunk kc]
    u32x4 v[8];      // V^T slices: [d tile]
};

// Cache row that lane (l16) of column block c covers inside a 32-row tile.
// Rows are ordered so that the S^T fragment of lane group lg covers tile
// rows 8*lg .. 8*lg+7.
__device__ __forceinline__ int tile_row(int c, int l16) {
    return 8 * (l16 >> 2) + 4 * c + (l16 & 3);
}

__device__ __forceinline__ void load_tile(TileRegs& R, const uint16_t* kslab,
                                          const uint16_t* vslab, int t0, int l16, int lg,
                                          int append_row, const uint16_t* knew_row) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int t = t0 + tile_row(c, l16);
        const uint16_t* kr = (t == append_row) ? knew_row : kslab + (size_t)t * D;
        kr += 8 * lg;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) R.k[c][kc] = load_stream16(kr + 32 * kc);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
        R.v[dt] = load_stream16(vslab + vt_off(t0, 16 * dt + l16) + 8 * lg);
}

__device__ __forceinline__ bf16x8 as_bf(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Merge kernel: one workgroup per slab (or per block of a slab's rows), the
// folding of merge.h.  Slabs with many splits (few slabs per launch) use 1024
// threads.
template <int NTH>
__global__ __launch_bounds__(NTH) void attn_combine_kernel(AttnLaunch p) {
    __shared__ float red[NTH * 10];
    // blockIdx.z: a block of the slab's query rows (one block unless the
    // launch spreads many-split rows over several workgroups).
    const int rpb = (p.rows + gridDim.z - 1) / gridDim.z;
    combine_rows<NTH, false>(p, blockIdx.x, blockIdx.y, blockIdx.z * rpb, rpb, red);
}


// Row t of cache slab cslab <- the new row of sequence slab `slab`.
template <typename T>
__device__ void write_append_row(const AttnLaunch& p, size_t slab, size_t cslab, int t) {
    const T* kn = reinterpret_cast<const T*>(p.k_new) + slab * D;
    const T* vn = reinterpret_cast<const T*>(p.v_new) + slab * D;
    T* kc = const_cast<T*>(reinterpret_cast<const T*>(p.k)) + cslab * p.t_cap * D;
    T* vc = const_cast<T*>(reinterpret_cast<const T*>(p.v)) + cslab * p.t_cap * D;
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        kc[(size_t)t * D + d] = kn[d];
        vc[vt_off(t, d)] = vn[d];
    }
}

template <int NT, int W, int PF>
__global__ __launch_bounds__(W * 64) void attn_bf16_kernel(AttnLaunch p) {
    constexpr int RP = 16 * NT;
    // Workgroups are dealt to the eight XCDs in turn.  With many splits per
    // slab the launch renumbers them so that each XCD streams a contiguous
    // run of (split, head, batch) blocks: at batch 1, 8 KV heads and 33K
    // rows (32 splits per slab) every XCD then streams one whole slab,
    // measured 2.5% faster per call; launches with few splits per slab were
    // 0.2-0.5% slower with it and keep the plain order.
    // Wave merge, then (in the last workgroup of a slab) the split merge.
    __shared__ float buf[W * 16 * D];
    static_assert(W * 16 * D >= W * 64 * 10, "LDS of the split merge");
    const BlockXYZ blk = xcd_run_block(p.xcd_runs);
    const int s = blk.x, j = blk.y, b = blk.z;
    const int slab = b * p.hkv + j;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int l16 = lane & 15, lg = lane >> 4;
    const int phys = seq_phys(p.sm, b);
    const int T = seq_rows(p.sm, b, phys);
    const int ntiles = (T + ATTN_TILE - 1) / ATTN_TILE;
    const int tile_begin = s * p.tps;
    const int tile_end = min(tile_begin + p.tps, ntiles);
    if (tile_begin >= ntiles) {
        // A split past the sequence's end (the launch is planned for the
        // longest one): an empty partial, or, for a sequence without rows
        // and a single split, its final zero output.
        const size_t slabs = (size_t)p.nb * p.hkv;
        for (int r = tid; r < p.rows; r += blockDim.x) {
            if (p.nsplit == 1) {
                const int qi = r / p.g, h = j * p.g + r % p.g;
                float* dst = p.out + p.out_off[qi] + ((size_t)b * p.hq + h) * D;
                for (int d = 0; d < D; ++d) dst[d] = 0.f;
                if (p.lse) p.lse[p.lse_off[qi] + (size_t)b * p.hq + h] = -INFINITY;
            } else {
                float* ml = p.part + slabs * p.nsplit * RP * D + ((size_t)slab * p.nsplit + s) * RP * 2;
                if (p.arrive) {
                    const auto ml2 = __builtin_bit_cast(u32x2, f32x2{-INFINITY, 0.f});
                    __builtin_amdgcn_raw_buffer_store_b64(ml2, part_rsrc(p.part),
                                                          (int)((ml + r * 2 - p.part) * 4), 0, CPOL_SC1);
                } else {
                    ml[r * 2] = -INFINITY;
                    ml[r * 2 + 1] = 0.f;
                }
            }
        }
        if (p.nsplit > 1 && p.arrive && arrive_last(p.arrive + slab, p.nsplit))
            combine_rows<W * 64, true>(p, j, b, 0, p.rows, buf);
        return;
    }
    const size_t cslab = (size_t)phys * p.hkv + j;

    const uint16_t* kslab = reinterpret_cast<const uint16_t*>(p.k) + cslab * p.t_cap * D;
    const uint16_t* vslab = reinterpret_cast<const uint16_t*>(p.v) + cslab * p.t_cap * D;
    const int append_row = p.append_read ? T - 1 : -1;
    const uint16_t* knew_row =
        p.append_read ? reinterpret_cast<const uint16_t*>(p.k_new) + (size_t)slab * D : kslab;
    const uint16_t* vnew_row =
        p.append_read ? reinterpret_cast<const uint16_t*>(p.v_new) + (size_t)slab * D : kslab;

    // Q^T operand fragments: lane holds query row nt*16 + l16, channels
    // 32*kc + 8*lg .. +8.
    bf16x8 qB[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = nt * 16 + l16;
        if (r < p.rows) {
            const int qi = r / p.g, h = j * p.g + r % p.g;
            const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + p.q_off[qi] +
                                 ((size_t)b * p.hq + h) * D + 8 * lg;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) qB[nt][kc] = as_bf(load16(qp + 32 * kc));
        } else {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) qB[nt][kc] = as_bf(u32x4{0u, 0u, 0u, 0u});
        }
    }

    f32x4 acc[NT][8];
    float m[NT], lsum[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m[nt] = M_FLOOR;      // finite: the first tile's rows always move it
        lsum[nt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float scale = p.scale;

    // One 32-row tile.  TAIL marks the slab's last tile: rows past the end
    // are masked (their K and V bits are arbitrary: P is zeroed and so is V,
    // since 0 * NaN would poison the sum) and the appended row's V comes from
    // v_new.  Interior tiles take no branch at all.
    auto compute = [&](TileRegs& R, int t0, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        if constexpr (TAIL) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const uint16_t vn = vnew_row[16 * dt + l16];
                u16x8 e = __builtin_bit_cast(u16x8, R.v[dt]);
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int t = t0 + 8 * lg + jj;
                    e[jj] = (t == append_row) ? vn : ((t >= T) ? (uint16_t)0 : e[jj]);
                }
                R.v[dt] = __builtin_bit_cast(u32x4, e);
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 S[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                S[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kc = 0; kc < 4; ++kc)
                    S[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(R.k[c][kc]), qB[nt][kc],
                                                                    S[c], 0, 0, 0);
            }
            // S[c][i]: query row nt*16 + l16, cache row t0 + 8*lg + 4*c + i.
            float sv[8];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = S[c][i] * scale;
                    if constexpr (TAIL) x = (t0 + 8 * lg + 4 * c + i >= T) ? -INFINITY : x;
                    sv[4 * c + i] = x;
                }
            float mx = sv[0];
#pragma unroll
            for (int jj = 1; jj < 8; ++jj) mx = fmaxf(mx, sv[jj]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            // The reference maximum moves only when a logit exceeds it by more
            // than 2^8 in p; the accumulators are rescaled only on the
            // (wave-uniform) tiles where some row's reference moved.
            const bool move = (mx - m[nt]) * LOG2E > 8.f;
            const float mnew = move ? mx : m[nt];
            const float alpha = exp2f((m[nt] - mnew) * LOG2E);
            const bool any_move = __ballot(move) != 0;
            m[nt] = mnew;
            float ps = 0.f;
            u16x8 hi, lo;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const float pj = exp2f((sv[jj] - mnew) * LOG2E);
                ps += pj;
                const uint16_t h16 = f32_to_bf16(pj);
                hi[jj] = h16;
                lo[jj] = f32_to_bf16(pj - bf16_to_f32(h16));
            }
            lsum[nt] = lsum[nt] * alpha + ps;
            const bf16x8 pH = __builtin_bit_cast(bf16x8, hi);
            const bf16x8 pL = __builtin_bit_cast(bf16x8, lo);
            if (any_move) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) acc[nt][dt] *= alpha;
            }
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(R.v[dt]), pH,
                                                                       acc[nt][dt], 0, 0, 0);
                acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(R.v[dt]), pL,
                                                                       acc[nt][dt], 0, 0, 0);
            }
        }
    };
    using Interior = std::integral_constant<bool, false>;
    using Last = std::integral_constant<bool, true>;

    // Interior tiles of this split (the slab's last tile is left out), taken
    // round-robin by the waves.
    const int main_end = min(tile_end, ntiles - 1);
    const int n_main = max(0, main_end - tile_begin);
    auto tile_at = [&](int i) { return tile_begin + i; };
    if constexpr (PF == 0) {
        // One tile (16 KB) of loads in flight per wave.
        for (int i = wave; i < n_main; i += W) {
            TileRegs R;
            load_tile(R, kslab, vslab, tile_at(i) * ATTN_TILE, l16, lg, -1, kslab);
            compute(R, tile_at(i) * ATTN_TILE, Interior{});
        }
    } else {
        // Two tiles in flight per wave: the next tile's loads are issued
        // before the current tile is computed.  Inside the loop body every
        // load is unconditional, so the compiler's wait counts only cover
        // the older tile; two named register sets avoid copies.
        const int n = wave < n_main ? (n_main - wave + W - 1) / W : 0;   // tiles of this wave
        auto t0_of = [&](int k) { return tile_at(wave + k * W) * ATTN_TILE; };
        if (n > 0) {
            TileRegs RA, RB;
            load_tile(RA, kslab, vslab, t0_of(0), l16, lg, -1, kslab);
            int k = 0;
            for (; k + 2 < n; k += 2) {
                load_tile(RB, kslab, vslab, t0_of(k + 1), l16, lg, -1, kslab);
                compute(RA, t0_of(k), Interior{});
                load_tile(RA, kslab, vslab, t0_of(k + 2), l16, lg, -1, kslab);
                compute(RB, t0_of(k + 1), Interior{});
            }
            if (k + 1 < n) {
                load_tile(RB, kslab, vslab, t0_of(k + 1), l16, lg, -1, kslab);
                compute(RA, t0_of(k), Interior{});
                compute(RB, t0_of(k + 1), Interior{});
            } else {
                compute(RA, t0_of(k), Interior{});
            }
        }
    }
    // The slab's last tile, by the wave whose round-robin turn it is.
    if (tile_end == ntiles && wave == (ntiles - 1 - tile_begin) % W) {
        TileRegs R;
        const int t0 = (ntiles - 1) * ATTN_TILE;
        load_tile(R, kslab, vslab, t0, l16, lg, append_row, knew_row);
        compute(R, t0, Last{});
    }

    // Row sums: each of the four lane groups holds a quarter of the rows.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        lsum[nt] += __shfl_xor(lsum[nt], 16);
        lsum[nt] += __shfl_xor(lsum[nt], 32);
    }

    // Merge the four waves through LDS, one 16-row block at a time, and
    // write this workgroup's partial.
    __shared__ float wm[W][16], wl[W][16];
    constexpr int EPT = 2048 / (W * 64);  // merged outputs per thread (16 rows x 128)
    auto store_ept = [](float* dst, const float* o) {
        if constexpr (EPT % 4 == 0) {
#pragma unroll
            for (int e = 0; e < EPT; e += 4)
                *reinterpret_cast<f32x4*>(dst + e) = f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]};
        } else {
#pragma unroll
            for (int e = 0; e < EPT; ++e) dst[e] = o[e];
        }
    };
    const size_t slabs = (size_t)p.nb * p.hkv;
    float* part_acc = p.part + ((size_t)slab * p.nsplit + s) * RP * D;
    float* part_ml = p.part + slabs * p.nsplit * RP * D + ((size_t)slab * p.nsplit + s) * RP * 2;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        if (lg == 0) {
            wm[wave][l16] = m[nt];
            wl[wave][l16] = lsum[nt];
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) buf[(wave * 16 + l16) * D + 16 * dt + 4 * lg + i] = acc[nt][dt][i];
        __syncthreads();
        {
            const int n = tid / (D / EPT), d0 = (tid % (D / EPT)) * EPT;
            float M = wm[0][n];
#pragma unroll
            for (int w = 1; w < W; ++w) M = fmaxf(M, wm[w][n]);
            float f[W], L = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                f[w] = exp2f((wm[w][n] - M) * LOG2E);   // waves without rows: 2^(-huge) = 0
                L += f[w] * wl[w][n];
            }
            float o[EPT];
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                float a = 0.f;
#pragma unroll
                for (int w = 0; w < W; ++w) a += f[w] * buf[(w * 16 + n) * D + d0 + e];
                o[e] = a;
            }
            const int r = nt * 16 + n;
            if (p.nsplit == 1) {
                // The whole slab is this workgroup's: finish the rows here.
                if (r < p.rows) {
                    const float inv = 1.f / L;
                    const int qi = r / p.g, h = j * p.g + r % p.g;
                    float* dst = p.out + p.out_off[qi] + ((size_t)b * p.hq + h) * D + d0;
#pragma unroll
                    for (int e = 0; e < EPT; ++e) o[e] *= inv;
                    store_ept(dst, o);
                    if (d0 == 0 && p.lse) p.lse[p.lse_off[qi] + (size_t)b * p.hq + h] = M + logf(L);
                }
            } else if (r < p.rows) {          // padding rows are never merged
                if (p.arrive) {
                    store_part_coh<EPT>(p, part_acc, part_ml, r, d0, o, M, L);
                } else {
                    store_ept(part_acc + (size_t)r * D + d0, o);
                    if (d0 == 0) {
                        part_ml[r * 2] = M;
                        part_ml[r * 2 + 1] = L;
                    }
                }
            }
        }
        __syncthreads();
    }

    if (p.append_write && tile_end == ntiles) write_append_row<uint16_t>(p, slab, cslab, T - 1);
    if (p.nsplit > 1 && p.arrive && arrive_last(p.arrive + slab, p.nsplit))
        combine_rows<W * 64, true>(p, j, b, 0, p.rows, buf);
}

// float32 path: plain VALU arithmetic, up to 16 query rows per launch.
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnLaunch p) {
    constexpr int TT = ATTN_TILE_F32;
    const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int slab = b * p.hkv + j;
    const int tid = threadIdx.x;
    const int phys = seq_phys(p.sm, b);
    const int T = seq_rows(p.sm, b, phys);     // 0 rows: no tile, an empty partial
    const int ntiles = (T + TT - 1) / TT;
    const int tile_begin = s * p.tps;
    const int tile_end = min(tile_begin + p.tps, ntiles);
    const size_t cslab = (size_t)max(phys, 0) * p.hkv + j;
    const float* kslab = reinterpret_cast<const float*>(p.k) + cslab * p.t_cap * D;
    const float* vslab = reinterpret_cast<const float*>(p.v) + cslab * p.t_cap * D;
    const float* knew = reinterpret_cast<const float*>(p.k_new) + (size_t)slab * D;
    const float* vnew = reinterpret_cast<const float*>(p.v_new) + (size_t)slab * D;
    const int append_row = p.append_read ? T - 1 : -1;

    __shared__ float qs[16][D];
    __shared__ float Sx[16][TT + 1];
    __shared__ float mrow[16], lrow[16], arow[16];

    for (int idx = tid; idx < 16 * D; idx += blockDim.x) {
        const int r = idx / D, d = idx % D;
        float x = 0.f;
        if (r < p.rows) {
            const int qi = r / p.g, h = j * p.g + r % p.g;
            x = reinterpret_cast<const float*>(p.q)[p.q_off[qi] + ((size_t)b * p.hq + h) * D + d];
        }
        qs[r][d] = x;
    }
    if (tid < 16) {
        mrow[tid] = -INFINITY;
        lrow[tid] = 0.f;
    }
    __syncthreads();

    const int d = tid % D, half = tid / D;   // P*V: channel d, rows half + 2k
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;

    for (int tile = tile_begin; tile < tile_end; ++tile) {
        const int t0 = tile * TT;
        // S = scale * q . k for 64 rows; four lanes per row, 32 channels each.
        {
            const int tr = tid / 4, part = tid % 4;
            const int t = t0 + tr;
            float kv[32];
            const float* kr = (t == append_row) ? knew : kslab + (size_t)t * D;
#pragma unroll
            for (int x = 0; x < 32; x += 4) {
                const f32x4 v4 = *reinterpret_cast<const f32x4*>(kr + 32 * part + x);
                kv[x] = v4[0]; kv[x + 1] = v4[1]; kv[x + 2] = v4[2]; kv[x + 3] = v4[3];
            }
            for (int r = 0; r < 16; ++r) {
                float a = 0.f;
#pragma unroll
                for (int x = 0; x < 32; ++x) a = fmaf(qs[r][32 * part + x], kv[x], a);
                a += __shfl_xor(a, 1);
                a += __shfl_xor(a, 2);
                if (part == 0) Sx[r][tr] = (t < T) ? a * p.scale : -INFINITY;
            }
        }
        __syncthreads();
        // Online softmax: 16 threads per row, 4 columns each.
        {
            const int r = tid / 16, sub = tid % 16;
            float mx = -INFINITY;
#pragma unroll
            for (int c = 0; c < 4; ++c) mx = fmaxf(mx, Sx[r][4 * sub + c]);
#pragma unroll
            for (int mk = 1; mk < 16; mk <<= 1) mx = fmaxf(mx, __shfl_xor(mx, mk));
            const float mold = mrow[r];
            const float mnew = fmaxf(mold, mx);
            float ps = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float pv = expf(Sx[r][4 * sub + c] - mnew);
                Sx[r][4 * sub + c] = pv;
                ps += pv;
            }
#pragma unroll
            for (int mk = 1; mk < 16; mk <<= 1) ps += __shfl_xor(ps, mk);
            if (sub == 0) {
                const float a = expf(mold - mnew);
                arow[r] = a;
                lrow[r] = lrow[r] * a + ps;
                mrow[r] = mnew;
            }
        }
        __syncthreads();
        // acc[r][d] = acc * alpha + sum_t p[r][t] V^T[d][t]
        {
            float vv[TT];
#pragma unroll
            for (int x = 0; x < TT; x += 4) {
                const f32x4 v4 = *reinterpret_cast<const f32x4*>(vslab + vt_off(t0 + x, d));
                vv[x] = v4[0]; vv[x + 1] = v4[1]; vv[x + 2] = v4[2]; vv[x + 3] = v4[3];
            }
            if (t0 + TT >= T) {   // last tile: rows past the end, appended row
#pragma unroll
                for (int x = 0; x < TT; ++x) {
                    if (t0 + x == append_row) vv[x] = vnew[d];
                    else if (t0 + x >= T) vv[x] = 0.f;
                }
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int r = half + 2 * k;
                float a = acc[k] * arow[r];
#pragma unroll
                for (int x = 0; x < TT; ++x) a = fmaf(Sx[r][x], vv[x], a);
                acc[k] = a;
            }
        }
        __syncthreads();
    }

    const size_t slabs = (size_t)p.nb * p.hkv;
    float* part_acc = p.part + ((size_t)slab * p.nsplit + s) * 16 * D;
    float* part_ml = p.part + slabs * p.nsplit * 16 * D + ((size_t)slab * p.nsplit + s) * 16 * 2;
#pragma unroll
    for (int k = 0; k < 8; ++k) part_acc[(size_t)(half + 2 * k) * D + d] = acc[k];
    if (tid < 16) {
        part_ml[tid * 2] = mrow[tid];
        part_ml[tid * 2 + 1] = lrow[tid];
    }
    if (p.append_write && tile_begin < ntiles && tile_end == ntiles)
        write_append_row<float>(p, slab, cslab, T - 1);
}

// Row rows(b) - 1 of every slab of sequence b <- its new row.
template <typename T>
__global__ __launch_bounds__(128) void append_kernel(T* k, T* v, int hkv, int t_cap, SeqMap sm,
                                                     const T* k_new, const T* v_new) {
    const int b = blockIdx.y;
    const size_t slab = (size_t)b * hkv + blockIdx.x;
    const int phys = seq_phys(sm, b);
    const int t = seq_rows(sm, b, phys) - 1;
    if (t < 0) return;
    const size_t cslab = (size_t)phys * hkv + blockIdx.x;
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        k[(cslab * t_cap + t) * D + d] = k_new[slab * D + d];
        v[cslab * t_cap * D + vt_off(t, d)] = v_new[slab * D + d];
    }
}

}  // namespace

hipError_t launch_attn(const AttnLaunch& p, int dtype, int nt, hipStream_t st) {
    const dim3 grid(p.nsplit, p.hkv, p.nb);
    if (dtype == 0) {
        hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(256), 0, st, p);
    } else {
        auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(ATTN_WAVES * 64), 0, st, p); };
        if (nt == 1)
            go(attn_bf16_kernel<1, ATTN_WAVES, 1>);
        else if (nt == 2)
            go(attn_bf16_kernel<2, ATTN_WAVES, 1>);
        else
            go(attn_bf16_kernel<4, ATTN_WAVES, 1>);
    }
    // bf16 launches with one split per slab finish their rows themselves, and
    // so do those whose last workgroup per slab merges.
    if (dtype == 0 || (p.nsplit > 1 && !p.arrive)) return launch_attn_combine(p, st);
    return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnLaunch& p, hipStream_t st) {
    const long long work = (long long)p.rows * (D / 8) * p.nsplit;   // (item, split) pairs per slab
    if (p.nsplit >= 8 && work > 4 * 256) {
        // Up to 16 split groups per item and 1024 threads: a workgroup takes
        // 1024 / (16 * groups) rows (4 once a slab has 16 splits or more),
        // so every thread folds about nsplit / 16 splits.
        const int groups = std::min(p.nsplit, 16);
        const int rpb = std::max(1, 1024 / ((D / 8) * groups));
        const int nrb = (p.rows + rpb - 1) / rpb;
        hipLaunchKernelGGL(attn_combine_kernel<1024>, dim3(p.hkv, p.nb, nrb), dim3(1024), 0, st, p);
    } else {
        hipLaunchKernelGGL(attn_combine_kernel<256>, dim3(p.hkv, p.nb), dim3(256), 0, st, p);
    }
    return hipGetLastError();
}

hipError_t launch_append(const void* k, const void* v, int nb, int hkv, int t_cap,
                         const SeqMap& sm, const void* k_new, const void* v_new, int elem,
                         hipStream_t st) {
    const dim3 grid(hkv, nb);
    if (elem == 4)
        hipLaunchKernelGGL(append_kernel<float>, grid, dim3(128), 0, st, (float*)k, (float*)v,
                           hkv, t_cap, sm, (const float*)k_new, (const float*)v_new);
    else
        hipLaunchKernelGGL(append_kernel<uint16_t>, grid, dim3(128), 0, st, (uint16_t*)k,
                           (uint16_t*)v, hkv, t_cap, sm, (const uint16_t*)k_new,
                           (const uint16_t*)v_new);
    return hipGetLastError();
}

}  // namespace kvc
