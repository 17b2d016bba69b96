// Observation-window score and value range over one cache slot.
//
// VASE summary (gist.science 2606.03928): §2.B scores rows by the attention
// the last decode queries (SnapKV's observation window) pay them, and §2.A
// measures each value row by Range(v) = max(v) - min(v).
//
// score[b][j][t] = sum over the g heads of kv head j and the w window rows i
// of softmax_t(scale * q_obs[i][b][h] . K[t]), where window row i sees rows
// t <= t_len - w + i.  The g*w query rows against a 32-row K tile are a real
// dense contraction (128-160 rows x 128 channels x 32 rows), so it runs on
// v_mfma_f32_16x16x32_bf16: A = 16 query rows x 32 channels, B = 32 channels
// x 16 cache rows; the output lane layout puts one cache row per lane column,
// so the column sums over query rows are in-lane adds plus two cross-lane
// steps.  The score pass gives each wave whole tiles and all g*w query rows
// (staged in LDS); every sum is taken in a fixed order (deterministic).
//
// Without the log-normalisers of the window rows a first pass computes them:
// each wave owns 32 query rows (one head's window) and keeps a per-row online
// max / sum over its workgroup's tiles, then a small kernel merges the splits'
// pairs (kernel boundaries order the two, so no cross-workgroup fences are
// needed).  The range is fused into the score pass: the wave that takes a
// tile also reads the tile's V block.
//
// Ragged batches: sequence b has its own row count T_b (window row i sees
// t <= T_b - w + i; a row that sees nothing adds nothing) and is read from
// cache entry phys(b); per-row outputs keep the launch's t_len as their row
// stride.
#include <type_traits>

#include "common.h"
#include "kvc_internal.h"

namespace kvc {

namespace {

__device__ __forceinline__ bf16x8 as_bf(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Lane permutation inside a 16-lane row (DPP, a plain VALU move).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Max / min over the 16 lanes of a row; every lane of the row gets it.
// Swap neighbours, swap pairs, mirror the half-rows, mirror the row.
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    return fmaxf(v, dpp_mov<0x140>(v));
}
__device__ __forceinline__ float row16_min(float v) {
    v = fminf(v, dpp_mov<0xB1>(v));
    v = fminf(v, dpp_mov<0x4E>(v));
    v = fminf(v, dpp_mov<0x141>(v));
    return fminf(v, dpp_mov<0x140>(v));
}

// V block of the 32 rows t0..t0+31 of one slab (one wave): lane (l16, lg)
// gets channels 16*dt + l16 of rows t0 + 8*lg .. +8.
__device__ __forceinline__ void load_vtile(u32x4 (&x)[8], const uint16_t* vslab, int t0, int lane) {
    const int l16 = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) x[dt] = load_stream16(vslab + vt_off(t0, 16 * dt + l16) + 8 * lg);
}

// Range of those 32 rows from the loaded block.
__device__ __forceinline__ void range_tile_bf16(const u32x4 (&x)[8], int t0, int T,
                                                float* range_out, int lane) {
    const int l16 = lane & 15, lg = lane >> 4;
    float mx[8], mn[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        mx[jj] = -INFINITY;
        mn[jj] = INFINITY;
    }
    // Two channel blocks per step, so each step is one three-input max and
    // one three-input min per row.
#pragma unroll
    for (int dt = 0; dt < 8; dt += 2) {
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            const float a0 = bf16lo(x[dt][w2]), a1 = bf16lo(x[dt + 1][w2]);
            const float b0 = bf16hi(x[dt][w2]), b1 = bf16hi(x[dt + 1][w2]);
            mx[2 * w2] = fmaxf(mx[2 * w2], fmaxf(a0, a1));
            mn[2 * w2] = fminf(mn[2 * w2], fminf(a0, a1));
            mx[2 * w2 + 1] = fmaxf(mx[2 * w2 + 1], fmaxf(b0, b1));
            mn[2 * w2 + 1] = fminf(mn[2 * w2 + 1], fminf(b0, b1));
        }
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        mx[jj] = row16_max(mx[jj]);
        mn[jj] = row16_min(mn[jj]);
    }
    if (l16 == 0) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int t = t0 + 8 * lg + jj;
            if (t < T) range_out[t] = mx[jj] - mn[jj];
        }
    }
}

// Query fragments of one wave: 2 blocks of 16 rows, 4 channel chunks.
struct QFrag {
    bf16x8 a[2][4];
};

__device__ __forceinline__ void load_qfrag(QFrag& Q, const ScoreLaunch& p, int b, int j, int wave,
                                           int l16, int lg) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const int R = wave * 32 + mt * 16 + l16;
        if (R < p.rows) {
            const int h = j * p.g + R / p.w, iw = R % p.w;
            const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q_obs) +
                                 (((size_t)iw * p.q_nb + score_qrow(p.q_idx, b)) * p.hq + h) * D +
                                 8 * lg;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) Q.a[mt][kc] = as_bf(load16(qp + 32 * kc));
        } else {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) Q.a[mt][kc] = as_bf(u32x4{0u, 0u, 0u, 0u});
        }
    }
}

// The K operand fragments of one 32-row tile: rows t0 + 16*cg + l16.
__device__ __forceinline__ void load_ktile(u32x4 (&kb)[2][4], const uint16_t* kslab, int t0,
                                           int l16, int lg) {
#pragma unroll
    for (int cg = 0; cg < 2; ++cg) {
        const uint16_t* kr = kslab + (size_t)(t0 + 16 * cg + l16) * D + 8 * lg;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) kb[cg][kc] = load16(kr + 32 * kc);
    }
}

// S[mt][cg][i] = q_row(wave*32 + mt*16 + 4*lg + i) . k_row(t0 + 16*cg + l16)
__device__ __forceinline__ void score_tile_product(const QFrag& Q, const u32x4 (&kb)[2][4],
                                                   f32x4 S[2][2]) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Q.a[mt][kc], as_bf(kb[cg][kc]), acc,
                                                              0, 0, 0);
            S[mt][cg] = acc;
        }
}

constexpr float LOG2E = 1.4426950408889634f;

// Merge two (max, sum-of-exp) pairs.
__device__ __forceinline__ void ms_merge(float& m, float& z, float m2, float z2) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    z = z * exp2f((m - mn) * LOG2E) + z2 * exp2f((m2 - mn) * LOG2E);
    m = mn;
}

// Pass 1: per window row, max and sum of exp over its visible rows.  Each
// wave owns 32 window rows and runs them against every tile of its split.
// PF = 1 keeps the next tile's K loads in flight while a tile is computed
// (two register sets; at most 512 threads, i.e. 256 window rows, so that
// the registers fit); PF = 0 serves larger windows one tile at a time.
template <int PF>
__global__ __launch_bounds__(PF ? 512 : 1024) void score_stats_bf16(ScoreLaunch p) {
    const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int slab = b * p.hkv + j;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int l16 = lane & 15, lg = lane >> 4;
    const int phys = seq_phys(p.sm, b);
    const int T = seq_rows(p.sm, b, phys);   // a split past the end writes (-inf, 0)
    const int ntiles = (T + SCORE_TILE - 1) / SCORE_TILE;
    const int tile_begin = s * p.tps, tile_end = min(tile_begin + p.tps, ntiles);
    const uint16_t* kslab =
        reinterpret_cast<const uint16_t*>(p.k) + ((size_t)max(phys, 0) * p.hkv + j) * p.t_cap * D;

    QFrag Q;
    load_qfrag(Q, p, b, j, wave, l16, lg);
    float m[2][4], z[2][4];
    int lim[2][4];   // last visible cache row of each of the lane's rows
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m[mt][i] = -INFINITY;
            z[mt][i] = 0.f;
            const int R = wave * 32 + mt * 16 + 4 * lg + i;
            lim[mt][i] = (R < p.rows) ? T - p.w + R % p.w : -1;
        }
    auto fold = [&](const u32x4 (&kb)[2][4], int t0) {
        f32x4 S[2][2];
        score_tile_product(Q, kb, S);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x0 = S[mt][0][i] * p.scale, x1 = S[mt][1][i] * p.scale;
                if (t0 + l16 > lim[mt][i]) x0 = -INFINITY;
                if (t0 + 16 + l16 > lim[mt][i]) x1 = -INFINITY;
                const float mn = fmaxf(m[mt][i], fmaxf(x0, x1));
                if (mn != -INFINITY) {
                    z[mt][i] = z[mt][i] * exp2f((m[mt][i] - mn) * LOG2E) +
                               exp2f((x0 - mn) * LOG2E) + exp2f((x1 - mn) * LOG2E);
                    m[mt][i] = mn;
                }
            }
    };
    if constexpr (PF == 0) {
        for (int tile = tile_begin; tile < tile_end; ++tile) {
            u32x4 kb[2][4];
            load_ktile(kb, kslab, tile * SCORE_TILE, l16, lg);
            fold(kb, tile * SCORE_TILE);
        }
    } else {
        // Tiles in order (the fold's order is the same as with PF = 0); the
        // loads inside the loop body are unconditional.
        const int n = max(0, tile_end - tile_begin);
        auto t0_of = [&](int k) { return (tile_begin + k) * SCORE_TILE; };
        if (n > 0) {
            u32x4 KA[2][4], KB[2][4];
            load_ktile(KA, kslab, t0_of(0), l16, lg);
            int k = 0;
            for (; k + 2 < n; k += 2) {
                load_ktile(KB, kslab, t0_of(k + 1), l16, lg);
                fold(KA, t0_of(k));
                load_ktile(KA, kslab, t0_of(k + 2), l16, lg);
                fold(KB, t0_of(k + 1));
            }
            if (k + 1 < n) {
                load_ktile(KB, kslab, t0_of(k + 1), l16, lg);
                fold(KA, t0_of(k));
                fold(KB, t0_of(k + 1));
            } else {
                fold(KA, t0_of(k));
            }
        }
    }
    // Merge the 16 lanes (cache-row columns) that share each query row.
#pragma unroll
    for (int k = 1; k < 16; k <<= 1)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float m2 = __shfl_xor(m[mt][i], k), z2 = __shfl_xor(z[mt][i], k);
                ms_merge(m[mt][i], z[mt][i], m2, z2);
            }
    float* st = p.stats + ((size_t)slab * p.nsplit + s) * p.rows_pad * 2;
    if (l16 == 0) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int R = wave * 32 + mt * 16 + 4 * lg + i;
                st[R * 2] = m[mt][i];
                st[R * 2 + 1] = z[mt][i];
            }
    }
}

// Pass 1 in the score pass's structure (windows of up to 256 rows): the
// slab's g*w window queries are staged in LDS once per workgroup and each
// wave takes whole 32-row tiles (round-robin), so every K byte is loaded by
// one wave once.  The product runs transposed, S^T = K Q^T (the K tile is
// the A operand as loaded, the staged queries the B operand), so a lane
// holds one window row and eight cache rows of the tile per 16-row query
// block, and each row needs one running (reference, sum) pair per lane:
// sum += e^(x - ref), one fma and one bare exp2 per logit.  The reference is
// a logit the lane has seen; it moves (rescaling the sum) only when a
// logit exceeds it by more than RESCALE (a wave-uniform branch, taken on the
// first tile and then rarely), so a term is at most e^RESCALE and a slab's
// sum stays far below the float32 range, while the largest term is at least
// 1 (terms the bare exp2 flushes to zero are below 2^-126 of the sum).  The
// four lanes that share a row and then the four waves merge their pairs in a
// fixed order; the workgroup writes one (reference, sum) pair per row and
// split, in natural-log units, for score_lse_merge.
constexpr float RESCALE = 40.f;

template <int MT>
__global__ __launch_bounds__(256) void score_stats_tiles_bf16(ScoreLaunch p) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NW = 4;
    const BlockXYZ blk = xcd_run_block(true);
    const int s = blk.x, j = blk.y, b = blk.z;
    const int slab = b * p.hkv + j;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int l16 = lane & 15, lg = lane >> 4;
    const int phys = seq_phys(p.sm, b);
    const int T = seq_rows(p.sm, b, phys);     // a split past the end writes (-inf, 0)
    const int ntiles = (T + SCORE_TILE - 1) / SCORE_TILE;
    const int tile_begin = s * p.tps, tile_end = min(tile_begin + p.tps, ntiles);
    uint16_t* qs = reinterpret_cast<uint16_t*>(smem);                          // [MT*16][QPITCH]

    const uint16_t* q = reinterpret_cast<const uint16_t*>(p.q_obs);
    const int qb = score_qrow(p.q_idx, b);
    for (int x = tid; x < MT * 16 * (D / 8); x += blockDim.x) {
        const int R = x / (D / 8), c = x % (D / 8);
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (R < p.rows) {
            const int h = j * p.g + R / p.w, iw = R % p.w;
            v = load16(q + (((size_t)iw * p.q_nb + qb) * p.hq + h) * D + 8 * c);
        }
        *reinterpret_cast<u32x4*>(qs + R * SCORE_QPITCH + 8 * c) = v;
    }
    __syncthreads();

    const uint16_t* kslab =
        reinterpret_cast<const uint16_t*>(p.k) + ((size_t)max(phys, 0) * p.hkv + j) * p.t_cap * D;
    const float c1 = p.scale * LOG2E;
    float m[MT], z[MT];
    int lim[MT];                  // last cache row the lane's window row sees
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        m[mt] = -INFINITY;
        z[mt] = 0.f;
        const int R = mt * 16 + l16;
        lim[mt] = R < p.rows ? T - p.w + R % p.w : -1;   // padding rows see nothing
    }

    auto body = [&](const u32x4 (&kb)[2][4], int t0, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4 S[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            const uint16_t* qrow = qs + (mt * 16 + l16) * SCORE_QPITCH + 8 * lg;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const bf16x8 bq = as_bf(*reinterpret_cast<const u32x4*>(qrow + 32 * kc));
                S[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(kb[0][kc]), bq, S[0], 0, 0, 0);
                S[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(kb[1][kc]), bq, S[1], 0, 0, 0);
            }
            // S[cg][i]: cache row t0 + 16*cg + 4*lg + i, window row mt*16 + l16
            float xm = -INFINITY;
#pragma unroll
            for (int cg = 0; cg < 2; ++cg)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool v = !TAIL || t0 + 16 * cg + 4 * lg + i <= lim[mt];
                    xm = fmaxf(xm, v ? S[cg][i] : -INFINITY);
                }
            xm *= p.scale;
            const bool need = xm > m[mt] + RESCALE;
            if (__builtin_amdgcn_ballot_w64(need)) {
                if (need) {
                    z[mt] = m[mt] == -INFINITY ? 0.f : z[mt] * exp2f((m[mt] - xm) * LOG2E);
                    m[mt] = xm;
                }
            }
            const float nl = -m[mt] * LOG2E;
            float acc = 0.f;
#pragma unroll
            for (int cg = 0; cg < 2; ++cg)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float pr = __builtin_amdgcn_exp2f(fmaf(S[cg][i], c1, nl));
                    if constexpr (TAIL) pr = t0 + 16 * cg + 4 * lg + i <= lim[mt] ? pr : 0.f;
                    acc += pr;
                }
            if (m[mt] != -INFINITY) z[mt] += acc;     // a row with no reference yet saw nothing
        }
    };
    using Interior = std::integral_constant<bool, false>;
    using Tail = std::integral_constant<bool, true>;
    for (int tile = tile_begin + wave; tile < tile_end; tile += NW) {
        const int t0 = tile * SCORE_TILE;
        u32x4 kb[2][4];
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) {
            const uint16_t* kr = kslab + (size_t)(t0 + 16 * cg + l16) * D + 8 * lg;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) kb[cg][kc] = load_stream16(kr + 32 * kc);
        }
        if (t0 + SCORE_TILE - 1 <= T - p.w)
            body(kb, t0, Interior{});
        else
            body(kb, t0, Tail{});
    }
    // the four lane groups (cache rows) that share each window row
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int k = 16; k < 64; k <<= 1) {
            const float m2 = __shfl_xor(m[mt], k), z2 = __shfl_xor(z[mt], k);
            ms_merge(m[mt], z[mt], m2, z2);
        }
    // the four waves, in order, through LDS (the staged queries are done)
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);                 // [NW][MT*16][2]
    if (lg == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int R = mt * 16 + l16;
            red[(wave * MT * 16 + R) * 2] = m[mt];
            red[(wave * MT * 16 + R) * 2 + 1] = z[mt];
        }
    }
    __syncthreads();
    float* st = p.stats + ((size_t)slab * p.nsplit + s) * p.rows_pad * 2;
    for (int R = tid; R < p.rows; R += blockDim.x) {
        float mm = red[R * 2], zz = red[R * 2 + 1];
        for (int w2 = 1; w2 < NW; ++w2)
            ms_merge(mm, zz, red[(w2 * MT * 16 + R) * 2], red[(w2 * MT * 16 + R) * 2 + 1]);
        st[R * 2] = zz > 0.f ? mm : -INFINITY;
        st[R * 2 + 1] = zz;
    }
}

// Merge the splits' (max, sum) pairs of every window row into its
// log-normaliser; one workgroup per slab, one thread per row, splits folded
// in order.
// Merge of the statistics splits: one workgroup per slab; SG threads share a
// window row when the slab has fewer rows than threads, each folding every
// SG-th split, in two passes with independent reads (the row's maximum over
// the splits' m, then sum_s z_s e^(m_s - M); a split without visible rows
// has m = -inf), the split groups combined through LDS in a fixed order.
__global__ __launch_bounds__(1024) void score_lse_merge(ScoreLaunch p) {
    constexpr int NTH = 1024;
    __shared__ float red[NTH];
    const int slab = blockIdx.y * p.hkv + blockIdx.x, tid = threadIdx.x;
    const float* all = p.stats + (size_t)slab * p.nsplit * p.rows_pad * 2;
    const int SG = max(1, min(p.nsplit, NTH / max(1, p.rows)));
    const int per = SG == 1 ? NTH : p.rows;
    for (int R0 = 0; R0 < p.rows; R0 += per) {
        const int sg = tid / per, R = R0 + tid % per;
        const bool act = sg < SG && R < p.rows;
        float mm = -INFINITY, zz = 0.f;
        if (act)
#pragma unroll 4
            for (int sp = sg; sp < p.nsplit; sp += SG)
                mm = fmaxf(mm, all[((size_t)sp * p.rows_pad + R) * 2]);
        red[tid] = mm;
        __syncthreads();
        if (act)
            for (int s2 = 0; s2 < SG; ++s2) mm = fmaxf(mm, red[s2 * per + tid % per]);
        __syncthreads();
        if (act && mm != -INFINITY)
#pragma unroll 4
            for (int sp = sg; sp < p.nsplit; sp += SG) {
                const float m2 = all[((size_t)sp * p.rows_pad + R) * 2];
                const float z2 = all[((size_t)sp * p.rows_pad + R) * 2 + 1];
                zz += m2 == -INFINITY ? 0.f : z2 * exp2f((m2 - mm) * LOG2E);
            }
        red[tid] = zz;
        __syncthreads();
        if (act && sg == 0) {
            for (int s2 = 1; s2 < SG; ++s2) zz += red[s2 * per + tid % per];
            p.lse_ws[(size_t)slab * p.rows_pad + R] = mm + logf(zz);
        }
        __syncthreads();
    }
}

// Pass 2: column sums of the window softmax, plus the fused value range.
// The window queries of the slab (all g*w rows) and their log-normalisers
// are staged in LDS once per workgroup; each wave then takes whole 32-row
// tiles (round-robin), so every K and V byte is loaded by exactly one wave
// and a wave keeps its tile's K and V loads in flight while the other waves
// compute.  Per tile the wave runs all 16-row query blocks against the K
// tile (the A operand comes from LDS), adds p' = 2^(s*scale*log2 e -
// lse*log2 e + 64) over the block's rows in-lane with the bare hardware
// exp2 (one fma and one v_exp_f32 per logit), finishes the column sums with
// two cross-lane steps and scales them by 2^-64: the tile's 32 scores leave
// without any cross-wave reduction.  The 2^64 bias keeps every p >= 2^-190
// a normal float inside the sum (the bare exp2 does not return denormals),
// and since p <= 1 the biased terms cannot overflow.  The row pitch of the
// staged queries is 272 bytes, so the 16 rows one 16-byte A-operand read
// touches fall in distinct LDS banks.
constexpr int QPITCH = SCORE_QPITCH;
static_assert(QPITCH >= D && QPITCH % 8 == 0, "16-byte aligned staged rows");
constexpr float EXP_BIAS = 64.f;
constexpr float EXP_UNBIAS = 5.421010862427522e-20f;   // 2^-64

template <bool RANGE>
__global__ __launch_bounds__(256) void score_main_bf16(ScoreLaunch p) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NW = 4;
    // Contiguous runs of (split, head, batch) blocks per XCD: the splits of
    // a slab share the window queries they stage through one L2.
    const BlockXYZ blk = xcd_run_block(true);
    const int s = blk.x, j = blk.y, b = blk.z;
    const int slab = b * p.hkv + j;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int l16 = lane & 15, lg = lane >> 4;
    const int phys = seq_phys(p.sm, b);
    const int T = seq_rows(p.sm, b, phys);
    const int ntiles = (T + SCORE_TILE - 1) / SCORE_TILE;
    const int tile_begin = s * p.main_tps, tile_end = min(tile_begin + p.main_tps, ntiles);
    if (tile_begin >= ntiles) return;   // past the sequence's end (whole workgroup)
    const int MT = (p.rows + 15) / 16;
    uint16_t* qs = reinterpret_cast<uint16_t*>(smem);                          // [MT*16][QPITCH]
    float* l2s = reinterpret_cast<float*>(smem + (size_t)MT * 16 * QPITCH * 2);  // [MT*16] 64 - lse*log2 e
    int* lims = reinterpret_cast<int*>(l2s + MT * 16);                          // [MT*16]

    const uint16_t* q = reinterpret_cast<const uint16_t*>(p.q_obs);
    const int qb = score_qrow(p.q_idx, b);
    for (int x = tid; x < MT * 16 * (D / 8); x += blockDim.x) {
        const int R = x / (D / 8), c = x % (D / 8);
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (R < p.rows) {
            const int h = j * p.g + R / p.w, iw = R % p.w;
            v = load16(q + (((size_t)iw * p.q_nb + qb) * p.hq + h) * D + 8 * c);
        }
        *reinterpret_cast<u32x4*>(qs + R * QPITCH + 8 * c) = v;
    }
    for (int R = tid; R < MT * 16; R += blockDim.x) {
        if (R < p.rows) {
            const int h = j * p.g + R / p.w, iw = R % p.w;
            const float l = p.lse_obs ? p.lse_obs[((size_t)iw * p.q_nb + qb) * p.hq + h]
                                      : p.lse_ws[(size_t)slab * p.rows_pad + R];
            l2s[R] = EXP_BIAS - l * LOG2E;
            lims[R] = T - p.w + iw;
        } else {
            l2s[R] = -INFINITY;   // padding rows: p = 2^-inf = 0
            lims[R] = -1;
        }
    }
    __syncthreads();

    const size_t cslab = (size_t)phys * p.hkv + j;
    const uint16_t* kslab = reinterpret_cast<const uint16_t*>(p.k) + cslab * p.t_cap * D;
    const uint16_t* vslab = reinterpret_cast<const uint16_t*>(p.v) + cslab * p.t_cap * D;
    float* score = p.score + (size_t)slab * p.t_len;
    float* range = RANGE ? p.range + (size_t)slab * p.t_len : nullptr;
    const float c1 = p.scale * LOG2E;

    // TAIL: some (row, column) pairs of the tile are not visible (the causal
    // window, or columns past t_len whose K bits are arbitrary); they are
    // replaced by 0 with a select, never multiplied.
    auto body = [&](const u32x4 (&kb)[2][4], int t0, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        float c[2] = {0.f, 0.f};
        for (int mt = 0; mt < MT; ++mt) {
            f32x4 S[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            const uint16_t* qrow = qs + (mt * 16 + l16) * QPITCH + 8 * lg;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const bf16x8 a = as_bf(*reinterpret_cast<const u32x4*>(qrow + 32 * kc));
                S[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf(kb[0][kc]), S[0], 0, 0, 0);
                S[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf(kb[1][kc]), S[1], 0, 0, 0);
            }
            // S[cg][i]: query row mt*16 + 4*lg + i, cache row t0 + 16*cg + l16
            const f32x4 l2 = *reinterpret_cast<const f32x4*>(l2s + mt * 16 + 4 * lg);
#pragma unroll
            for (int cg = 0; cg < 2; ++cg)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float pr = __builtin_amdgcn_exp2f(fmaf(S[cg][i], c1, l2[i]));
                    if constexpr (TAIL)
                        pr = (t0 + 16 * cg + l16 <= lims[mt * 16 + 4 * lg + i]) ? pr : 0.f;
                    c[cg] += pr;
                }
        }
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) {
            c[cg] += __shfl_xor(c[cg], 16);
            c[cg] += __shfl_xor(c[cg], 32);
            const int t = t0 + 16 * cg + l16;
            if (lg == 0 && t < T) score[t] = c[cg] * EXP_UNBIAS;
        }
    };
    using Interior = std::integral_constant<bool, false>;
    using Tail = std::integral_constant<bool, true>;

    for (int tile = tile_begin + wave; tile < tile_end; tile += NW) {
        const int t0 = tile * SCORE_TILE;
        u32x4 kb[2][4], vb[8];
#pragma unroll
        for (int cg = 0; cg < 2; ++cg) {
            const uint16_t* kr = kslab + (size_t)(t0 + 16 * cg + l16) * D + 8 * lg;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) kb[cg][kc] = load_stream16(kr + 32 * kc);
        }
        if constexpr (RANGE) load_vtile(vb, vslab, t0, lane);
        if (t0 + SCORE_TILE - 1 <= T - p.w)
            body(kb, t0, Interior{});
        else
            body(kb, t0, Tail{});
        if constexpr (RANGE) range_tile_bf16(vb, t0, T, range, lane);
    }
}


// ---------------------------------------------------------------------------
// float32 path (VALU), 64-row tiles staged in LDS.
// ---------------------------------------------------------------------------
constexpr int FT = 64;

__device__ void f32_stage_k(float (*ks)[D + 1], const float* kslab, int t0, int tid, int nthr) {
    for (int idx = tid; idx < FT * D; idx += nthr) {
        const int t = idx / D, d = idx % D;
        ks[t][d] = kslab[(size_t)(t0 + t) * D + d];
    }
}

__device__ float f32_dot_row(const float* q, const float (*ks)[D + 1], int t) {
    float a = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) a = fmaf(q[d], ks[t][d], a);
    return a;
}

// One workgroup (256 threads) per (split, kv head, batch); thread
// (t = tid % 64, rgroup = tid / 64) handles window rows rgroup, rgroup+4, ...
__global__ __launch_bounds__(256) void score_f32(ScoreLaunch p, int stats_pass) {
    const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int slab = b * p.hkv + j;
    const int qb = score_qrow(p.q_idx, b);
    const int tid = threadIdx.x, tl = tid % FT, rg = tid / FT;
    const int phys = seq_phys(p.sm, b);
    const int T = seq_rows(p.sm, b, phys);
    const int ntiles = (T + FT - 1) / FT;
    const int tile_begin = s * p.tps, tile_end = min(tile_begin + p.tps, ntiles);
    const size_t cslab = (size_t)max(phys, 0) * p.hkv + j;
    const float* kslab = reinterpret_cast<const float*>(p.k) + cslab * p.t_cap * D;
    const float* vslab = reinterpret_cast<const float*>(p.v) + cslab * p.t_cap * D;
    __shared__ float ks[FT][D + 1];
    __shared__ float csum[4][FT];

    // Rows rg + 4k, k < 32: at most 128 window rows on this path, so the
    // per-row state stays in registers.
    constexpr int MAXR = 32;
    float m[MAXR], z[MAXR];
#pragma unroll
    for (int k = 0; k < MAXR; ++k) {
        m[k] = -INFINITY;
        z[k] = 0.f;
    }
    for (int tile = tile_begin; tile < tile_end; ++tile) {
        const int t0 = tile * FT;
        __syncthreads();
        f32_stage_k(ks, kslab, t0, tid, blockDim.x);
        __syncthreads();
        const int t = t0 + tl;
        float c = 0.f;
#pragma unroll
        for (int k = 0; k < MAXR; ++k) {
            const int R = rg + 4 * k;
            if (R >= p.rows) continue;
            const int h = j * p.g + R / p.w, iw = R % p.w;
            const float* q = reinterpret_cast<const float*>(p.q_obs) +
                             (((size_t)iw * p.q_nb + qb) * p.hq + h) * D;
            const float x = f32_dot_row(q, ks, tl) * p.scale;
            const bool vis = t <= T - p.w + iw;
            if (stats_pass) {
                if (vis) {
                    const float mn = fmaxf(m[k], x);
                    z[k] = z[k] * expf(m[k] - mn) + expf(x - mn);
                    m[k] = mn;
                }
            } else if (vis) {
                const float l = p.lse_obs ? p.lse_obs[((size_t)iw * p.q_nb + qb) * p.hq + h]
                                          : p.lse_ws[(size_t)slab * p.rows_pad + R];
                c += expf(x - l);
            }
        }
        if (!stats_pass) {
            csum[rg][tl] = c;
            __syncthreads();
            if (tid < FT && t0 + tid < T) {
                p.score[(size_t)slab * p.t_len + t0 + tid] =
                    csum[0][tid] + csum[1][tid] + csum[2][tid] + csum[3][tid];
                if (p.range) {
                    float mx = -INFINITY, mn = INFINITY;
                    for (int d = 0; d < D; ++d) {
                        const float v = vslab[vt_off(t0 + tid, d)];
                        mx = fmaxf(mx, v);
                        mn = fminf(mn, v);
                    }
                    p.range[(size_t)slab * p.t_len + t0 + tid] = mx - mn;
                }
            }
        }
    }
    if (!stats_pass) return;
    // Merge across the 64 cache-row lanes of each row group; a separate
    // kernel merges the splits.
    float* st = p.stats + ((size_t)slab * p.nsplit + s) * p.rows_pad * 2;
#pragma unroll
    for (int k = 0; k < MAXR; ++k) {
        const int R = rg + 4 * k;
        float mm = m[k], zz = z[k];
        for (int msk = 1; msk < 64; msk <<= 1) {
            const float m2 = __shfl_xor(mm, msk), z2 = __shfl_xor(zz, msk);
            ms_merge(mm, zz, m2, z2);
        }
        if (tl == 0 && R < p.rows) {
            st[R * 2] = mm;
            st[R * 2 + 1] = zz;
        }
    }
}

// Standalone value range: one workgroup of four waves per 512 rows of a
// slab; wave w reduces channels 32w .. 32w+31, lanes own 8 rows each.
template <typename E>
__global__ __launch_bounds__(256) void value_range_kernel(const E* v, int hkv, int t_cap,
                                                          SeqMap sm, float* range) {
    constexpr int VEC = 16 / sizeof(E);          // rows per 16-byte access
    constexpr int ROWS = VEC * WAVE;             // rows per workgroup
    const int b = blockIdx.z;
    const int slab = b * hkv + blockIdx.y;
    const int phys = seq_phys(sm, b);
    const int t_len = seq_rows(sm, b, phys);
    if (blockIdx.x * ROWS >= t_len) return;      // past the sequence's end
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int t0 = blockIdx.x * ROWS + lane * VEC;
    const E* vs = v + ((size_t)phys * hkv + blockIdx.y) * t_cap * D;
    __shared__ float smx[4][ROWS], smn[4][ROWS];
    float mx[VEC], mn[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        mx[e] = -INFINITY;
        mn[e] = INFINITY;
    }
    if (t0 < t_len) {
        for (int d = 32 * wave; d < 32 * wave + 32; ++d) {
            const u32x4 x = load16(vs + vt_off(t0, d));
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                float f;
                if constexpr (sizeof(E) == 2) f = (e & 1) ? bf16hi(x[e / 2]) : bf16lo(x[e / 2]);
                else f = __uint_as_float(x[e]);
                mx[e] = fmaxf(mx[e], f);
                mn[e] = fminf(mn[e], f);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        smx[wave][lane * VEC + e] = mx[e];
        smn[wave][lane * VEC + e] = mn[e];
    }
    __syncthreads();
    for (int x = tid; x < ROWS; x += blockDim.x) {
        const int t = blockIdx.x * ROWS + x;
        if (t < t_len) {
            const float a = fmaxf(fmaxf(smx[0][x], smx[1][x]), fmaxf(smx[2][x], smx[3][x]));
            const float c = fminf(fminf(smn[0][x], smn[1][x]), fminf(smn[2][x], smn[3][x]));
            range[(size_t)slab * sm.t_len + t] = a - c;
        }
    }
}

// Value range of a cache whose values are [t][D] rows (a prefill's layout):
// a group of D / VEC lanes reads one row with 16-byte loads, and the group's
// maximum and minimum meet through lane exchanges inside the group.  Each
// group takes ITER rows of the workgroup's block, every load issued before
// the first reduction.
template <typename E>
__global__ __launch_bounds__(256) void value_range_rows_kernel(const E* v, int hkv, int t_cap,
                                                               SeqMap sm, float* range) {
    constexpr int VEC = 16 / sizeof(E);          // elements per 16-byte access
    constexpr int LPR = D / VEC;                 // lanes per row: 16 (bf16), 32 (float)
    constexpr int RPI = 256 / LPR;               // rows per iteration of the workgroup
    constexpr int ITER = 4;
    const int b = blockIdx.z;
    const int slab = b * hkv + blockIdx.y;
    const int phys = seq_phys(sm, b);
    const int t_len = seq_rows(sm, b, phys);
    const int base = blockIdx.x * RPI * ITER;
    if (base >= t_len) return;                   // past the sequence's end
    const int tid = threadIdx.x, grp = tid / LPR, ln = tid % LPR;
    const E* vs = v + ((size_t)phys * hkv + blockIdx.y) * t_cap * D;
    u32x4 x[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int t = base + it * RPI + grp;
        x[it] = u32x4{0u, 0u, 0u, 0u};
        if (t < t_len) x[it] = load_stream16(vs + (size_t)t * D + ln * VEC);
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        float mx = -INFINITY, mn = INFINITY;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float f;
            if constexpr (sizeof(E) == 2) f = (e & 1) ? bf16hi(x[it][e / 2]) : bf16lo(x[it][e / 2]);
            else f = __uint_as_float(x[it][e]);
            mx = fmaxf(mx, f);
            mn = fminf(mn, f);
        }
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) {      // stays inside the lane group
            mx = fmaxf(mx, __shfl_xor(mx, m));
            mn = fminf(mn, __shfl_xor(mn, m));
        }
        const int t = base + it * RPI + grp;
        if (ln == 0 && t < t_len) range[(size_t)slab * sm.t_len + t] = mx - mn;
    }
}

}  // namespace

hipError_t launch_score(const ScoreLaunch& p, int dtype, hipStream_t st) {
    const dim3 grid(p.nsplit, p.hkv, p.nb);
    if (dtype == 0) {
        if (!p.lse_obs) {
            hipLaunchKernelGGL(score_f32, grid, dim3(256), 0, st, p, 1);
            hipLaunchKernelGGL(score_lse_merge, dim3(p.hkv, p.nb), dim3(1024), 0, st, p);
        }
        hipLaunchKernelGGL(score_f32, grid, dim3(256), 0, st, p, 0);
    } else {
        const int nw = (p.rows + 31) / 32;
        const dim3 mgrid(p.main_nsplit, p.hkv, p.nb);
        const size_t lds = score_main_lds_bytes(p.rows);
        if (!p.lse_obs) {
            const int mt = (p.rows + 15) / 16;
            if (score_stats_tiled(p.rows)) {
                // the statistics pass on the score pass's grid; its staged
                // queries cover the even block count the kernel is built for
                ScoreLaunch q = p;
                q.nsplit = p.main_nsplit;
                q.tps = p.main_tps;
                const size_t lds_st = score_main_lds_bytes(((mt + 1) / 2) * 32);
                hipError_t e = hipErrorInvalidValue;
                auto go_stats = [&](auto kern) {
                    if (lds_st > 64 * 1024 &&
                        hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                            hipFuncAttributeMaxDynamicSharedMemorySize,
                                            (int)lds_st) != hipSuccess)
                        return hipErrorInvalidValue;
                    hipLaunchKernelGGL(kern, mgrid, dim3(256), lds_st, st, q);
                    return hipSuccess;
                };
                switch ((mt + 1) / 2) {   // MT rounded up to even: padding blocks see nothing
                    case 1: e = go_stats(score_stats_tiles_bf16<2>); break;
                    case 2: e = go_stats(score_stats_tiles_bf16<4>); break;
                    case 3: e = go_stats(score_stats_tiles_bf16<6>); break;
                    case 4: e = go_stats(score_stats_tiles_bf16<8>); break;
                    case 5: e = go_stats(score_stats_tiles_bf16<10>); break;
                    case 6: e = go_stats(score_stats_tiles_bf16<12>); break;
                    case 7: e = go_stats(score_stats_tiles_bf16<14>); break;
                    default: e = go_stats(score_stats_tiles_bf16<16>); break;
                }
                if (e != hipSuccess) return e;
                hipLaunchKernelGGL(score_lse_merge, dim3(p.hkv, p.nb), dim3(1024), 0, st, q);
            } else {
                if (nw <= 8)
                    hipLaunchKernelGGL(score_stats_bf16<1>, grid, dim3(nw * WAVE), 0, st, p);
                else
                    hipLaunchKernelGGL(score_stats_bf16<0>, grid, dim3(nw * WAVE), 0, st, p);
                hipLaunchKernelGGL(score_lse_merge, dim3(p.hkv, p.nb), dim3(1024), 0, st, p);
            }
        }
        auto go = [&](auto kern) {
            if (lds > 64 * 1024 &&
                hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
                return hipErrorInvalidValue;
            hipLaunchKernelGGL(kern, mgrid, dim3(256), lds, st, p);
            return hipSuccess;
        };
        if ((p.range ? go(score_main_bf16<true>) : go(score_main_bf16<false>)) != hipSuccess)
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_value_range(const void* v, bool v_rows, int nb, int hkv, int t_cap,
                              const SeqMap& sm, int dtype, float* range, hipStream_t st) {
    if (v_rows) {
        const int rows_per_wg = (dtype == 0 ? 8 : 16) * 4;
        const dim3 grid((sm.t_len + rows_per_wg - 1) / rows_per_wg, hkv, nb);
        if (dtype == 0)
            hipLaunchKernelGGL(value_range_rows_kernel<float>, grid, dim3(256), 0, st,
                               (const float*)v, hkv, t_cap, sm, range);
        else
            hipLaunchKernelGGL(value_range_rows_kernel<uint16_t>, grid, dim3(256), 0, st,
                               (const uint16_t*)v, hkv, t_cap, sm, range);
        return hipGetLastError();
    }
    if (dtype == 0) {
        const dim3 grid((sm.t_len + 4 * WAVE - 1) / (4 * WAVE), hkv, nb);
        hipLaunchKernelGGL(value_range_kernel<float>, grid, dim3(256), 0, st, (const float*)v, hkv,
                           t_cap, sm, range);
    } else {
        const dim3 grid((sm.t_len + 8 * WAVE - 1) / (8 * WAVE), hkv, nb);
        hipLaunchKernelGGL(value_range_kernel<uint16_t>, grid, dim3(256), 0, st,
                           (const uint16_t*)v, hkv, t_cap, sm, range);
    }
    return hipGetLastError();
}

}  // namespace kvc
