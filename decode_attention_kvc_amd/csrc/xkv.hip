// Cross-layer factorisation and selective reconstruction (xKV).
//
// xKV summary (gist.science 2503.18893), §2.2: the caches of W consecutive
// layers are concatenated side by side and a rank-r SVD gives one token basis
// A shared by the window and one reconstruction matrix B_l per layer; §2.3:
// at decode only the rows of the chunks whose landmarks score best against
// the query are rebuilt from A and B_l and attended.
//
// Factorisation, per (keys or values, batch entry b, KV head j), of
// X = [X_1 | ... | X_W] (T x n, n = W * 128):
//  1. xkv_gram: G = X^T X on v_mfma_f32_16x16x32_bf16, one workgroup per
//     pair of layers (I <= J) streaming the rows once; each 32-row tile of
//     both layers is staged in LDS channel-major (key rows are transposed on
//     the way in, value tiles already are), so both operands are 16-byte
//     reads.  Rows past t_len are staged as zeros.
//  2. xkv_subspace: one workgroup per problem runs `iters` steps of subspace
//     iteration on G from a Gaussian start (Box-Muller on Philox words):
//     Z = G V on v_mfma_f32_16x16x4f32 (the A operand is read along G's rows,
//     which G's symmetry allows), then modified Gram-Schmidt in LDS (twice
//     after the last step).  V (n x r, orthonormal columns) converges to the
//     top-r right singular subspace of X; X V V^T is the rank-r truncation,
//     A = X V and B_l = (rows l*128 .. l*128+127 of V)^T.
//  3. xkv_project: A = X V on MFMA with V^T as bf16 in LDS, stored as bf16,
//     and for keys the landmark of every 8-row chunk: the mean of its stored
//     A rows.
// Decode, one launch with one workgroup per (b, j) (section 4): q~_h = B_l q_h
// (r numbers per head); the chunk scores max_h q~_h . landmark on MFMA; the
// exact top-k of the chunks (ties to the lower chunk); attention over the
// kept rows in the rank space, q_h . (A_t B_l) = q~_h . A_t and
// sum_t p_t A_t B_l = (sum_t p_t A_t) B_l, so the selected rows are rebuilt
// implicitly and never written; the output projected by B_l^V and merged
// with an optional second part (rows appended after the factorisation,
// attended separately) by log-sum-exp weights.  The value basis is stored
// chunk-transposed (av_off) for the rank-space P*V product.
#include <algorithm>

#include "common.h"
#include "kvc_internal.h"
#include "merge.h"
#include "philox.h"
#include "radix.h"

namespace kvc {

namespace {

constexpr int XT = 32;          // rows per tile
constexpr int GP = 40;          // bf16 per staged channel row of a tile (80 bytes)
constexpr int CHUNK = 8;        // rows per landmark chunk
constexpr int VPITCH = XT + 2;  // bf16 per channel in a wave's value transpose buffer
constexpr int MAXG = 8;         // query heads per KV head on the decode path
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// ---------------------------------------------------------------------------
// 1. Gram matrix
// ---------------------------------------------------------------------------
template <bool IS_V>
__global__ __launch_bounds__(256) void xkv_gram(XkvLaunch p) {
    __shared__ __align__(16) uint16_t st[2][D * GP];
    const int j = blockIdx.y, b = blockIdx.z;
    int I = 0, J = 0;
    {
        int q = blockIdx.x;
        for (int a = 0; a < p.window; ++a) {
            if (q < p.window - a) {
                I = a;
                J = a + q;
                break;
            }
            q -= p.window - a;
        }
    }
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int l16 = lane & 15, lg = lane >> 4;
    const size_t cs = ((size_t)b * p.hkv + j) * p.t_cap * D;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(IS_V ? p.v : p.k);
    const uint16_t* xI = src + (size_t)I * p.slot_stride + cs;
    const uint16_t* xJ = src + (size_t)J * p.slot_stride + cs;
    const int T = p.t_len, n = p.window * D;
    const int nside = (I == J) ? 1 : 2;

    f32x4 acc[2][8];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) acc[ib][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ntiles = (T + XT - 1) / XT;
    for (int tile = 0; tile < ntiles; ++tile) {
        const int t0 = tile * XT;
        for (int side = 0; side < nside; ++side) {
            const uint16_t* x = side ? xJ : xI;
            uint16_t* dst = st[side];
#pragma unroll
            for (int u = 0; u < 2; ++u) {          // 512 16-byte pieces of the 8 KB tile
                const int c = tid + 256 * u;
                if constexpr (IS_V) {
                    const int ch = c >> 2, q4 = c & 3;    // channel, 8-row group
                    u32x4 v = load_stream16(x + vt_off(t0, ch) + 8 * q4);
                    if (t0 + 8 * q4 + 8 > T) {
                        u16x8 e = __builtin_bit_cast(u16x8, v);
#pragma unroll
                        for (int k = 0; k < 8; ++k) e[k] = (t0 + 8 * q4 + k < T) ? e[k] : (uint16_t)0;
                        v = __builtin_bit_cast(u32x4, e);
                    }
                    *reinterpret_cast<u32x4*>(dst + ch * GP + 8 * q4) = v;
                } else {
                    // a wave writes 32 consecutive rows of each channel: no
                    // two lanes of a write share an LDS bank
                    const int r = c & 31, c8 = (c >> 5) * 8;   // row, first channel
                    u32x4 v = u32x4{0u, 0u, 0u, 0u};
                    if (t0 + r < T) v = load_stream16(x + (size_t)(t0 + r) * D + c8);
                    const u16x8 e = __builtin_bit_cast(u16x8, v);
#pragma unroll
                    for (int k = 0; k < 8; ++k) dst[(c8 + k) * GP + r] = e[k];
                }
            }
        }
        __syncthreads();
        const uint16_t* sI = st[0];
        const uint16_t* sJ = st[nside - 1];
        bf16x8 a[2], bb[8];
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
            a[ib] = as_bf(*reinterpret_cast<const u32x4*>(sI + (32 * wave + 16 * ib + l16) * GP + 8 * lg));
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
            bb[jb] = as_bf(*reinterpret_cast<const u32x4*>(sJ + (16 * jb + l16) * GP + 8 * lg));
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int jb = 0; jb < 8; ++jb)
                acc[ib][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ib], bb[jb], acc[ib][jb], 0, 0, 0);
        __syncthreads();
    }
    // acc[ib][jb][i]: G[I*128 + 32*wave + 16*ib + 4*lg + i][J*128 + 16*jb + l16]
    float* G = p.gram + ((size_t)((IS_V ? p.nb : 0) + b) * p.hkv + j) * n * n;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 8; ++jb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = I * D + 32 * wave + 16 * ib + 4 * lg + i;
                const int col = J * D + 16 * jb + l16;
                G[(size_t)row * n + col] = acc[ib][jb][i];
                if (I != J) G[(size_t)col * n + row] = acc[ib][jb][i];
            }
}

// ---------------------------------------------------------------------------
// 2. Subspace iteration
// ---------------------------------------------------------------------------
// Modified Gram-Schmidt on the R columns of Z ([n][R + 1] floats in LDS), one
// column at a time: normalise it (a column of norm 0 stays 0), then remove it
// from the later columns (wave w takes columns j+1+w, j+5+w, ...).
template <int R>
__device__ void mgs(float* Z, int n, float* red) {
    constexpr int RP = R + 1;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    for (int j = 0; j < R; ++j) {
        float s = 0.f;
        for (int i = tid; i < n; i += 256) {
            const float z = Z[i * RP + j];
            s = fmaf(z, z, s);
        }
        s = wave_sum(s);
        if (lane == 0) red[wave] = s;
        __syncthreads();
        const float nrm2 = (red[0] + red[1]) + (red[2] + red[3]);
        const float inv = nrm2 > 1e-30f ? 1.0f / sqrtf(nrm2) : 0.f;
        for (int i = tid; i < n; i += 256) Z[i * RP + j] *= inv;
        __syncthreads();
        for (int k = j + 1 + wave; k < R; k += 4) {
            float d = 0.f;
            for (int i = lane; i < n; i += WAVE) d = fmaf(Z[i * RP + j], Z[i * RP + k], d);
            d = wave_sum(d);
            for (int i = lane; i < n; i += WAVE) Z[i * RP + k] = fmaf(-d, Z[i * RP + j], Z[i * RP + k]);
        }
        __syncthreads();
    }
}

template <int R>
__global__ __launch_bounds__(256) void xkv_subspace(XkvLaunch p) {
    extern __shared__ float Zs[];          // [n][R + 1]
    __shared__ float red[4];
    constexpr int RP = R + 1;
    constexpr int CB = R / 16;
    const int prob = blockIdx.x;           // (keys, values) x nb x hkv
    const int n = p.window * D;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int l16 = lane & 15, lg = lane >> 4;
    const float* G = p.gram + (size_t)prob * n * n;

    // Gaussian start: element x from words 0, 1 of Philox4x32-10 at counter
    // (x, problem, 0x786b76, 0) under the caller's seed.
    for (int x = tid; x < n * R; x += 256) {
        const Philox4 w = philox4x32_10((uint32_t)x, (uint32_t)prob, 0x786b76u, 0u, p.seed_lo,
                                        p.seed_hi);
        const float u1 = ((float)w.x0 + 1.0f) * 2.3283064365386963e-10f;
        const float u2 = (float)w.x1 * 2.3283064365386963e-10f;
        Zs[(x / R) * RP + x % R] = sqrtf(-2.0f * logf(u1)) * cosf(6.283185307179586f * u2);
    }
    __syncthreads();
    mgs<R>(Zs, n, red);

    const int nib = n / 16;                // 16-row blocks of Z; wave w owns w, w+4, ...
    for (int it = 0; it < p.iters; ++it) {
        f32x4 acc[8][CB];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) acc[u][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // four k-steps per round: their 32 G loads are issued together
        for (int k0 = 0; k0 < n; k0 += 16) {
            float ga[4][8];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float* grow = G + (size_t)(k0 + 4 * kk + lg) * n;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int ib = wave + 4 * u;
                    ga[kk][u] = ib < nib ? grow[16 * ib + l16] : 0.f;   // G[16ib + l16][k] by symmetry
                }
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                float bv[CB];
#pragma unroll
                for (int cb = 0; cb < CB; ++cb) bv[cb] = Zs[(k0 + 4 * kk + lg) * RP + 16 * cb + l16];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (wave + 4 * u < nib) {
#pragma unroll
                        for (int cb = 0; cb < CB; ++cb)
                            acc[u][cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[kk][u], bv[cb],
                                                                              acc[u][cb], 0, 0, 0);
                    }
                }
            }
        }
        __syncthreads();                   // every wave is done reading V
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int ib = wave + 4 * u;
            if (ib < nib) {
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Zs[(16 * ib + 4 * lg + i) * RP + 16 * cb + l16] = acc[u][cb][i];
            }
        }
        __syncthreads();
        mgs<R>(Zs, n, red);
        if (it == p.iters - 1) mgs<R>(Zs, n, red);
    }

    const int slabs = p.nb * p.hkv;
    const bool is_v = prob >= slabs;
    float* out = (is_v ? p.bv : p.bk) + (size_t)(prob % slabs) * n * R;
    uint16_t* vt = p.vt + (size_t)prob * R * n;
    for (int x = tid; x < n * R; x += 256) {
        const int i = x / R, c = x % R;
        const float v = Zs[i * RP + c];
        out[x] = v;
        vt[(size_t)c * n + i] = f32_to_bf16(v);
    }
}

// Element of the value basis A_V[t][c] in its chunk-transposed layout
// [t / 8][c][t % 8]: the 8 rows of a chunk for one rank are 16 contiguous
// bytes, the operand layout of the decode's a~^T = A_V^T P^T product.
template <int R>
__host__ __device__ __forceinline__ size_t av_off(int t, int c) {
    return (size_t)(t / CHUNK) * (R * CHUNK) + (size_t)c * CHUNK + (t % CHUNK);
}

// ---------------------------------------------------------------------------
// 3. Projection A = X V and key landmarks
// ---------------------------------------------------------------------------
template <bool IS_V, int R>
__global__ __launch_bounds__(256) void xkv_project(XkvLaunch p) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int CB = R / 16;
    const int n = p.window * D, vtp = n + 8;
    uint16_t* vts = reinterpret_cast<uint16_t*>(smem);          // [R][vtp] bf16 V^T
    uint16_t* tbuf = vts + R * vtp;                              // values: [4][D * VPITCH]
    const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int slab = b * p.hkv + j;
    const int prob = (IS_V ? p.nb * p.hkv : 0) + slab;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int l16 = lane & 15, lg = lane >> 4;

    const uint16_t* vt = p.vt + (size_t)prob * R * n;
    for (int x = tid; x < R * (n / 8); x += 256) {
        const int c = x / (n / 8), q = x % (n / 8);
        *reinterpret_cast<u32x4*>(vts + c * vtp + 8 * q) = load16(vt + (size_t)c * n + 8 * q);
    }
    __syncthreads();

    const uint16_t* src = reinterpret_cast<const uint16_t*>(IS_V ? p.v : p.k) +
                          ((size_t)b * p.hkv + j) * p.t_cap * D;
    uint16_t* A = reinterpret_cast<uint16_t*>(IS_V ? p.av : p.ak) + (size_t)slab * p.x_tcap * R;
    uint16_t* L = reinterpret_cast<uint16_t*>(p.lk) + (size_t)slab * (p.x_tcap / CHUNK) * R;
    uint16_t* vb = tbuf + wave * D * VPITCH;
    const int T = p.t_len;
    const int ntiles = (T + XT - 1) / XT;
    const int tile_begin = s * p.tps, tile_end = min(tile_begin + p.tps, ntiles);

    for (int tile = tile_begin + wave; tile < tile_end; tile += 4) {
        const int t0 = tile * XT;
        f32x4 Y[2][CB];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) Y[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int l = 0; l < p.window; ++l) {
            const uint16_t* x = src + (size_t)l * p.slot_stride;
            // A operand: row t0 + 16*rb + l16, channels 32*kc + 8*lg .. +8
            u32x4 xa[2][4];
            if constexpr (!IS_V) {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int kc = 0; kc < 4; ++kc)
                        xa[rb][kc] = load_stream16(x + (size_t)(t0 + 16 * rb + l16) * D + 32 * kc + 8 * lg);
            } else {
                // the value tile is channel-major: through the wave's LDS
                // buffer (one wave's LDS accesses execute in issue order)
                u32x4 vtl[8];
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
                    vtl[dt] = load_stream16(x + vt_off(t0, 16 * dt + l16) + 8 * lg);
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    uint32_t* dst = reinterpret_cast<uint32_t*>(vb + (16 * dt + l16) * VPITCH + 8 * lg);
#pragma unroll
                    for (int w2 = 0; w2 < 4; ++w2) dst[w2] = vtl[dt][w2];
                }
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int kc = 0; kc < 4; ++kc) {
                        u16x8 e;
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj)
                            e[jj] = vb[(32 * kc + 8 * lg + jj) * VPITCH + 16 * rb + l16];
                        xa[rb][kc] = __builtin_bit_cast(u32x4, e);
                    }
                __builtin_amdgcn_wave_barrier();
            }
#pragma unroll
            for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
                    const bf16x8 gb = as_bf(*reinterpret_cast<const u32x4*>(
                        vts + (16 * cb + l16) * vtp + l * D + 32 * kc + 8 * lg));
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
                        Y[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(xa[rb][kc]), gb,
                                                                            Y[rb][cb], 0, 0, 0);
                }
        }
        // Y[rb][cb][i]: row t0 + 16*rb + 4*lg + i, column 16*cb + l16.  Rows
        // past t_len (arbitrary cache bits) become zeros and are not stored.
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                float sum = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = t0 + 16 * rb + 4 * lg + i;
                    const uint16_t h = f32_to_bf16(t < T ? Y[rb][cb][i] : 0.f);
                    if (t < T) A[IS_V ? av_off<R>(t, 16 * cb + l16) : (size_t)t * R + 16 * cb + l16] = h;
                    sum += bf16_to_f32(h);
                }
                if constexpr (!IS_V) {
                    // chunk 2*rb + (lg >> 1) of the tile: lanes lg = 2h, 2h+1
                    sum += __shfl_xor(sum, 16);
                    const int chunk = t0 / CHUNK + 2 * rb + (lg >> 1);
                    const int cnt = min(CHUNK, T - chunk * CHUNK);
                    if ((lg & 1) == 0 && cnt > 0)
                        L[(size_t)chunk * R + 16 * cb + l16] = f32_to_bf16(sum / (float)cnt);
                }
            }
    }
}

// ---------------------------------------------------------------------------
// 4. Selective-reconstruction decode attention
// ---------------------------------------------------------------------------
// Ascending key for descending score (order-preserving float bits, inverted).
__device__ __forceinline__ uint32_t desc_key(float s) {
    const uint32_t u = __float_as_uint(s);
    const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ~asc;
}

// The k smallest of n keys (ties to the lower index), described as a masked
// prefix: key u is kept when (u & mask) < prefix, or when (u & mask) ==
// prefix and it is among the first *take such keys in index order (*cnt of
// them exist; take == cnt keeps them all).  The first digit is the top 11
// bits of the key, whose histogram the caller builds in sm.hist (2048 bins,
// one copy) while it stores the keys; further digits of 8 bits (LDS
// histograms in NC copies) follow only while the bin holding the k-th key
// is not kept whole, so score keys usually resolve in one more pass.
// 1 <= k <= n; every thread of the block must call it.
constexpr int TOPK_B0 = 11;
template <int NT, int NC>
__device__ void topk_prefix(const uint32_t* keys, int n, uint32_t k, RadixSmem<NT, NC>& sm,
                            uint32_t* prefix_out, uint32_t* mask_out, uint32_t* take_out,
                            uint32_t* cnt_out) {
    constexpr int PITCH = RadixSmem<NT, NC>::PITCH;
    constexpr int BPL = (1 << TOPK_B0) / NT;     // first-digit bins per thread
    static_assert(BPL >= 1 && NC * PITCH >= (1 << TOPK_B0), "first-digit histogram");
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    {
        uint32_t c[BPL], s = 0;
#pragma unroll
        for (int e = 0; e < BPL; ++e) {
            c[e] = sm.hist[tid * BPL + e];
            s += c[e];
        }
        const uint32_t incl = wave_incl_scan(s);
        if (lane == WAVE - 1) sm.wave_tot[wave] = incl;
        __syncthreads();
        uint32_t run = incl - s;
        for (int w = 0; w < wave; ++w) run += sm.wave_tot[w];
#pragma unroll
        for (int e = 0; e < BPL; ++e) {
            if (run < k && k <= run + c[e]) {
                sm.bcast[0] = tid * BPL + e;
                sm.bcast[1] = run;
                sm.bcast[2] = c[e];
            }
            run += c[e];
        }
        __syncthreads();
    }
    uint32_t cnt = sm.bcast[2];
    k -= sm.bcast[1];
    int shift = 32 - TOPK_B0;
    uint32_t prefix = sm.bcast[0] << shift, mask = ~((1u << shift) - 1u);
    while (cnt != k && shift > 0) {
        const int width = min(8, shift);
        shift -= width;
        // the first-digit histogram and bcast were read before the last barrier
        for (int i = tid; i < NC * PITCH; i += NT) sm.hist[i] = 0;
        __syncthreads();
        uint32_t* hist = sm.hist + (tid % NC) * PITCH;
        const uint32_t dmask = (1u << width) - 1u;
        for (int t = tid; t < n; t += NT) {
            const uint32_t u = keys[t];
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1u);
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
            uint32_t run = wave_incl_scan(s) - s;
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
        k -= sm.bcast[1];
        cnt = sm.bcast[2];
        prefix |= sm.bcast[0] << shift;
        mask |= dmask << shift;
    }
    *prefix_out = prefix;
    *mask_out = mask;
    *take_out = k;
    *cnt_out = cnt;
}

constexpr int XF_NT = 1024;            // threads of a decode row workgroup
constexpr int XF_NW = XF_NT / WAVE;
constexpr int XS_NT = 512;             // threads of a decode score workgroup

// x ~ hi + lo with both parts in bf16 (about 16 significant bits).
__device__ __forceinline__ void split_bf16(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
    u16x8 h, l;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = f32_to_bf16(x[e]);
        l[e] = f32_to_bf16(x[e] - bf16_to_f32(h[e]));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Hand-off between the workgroups of one launch without a cache writeback:
// partials are written with agent-scope stores (through to the device's
// coherence point), every store is complete (vmcnt 0) before the workgroup
// counts itself in, and the last workgroup to arrive reads the partials with
// agent-scope loads, which do not hit a stale line of its own XCD's L2; the
// counted arrival (arrive_last) is the one of the split-K attention merge,
// and the last workgroup returns the counter to zero for the next launch.
__device__ __forceinline__ void st_coh(float* a, float x) {
    __hip_atomic_store(a, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coh(const float* a) {
    return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// LDS floats of the score launch: B_l^K [D][R], the queries [MAXG][D], q~
// [MAXG][R] and the partial sums of q~ [NT].
__host__ __device__ constexpr int xs_floats(int r) {
    return D * r + MAXG * D + MAXG * r + (XS_NT > MAXG * r ? XS_NT : MAXG * r);
}
// LDS floats of the row launch besides the kept chunks and (when they fit)
// the chunk keys: B_l^V rows [D][R + 1], the waves' partials [NW][MAXG][R + 2],
// a~ [MAXG][R].
__host__ __device__ constexpr int xr_floats(int r) {
    return D * (r + 1) + XF_NW * MAXG * (r + 2) + MAXG * r;
}

// Decode, first launch, grid (split, j, b), 1024 threads: the chunk score
// keys of split s's share of the (b, j) landmarks (contiguous runs of
// 16-chunk blocks).
//  0. B_l^K and the queries are read (every wave's reads queued before the
//     landmark stream), then the first round of landmark rows;
//  1. q~_h = B_l q_h (from LDS), held as bf16 hi + lo fragments: for 16x32
//     operands the A fragment of q~ (heads x ranks) and the B fragment of
//     q~^T (ranks x heads) are the same registers; split 0 stores q~ in the
//     workspace for the second launch;
//  2. chunk scores S = q~ L^T on v_mfma_f32_16x16x32_bf16, 16 chunks per
//     product (heads padded to 16), max over the heads, order-preserving keys
//     into the workspace.
template <int R>
__global__ __launch_bounds__(XS_NT) void xkv_scores(XkvDecodeLaunch p) {
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NT = XS_NT, NW = XS_NT / WAVE;
    constexpr int KS = R / 32;           // 32-rank k-steps
    constexpr int UNB = 32 / NW;         // 16-chunk landmark blocks per wave and round
    constexpr int BPT = D * R / 4 / NT;  // float4 per thread of one B matrix
    constexpr int NPART = NT > MAXG * R ? NT / (MAXG * R) : 1;   // threads per (head, rank)
    constexpr int QX = MAXG * R * NPART; // (part, head, rank) items of q~
    constexpr int QPT = MAXG * D / NT;    // query elements per thread
    static_assert(UNB * NW == 32 && BPT >= 1 && D % NPART == 0 && QPT * NT == MAXG * D, "launch shape");
    const int sp = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int slab = b * p.hkv + j, g = p.g;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int l16 = lane & 15, lg = lane >> 4;
    const int T = p.t_len, nch = (T + CHUNK - 1) / CHUNK;
    const int n = p.window * D;
    const int nlb = (nch + 15) / 16;                              // 16-chunk blocks
    const int per = (nlb + p.ns - 1) / p.ns;
    const int lb0 = sp * per, nl = max(0, min(nlb, lb0 + per) - lb0);   // this split's blocks
    const int nlr = (nl + NW * UNB - 1) / (NW * UNB);             // rounds

    float* area = reinterpret_cast<float*>(smem);                 // B_l^K [D][R]
    float* qs = area + D * R;                                     // [MAXG][D] queries
    float* qt = qs + MAXG * D;                                    // [MAXG][R] q~
    float* qpart = qt + MAXG * R;                                 // [QX] partial sums of q~
    uint32_t* keys = p.ws_keys + (size_t)slab * nch;

    // 0. global reads
    const float* BK = p.bk + (size_t)slab * n * R + (size_t)p.layer * D * R;
    f32x4 bkr[BPT];
#pragma unroll
    for (int e = 0; e < BPT; ++e) bkr[e] = *reinterpret_cast<const f32x4*>(BK + 4 * (tid + e * NT));
    const size_t row0 = (size_t)b * p.hq + (size_t)j * g;        // first query row of (b, j)
    // query element tid + e NT is (head / D, channel % D); loads are
    // unconditional (clamped addresses, results selected after), so that the
    // compiler's wait counts cover only the older loads
    uint16_t qraw[QPT];
#pragma unroll
    for (int e = 0; e < QPT; ++e) {
        const int i = tid + e * NT;
        qraw[e] = reinterpret_cast<const uint16_t*>(p.q)[row0 * D + (i < g * D ? i : 0)];
    }
    // every wave's reads for q~ are queued ahead of the landmark stream
    __syncthreads();
    const uint16_t* L = reinterpret_cast<const uint16_t*>(p.lk) + (size_t)slab * (p.x_tcap / CHUNK) * R;
    // B fragment of L^T: chunk 16 blk + l16, ranks 32 ks + 8 lg .. +8
    auto chunk_of = [&](int r, int u) { return (lb0 + (r * UNB + u) * NW + wave) * 16 + l16; };
    auto in_split = [&](int r, int u) { return (r * UNB + u) * NW + wave < nl; };
    auto load_lm = [&](u32x4 (&w)[UNB][KS], int r) {
#pragma unroll
        for (int u = 0; u < UNB; ++u) {
            const int ch = chunk_of(r, u);
            const int chc = in_split(r, u) && ch < nch ? ch : 0;   // lk holds t_cap / 8 >= 8 rows
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) w[u][ks] = load16(L + (size_t)chc * R + 32 * ks + 8 * lg);
        }
    };
    u32x4 la[UNB][KS], lb[UNB][KS];
    load_lm(la, 0);
#pragma unroll
    for (int e = 0; e < BPT; ++e) *reinterpret_cast<f32x4*>(area + 4 * (tid + e * NT)) = bkr[e];
#pragma unroll
    for (int e = 0; e < QPT; ++e) {
        const int i = tid + e * NT;
        qs[i] = i < g * D ? bf16_to_f32(qraw[e]) : 0.f;
    }
    __syncthreads();

    // 1. q~ (NPART parts per (head, rank), contiguous channel ranges)
    for (int x = tid; x < QX; x += NT) {
        const int c = x % R, h = (x / R) % MAXG, part = x / (MAXG * R);
        constexpr int IPP = D / NPART;
        float a = 0.f;
        if (h < g)
            for (int i = part * IPP; i < (part + 1) * IPP; ++i) a = fmaf(qs[h * D + i], area[i * R + c], a);
        qpart[x] = a;
    }
    __syncthreads();
    for (int x = tid; x < MAXG * R; x += NT) {
        float a = 0.f;
#pragma unroll
        for (int part = 0; part < NPART; ++part) a += qpart[part * MAXG * R + x];
        qt[x] = a;
        if (sp == 0) p.ws_qt[(size_t)slab * MAXG * R + x] = a;
    }
    __syncthreads();
    bf16x8 qh[KS], ql[KS];               // head l16, ranks 32 ks + 8 lg .. +8
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = l16 < MAXG ? qt[l16 * R + 32 * ks + 8 * lg + e] : 0.f;
        split_bf16(x, qh[ks], ql[ks]);
    }

    load_lm(lb, 1);                     // the second round once q~'s reads are in
    // 2. chunk score keys
    auto score_lm = [&](const u32x4 (&w)[UNB][KS], int r) {
#pragma unroll
        for (int u = 0; u < UNB; ++u) {
            f32x4 S = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh[ks], as_bf(w[u][ks]), S, 0, 0, 0);
                S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql[ks], as_bf(w[u][ks]), S, 0, 0, 0);
            }
            // S[i]: head 4 lg + i, chunk 16 blk + l16
            float best = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * lg + i < g) best = fmaxf(best, S[i]);
            best = fmaxf(best, __shfl_xor(best, 16));            // heads 4..7 into lanes lg = 0
            const int ch = chunk_of(r, u);
            if (lg == 0 && in_split(r, u) && ch < nch) keys[ch] = desc_key(best);
        }
    };
    // Branch-free rounds: a round past the last one loads row 0 of the
    // landmarks in every lane (one cached line) and writes no key, so the
    // wait counts stay exact and one round is always in flight.
    for (int r = 0; r < nlr; r += 2) {
        score_lm(la, r);
        load_lm(la, r + 2);
        score_lm(lb, r + 1);
        load_lm(lb, r + 3);
    }
}

// Decode, second launch, grid (split, j, b), 1024 threads:
//  3. the chunk keys of (b, j) are read (into LDS when they fit) while their
//     first digit is counted, and the exact top-k of the keys (topk_prefix)
//     is emitted in chunk order, by every split alike;
//  4. per 32 kept rows (4 chunks; blocks split, split + ns, ... are this
//     split's): S^T = A_K q~^T with the kept rows loaded in the order that
//     makes each lane's S^T fragment its P^T operand (the 8 rows of chunk
//     lg), an online softmax whose reference maximum moves only when a
//     logit exceeds it by more than 8 (log2 units), P split into bf16 hi +
//     lo, and a~^T += A_V^T P^T, A_V stored chunk-transposed
//     ([chunk][rank][8 rows]) so that the A operand is one 16-byte load;
//  5. the waves' (reference, sum, a~) merge through LDS into the split's
//     partial; the last split of (b, j) to finish merges the partials, forms
//     o_h = B_l^V a~_h / z_h per (head, channel) and merges it with the
//     second part when one is given.
template <int R, bool GKEYS>
__global__ __launch_bounds__(XF_NT) void xkv_rows(XkvDecodeLaunch p) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ RadixSmem<XF_NT, 8> rs;
    __shared__ float hz[MAXG], hm[MAXG];
    constexpr int NT = XF_NT, NW = XF_NW;
    constexpr int KS = R / 32;           // 32-rank k-steps
    constexpr int RBK = R / 16;          // 16-rank blocks of a~^T
    constexpr int BVP = R + 1;           // float pitch of the staged B_l^V rows
    constexpr int PP = MAXG * (R + 2);   // floats of one split's partial
    static_assert(MAXG * D == NT, "launch shape");
    const int sp = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int slab = b * p.hkv + j, g = p.g, ns = p.ns;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int l16 = lane & 15, lg = lane >> 4;
    const int T = p.t_len, nch = (T + CHUNK - 1) / CHUNK;
    const int ksel = min(p.n_select, nch);
    const int n = p.window * D;

    float* bvs = reinterpret_cast<float*>(smem);                  // [D][R + 1]
    float* wp = bvs + D * BVP;                                    // [NW][MAXG][R + 2]
    float* qt = wp + NW * PP;                                     // [MAXG][R] a~
    int32_t* sel = reinterpret_cast<int32_t*>(qt + MAXG * R);     // [ksel] kept chunks
    const uint32_t* gkeys = p.ws_keys + (size_t)slab * nch;
    uint32_t* lkeys = reinterpret_cast<uint32_t*>(sel + ksel);    // [nch] when !GKEYS
    const uint32_t* keys = GKEYS ? gkeys : lkeys;

    // q~ fragments (head l16, ranks 32 ks + 8 lg .. +8) from the first launch
    bf16x8 qh[KS], ql[KS];
    {
        const float* qg = p.ws_qt + (size_t)slab * MAXG * R;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            float x[8];
            const int hh = l16 < MAXG ? l16 : 0;
            const f32x4 x0 = *reinterpret_cast<const f32x4*>(qg + hh * R + 32 * ks + 8 * lg);
            const f32x4 x1 = *reinterpret_cast<const f32x4*>(qg + hh * R + 32 * ks + 8 * lg + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = l16 < MAXG ? x0[e] : 0.f;
                x[4 + e] = l16 < MAXG ? x1[e] : 0.f;
            }
            split_bf16(x, qh[ks], ql[ks]);
        }
    }

    // 3. the ksel best chunks in ascending chunk order (all of them when
    // there are fewer): thread t owns chunks [t*per, (t+1)*per)
    if (ksel < nch) {
        for (int i = tid; i < (1 << TOPK_B0); i += NT) rs.hist[i] = 0;
        __syncthreads();
        for (int ch = tid; ch < nch; ch += NT) {
            const uint32_t key = gkeys[ch];
            if constexpr (!GKEYS) lkeys[ch] = key;
            atomicAdd(&rs.hist[key >> (32 - TOPK_B0)], 1u);
        }
        __syncthreads();
        uint32_t prefix, mask, take, cnt;
        topk_prefix<NT, 8>(keys, nch, (uint32_t)ksel, rs, &prefix, &mask, &take, &cnt);
        const int per = (nch + NT - 1) / NT;
        const int c0 = min(nch, tid * per), c1 = min(nch, c0 + per);
        // ranks among the keys equal to the prefix, needed only when some of
        // them are left out (the condition is the same in every thread)
        uint32_t eq0 = 0, tot;
        if (take != cnt) {
            uint32_t n_eq = 0;
            for (int ch = c0; ch < c1; ++ch) n_eq += (keys[ch] & mask) == prefix;
            eq0 = block_scan_u32<NT>(n_eq, rs, &tot);
        }
        auto kept = [&](uint32_t u, uint32_t& eq_rank) {
            const uint32_t um = u & mask;
            return (um < prefix) || (um == prefix && eq_rank++ < take);
        };
        uint32_t eq_rank = eq0, n_keep = 0;
        for (int ch = c0; ch < c1; ++ch) n_keep += kept(keys[ch], eq_rank);
        eq_rank = eq0;
        uint32_t pos = block_scan_u32<NT>(n_keep, rs, &tot);
        for (int ch = c0; ch < c1; ++ch) {
            if (kept(keys[ch], eq_rank)) {
                if (pos < (uint32_t)ksel) sel[pos] = ch;
                ++pos;
            }
        }
    } else {
        for (int ch = tid; ch < nch; ch += NT) sel[ch] = ch;
    }
    __syncthreads();
    if (p.selected && sp == 0)
        for (int x = tid; x < p.n_select; x += NT)
            p.selected[(size_t)slab * p.n_select + x] = x < ksel ? sel[x] : -1;

    // 4. kept rows, 32 (4 chunks) per block; block k is split k % ns's
    const uint16_t* AK = reinterpret_cast<const uint16_t*>(p.ak) + (size_t)slab * p.x_tcap * R;
    const uint16_t* AV = reinterpret_cast<const uint16_t*>(p.av) + (size_t)slab * p.x_tcap * R;
    const float scale2 = p.scale * LOG2E;
    const int nblk = (ksel + 3) / 4;
    struct RowRegs {
        u32x4 k[2][KS];   // A_K rows: MFMA block c, lane row l16
        u32x4 v[RBK];     // A_V^T: ranks 16 rb + l16, the 8 rows of kept chunk lg
    };
    auto load_blk = [&](RowRegs& X, int k) {
        const int qk = 4 * k + (l16 >> 2);
        const int ck = qk < ksel ? sel[qk] * CHUNK : T;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int t = ck + 4 * c + (l16 & 3);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                X.k[c][ks] = t < T ? load16(AK + (size_t)t * R + 32 * ks + 8 * lg) : u32x4{0u, 0u, 0u, 0u};
        }
        const int qv4 = 4 * k + lg;
        const int cv = qv4 < ksel ? sel[qv4] : -1;
#pragma unroll
        for (int rb = 0; rb < RBK; ++rb)
            X.v[rb] = cv >= 0 ? load16(AV + (size_t)cv * R * CHUNK + (16 * rb + l16) * CHUNK)
                              : u32x4{0u, 0u, 0u, 0u};
    };
    float mr = -INFINITY, zl = 0.f;      // head l16: reference maximum, this lane's sum
    f32x4 acc[RBK];                      // a~^T: rank 16 rb + 4 lg + i, head l16
#pragma unroll
    for (int rb = 0; rb < RBK; ++rb) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute_blk = [&](RowRegs& X, int k) {
        f32x4 S[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            S[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                S[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(X.k[c][ks]), qh[ks], S[c], 0, 0, 0);
                S[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(X.k[c][ks]), ql[ks], S[c], 0, 0, 0);
            }
        }
        // S[c][i]: head l16, row 4 c + i of kept chunk lg of this block
        const int qv4 = 4 * k + lg;
        const int cb = qv4 < ksel ? sel[qv4] * CHUNK : T;
        float sv[8];
        float mx = -INFINITY;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = cb + 4 * c + i < T ? S[c][i] * scale2 : -INFINITY;
                sv[4 * c + i] = x;
                mx = fmaxf(mx, x);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool move = mx > mr + 8.f;            // also the first block with a row
        const float mnew = move ? mx : mr;
        const float alpha = move ? exp2f(mr - mnew) : 1.f;   // 0 from -inf
        const bool any_move = __ballot(move) != 0;
        mr = mnew;
        float ps = 0.f;
        u16x8 hi, lo;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const float pj = sv[jj] == -INFINITY ? 0.f : exp2f(sv[jj] - mnew);
            ps += pj;
            const uint16_t h16 = f32_to_bf16(pj);
            hi[jj] = h16;
            lo[jj] = f32_to_bf16(pj - bf16_to_f32(h16));
        }
        zl = zl * alpha + ps;
        if (any_move) {
#pragma unroll
            for (int rb = 0; rb < RBK; ++rb) acc[rb] *= alpha;
        }
        if (cb + CHUNK > T && cb < T) {
            // the sequence's last chunk: its rows past T hold arbitrary bits
#pragma unroll
            for (int rb = 0; rb < RBK; ++rb) {
                u16x8 e = __builtin_bit_cast(u16x8, X.v[rb]);
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) e[jj] = cb + jj < T ? e[jj] : (uint16_t)0;
                X.v[rb] = __builtin_bit_cast(u32x4, e);
            }
        }
        const bf16x8 pH = __builtin_bit_cast(bf16x8, hi), pL = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
        for (int rb = 0; rb < RBK; ++rb) {
            acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(X.v[rb]), pH, acc[rb], 0, 0, 0);
            acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(X.v[rb]), pL, acc[rb], 0, 0, 0);
        }
    };
    // one block in flight per wave (sixteen waves: 128 KB per workgroup); a
    // second register set would not fit beside the accumulators
    for (int k = sp + ns * wave; k < nblk; k += ns * NW) {
        RowRegs X;
        load_blk(X, k);
        compute_blk(X, k);
    }

    // 5. the waves' partials (every lane of head l16 shares its reference)
    zl += __shfl_xor(zl, 16);
    zl += __shfl_xor(zl, 32);
    if (l16 < g) {
        float* d = wp + (wave * MAXG + l16) * (R + 2);
#pragma unroll
        for (int rb = 0; rb < RBK; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) d[16 * rb + 4 * lg + i] = acc[rb][i];
        if (lg == 0) {
            d[R] = mr;
            d[R + 1] = zl;
        }
    }
    __syncthreads();
    // this split's partial: [MAXG][R + 2] = (a~ [R], reference, sum) per head
    float* part = p.ws_part + (size_t)slab * ns * PP;
    for (int x = tid; x < g * (R + 1); x += NT) {
        const int h = x / (R + 1), c = x % (R + 1);
        float M = -INFINITY;
        for (int w2 = 0; w2 < NW; ++w2) M = fmaxf(M, wp[(w2 * MAXG + h) * (R + 2) + R]);
        float sum = 0.f;
        for (int w2 = 0; w2 < NW; ++w2) {
            const float* d = wp + (w2 * MAXG + h) * (R + 2);
            const float f = d[R] == -INFINITY ? 0.f : exp2f(d[R] - M);   // a wave without rows
            sum = f == 0.f ? sum : fmaf(f, d[c < R ? c : R + 1], sum);
        }
        float* dst = part + (size_t)sp * PP + h * (R + 2);
        if (c < R) {
            st_coh(dst + c, sum);
        } else {
            st_coh(dst + R, M);
            st_coh(dst + R + 1, sum);
        }
    }
    if (!arrive_last(p.ws_arrive + slab, ns)) return;

    // The last split of (b, j): B_l^V, the splits' partials merged, output.
    const float* BV = p.bv + (size_t)slab * n * R + (size_t)p.layer * D * R;
    for (int x = tid; x < D * R; x += NT) bvs[(x / R) * BVP + x % R] = BV[x];
    const size_t row0 = (size_t)b * p.hq + (size_t)j * g;        // first output row of (b, j)
    const bool qok = tid < g * D;                                 // (head tid / D, channel tid % D)
    const float o2 = (qok && p.o_in) ? p.o_in[row0 * D + tid] : 0.f;
    const float l2 = (qok && p.o_in) ? p.lse_in[row0 + tid / D] : -INFINITY;
    for (int x = tid; x < g * (R + 1); x += NT) {
        const int h = x / (R + 1), c = x % (R + 1);
        float M = -INFINITY;
        for (int s2 = 0; s2 < ns; ++s2) M = fmaxf(M, ld_coh(part + (size_t)s2 * PP + h * (R + 2) + R));
        float sum = 0.f;
        for (int s2 = 0; s2 < ns; ++s2) {
            const float* d = part + (size_t)s2 * PP + h * (R + 2);
            const float ms = ld_coh(d + R);
            const float f = ms == -INFINITY ? 0.f : exp2f(ms - M);       // a split without rows
            const float v = ld_coh(d + (c < R ? c : R + 1));
            sum = f == 0.f ? sum : fmaf(f, v, sum);
        }
        if (c < R) {
            qt[h * R + c] = sum;
        } else {
            hz[h] = sum;
            hm[h] = M;
        }
    }
    __syncthreads();
    if (qok) {
        const int h = tid / D, i = tid % D;
        float o = 0.f;
#pragma unroll 16
        for (int c = 0; c < R; ++c) o = fmaf(bvs[i * BVP + c], qt[h * R + c], o);
        const float zz = hz[h];
        float l1 = zz > 0.f ? (hm[h] + log2f(zz)) * LN2 : -INFINITY;
        o = zz > 0.f ? o / zz : 0.f;
        if (p.o_in) {
            const float mm = fmaxf(l1, l2);
            if (mm != -INFINITY) {
                const float w1 = (l1 == -INFINITY) ? 0.f : expf(l1 - mm);
                const float w2 = (l2 == -INFINITY) ? 0.f : expf(l2 - mm);
                o = (o * w1 + o2 * w2) / (w1 + w2);
                l1 = mm + logf(w1 + w2);
            }
        }
        p.out[row0 * D + tid] = o;
        if (i == 0 && p.lse) p.lse[row0 + h] = l1;
    }
}

}  // namespace

hipError_t launch_xkv_factor(const XkvLaunch& p, hipStream_t st) {
    const int n = p.window * D;
    const dim3 ggrid(p.window * (p.window + 1) / 2, p.hkv, p.nb);
    hipLaunchKernelGGL(xkv_gram<false>, ggrid, dim3(256), 0, st, p);
    hipLaunchKernelGGL(xkv_gram<true>, ggrid, dim3(256), 0, st, p);
    auto big = [&](const void* kern, size_t lds) {
        return lds <= 64 * 1024 ||
               hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) ==
                   hipSuccess;
    };
    const size_t zlds = (size_t)n * (p.rank + 1) * sizeof(float);
    const dim3 sgrid(2 * p.nb * p.hkv);
    const size_t vlds = (size_t)p.rank * (n + 8) * 2;
    const size_t tlds = (size_t)4 * D * VPITCH * 2;
    const dim3 pgrid(p.nsplit, p.hkv, p.nb);
    if (p.rank == 32) {
        if (!big((const void*)xkv_subspace<32>, zlds) || !big((const void*)xkv_project<false, 32>, vlds) ||
            !big((const void*)xkv_project<true, 32>, vlds + tlds))
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(xkv_subspace<32>, sgrid, dim3(256), zlds, st, p);
        hipLaunchKernelGGL((xkv_project<false, 32>), pgrid, dim3(256), vlds, st, p);
        hipLaunchKernelGGL((xkv_project<true, 32>), pgrid, dim3(256), vlds + tlds, st, p);
    } else {
        if (!big((const void*)xkv_subspace<64>, zlds) || !big((const void*)xkv_project<false, 64>, vlds) ||
            !big((const void*)xkv_project<true, 64>, vlds + tlds))
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(xkv_subspace<64>, sgrid, dim3(256), zlds, st, p);
        hipLaunchKernelGGL((xkv_project<false, 64>), pgrid, dim3(256), vlds, st, p);
        hipLaunchKernelGGL((xkv_project<true, 64>), pgrid, dim3(256), vlds + tlds, st, p);
    }
    return hipGetLastError();
}

size_t xkv_scores_lds(int rank) { return (size_t)xs_floats(rank) * 4; }

size_t xkv_rows_lds(int rank, int nch, int ksel, bool gkeys) {
    return ((size_t)xr_floats(rank) + ksel + (gkeys ? 0 : nch)) * 4;
}

hipError_t launch_xkv_decode(const XkvDecodeLaunch& p, bool gkeys, size_t rows_lds, hipStream_t st) {
    const dim3 grid(p.ns, p.hkv, p.nb);
    auto go = [&](auto kern, size_t lds, int nt) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(kern, grid, dim3(nt), lds, st, p);
        return hipGetLastError();
    };
    const size_t slds = xkv_scores_lds(p.rank);
    hipError_t e;
    if (p.rank == 32) {
        e = go(xkv_scores<32>, slds, XS_NT);
        if (e == hipSuccess)
            e = gkeys ? go(xkv_rows<32, true>, rows_lds, XF_NT) : go(xkv_rows<32, false>, rows_lds, XF_NT);
    } else {
        e = go(xkv_scores<64>, slds, XS_NT);
        if (e == hipSuccess)
            e = gkeys ? go(xkv_rows<64, true>, rows_lds, XF_NT) : go(xkv_rows<64, false>, rows_lds, XF_NT);
    }
    return e;
}

}  // namespace kvc
