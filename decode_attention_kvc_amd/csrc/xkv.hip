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
// Decode, three launches so that the whole chip streams the landmarks and
// the kept rows (one workgroup per (b, j) would leave half the CUs idle):
//  1. xkv_scores, (chunk split, b, j): q~_h = B_l q_h (r numbers per head)
//     and the chunk scores max_h q~_h . landmark;
//  2. xkv_attend, (row split, b, j): exact top-k of the chunks (radix
//     select, ties to the lower chunk; each split repeats it), then attention
//     over the split's share of the kept rows in the rank space:
//     q_h . (A_t B_l) = q~_h . A_t and sum_t p_t A_t B_l = (sum_t p_t A_t)
//     B_l, so the selected rows are rebuilt implicitly and never written;
//  3. xkv_output, (b, j): the splits' partials merge with log-sum-exp
//     weights, the output is projected by B_l^V, and an optional second part
//     (rows appended after the factorisation, attended separately) is merged
//     the same way.
#include "common.h"
#include "kvc_internal.h"
#include "philox.h"
#include "radix.h"

namespace kvc {

namespace {

constexpr int XT = 32;          // rows per tile
constexpr int GP = 40;          // bf16 per staged channel row of a tile (80 bytes)
constexpr int CHUNK = 8;        // rows per landmark chunk
constexpr int VPITCH = XT + 2;  // bf16 per channel in a wave's value transpose buffer
constexpr int MAXG = 8;         // query heads per KV head on the decode path
constexpr int XNT = 512;        // threads of a decode workgroup (two waves per SIMD)
constexpr int XNW = XNT / WAVE;
static_assert(XNT == 4 * D, "the output step maps one thread to a (head, channel) pair");

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
                    if (t < T) A[(size_t)t * R + 16 * cb + l16] = h;
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

// Lane permutations inside a 16-lane row (DPP: plain VALU moves).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum over aligned groups of N lanes (N = 4 or 8; every lane gets it): swap
// neighbours, swap pairs, then (N = 8) mirror the half-row.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    if constexpr (N == 8) v += dpp_mov<0x141>(v);
    return v;
}
// Sum over the lanes of a wave whose index agrees modulo N (N = 2 or 4):
// rotations inside each 16-lane row, then across the four rows.
template <int N>
__device__ __forceinline__ float strided_sum(float v) {
    if constexpr (N == 2) v += dpp_mov<0x122>(v);      // row_ror:2
    if constexpr (N <= 4) v += dpp_mov<0x124>(v);      // row_ror:4
    v += dpp_mov<0x128>(v);                             // row_ror:8
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Lanes per row of the rank space (8 columns each) and the dot products of
// one row with the G query vectors q~ held in registers, summed over the
// row's lanes (every lane of the group gets the sums).
template <int R, int G>
__device__ __forceinline__ void rank_dots(const u32x4& w, const float (&qr)[G][8], float (&s)[G]) {
    constexpr int LPR = R / 8;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a = fmaf(qr[h][2 * e], bf16lo(w[e]), a);
            a = fmaf(qr[h][2 * e + 1], bf16hi(w[e]), a);
        }
        s[h] = group_sum<LPR>(a);
    }
}

// q~_h = B_l q_h for the g heads of one (b, j) into LDS qt [MAXG][R] (heads
// past g: zero); qs is scratch for the queries as float [g][D].
template <int R>
__device__ __forceinline__ void rank_queries(const XkvDecodeLaunch& p, int slab, int b, int j,
                                             float* qs, float* qt) {
    const int tid = threadIdx.x, g = p.g, n = p.window * D;
    const float* BK = p.bk + (size_t)slab * n * R + (size_t)p.layer * D * R;
    const uint16_t* q = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)b * p.hq + j * g) * D;
    for (int x = tid; x < g * D; x += XNT) qs[x] = bf16_to_f32(q[x]);
    __syncthreads();
    for (int x = tid; x < MAXG * R; x += XNT) {
        const int h = x / R, c = x % R;
        float a0 = 0.f, a1 = 0.f;
        if (h < g) {
            const float* qh = qs + h * D;
#pragma unroll 16
            for (int i = 0; i < D; i += 2) {
                a0 = fmaf(qh[i], BK[i * R + c], a0);
                a1 = fmaf(qh[i + 1], BK[(i + 1) * R + c], a1);
            }
        }
        qt[h * R + c] = a0 + a1;
    }
    __syncthreads();
}

// Decode, step 1: grid (chunk split, j, b).  q~ (the first split also keeps
// it in the workspace for step 2) and the score keys of this split's chunks:
// max over the heads of q~_h . landmark, LPR lanes per chunk, UNR chunks in
// flight per lane group.
template <int R, int G>
__global__ __launch_bounds__(XNT) void xkv_scores(XkvDecodeLaunch p) {
    __shared__ float qs[MAXG * D];
    __shared__ float qt[MAXG * R];
    constexpr int LPR = R / 8;
    constexpr int NGRP = XNT / LPR;
    constexpr int UNR = G <= 4 ? 16 : 8;
    // The chunk splits of a (batch, KV head) pair read the same query
    // projection inputs: contiguous runs of blocks per XCD share them in L2.
    const BlockXYZ blk = xcd_run_block(true);
    const int s = blk.x, j = blk.y, b = blk.z;
    const int slab = b * p.hkv + j, g = p.g;
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int sub = lane % LPR, grp = tid / LPR;
    const int nch = (p.t_len + CHUNK - 1) / CHUNK;
    const int c0 = s * p.cps, c1 = min(nch, c0 + p.cps);
    rank_queries<R>(p, slab, b, j, qs, qt);
    if (s == 0)
        for (int x = tid; x < MAXG * R; x += XNT) p.ws_qt[(size_t)slab * MAXG * R + x] = qt[x];
    float qr[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) qr[h][e] = qt[h * R + 8 * sub + e];
    const uint16_t* L = reinterpret_cast<const uint16_t*>(p.lk) + (size_t)slab * (p.x_tcap / CHUNK) * R;
    uint32_t* keys = p.ws_keys + (size_t)slab * nch;
    for (int base = c0; base < c1; base += UNR * NGRP) {
        u32x4 w[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int ch = base + u * NGRP + grp;
            w[u] = ch < c1 ? load16(L + (size_t)ch * R + 8 * sub) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int ch = base + u * NGRP + grp;
            float sc[G];
            rank_dots<R, G>(w[u], qr, sc);
            float best = -INFINITY;
#pragma unroll
            for (int h = 0; h < G; ++h)
                if (h < g) best = fmaxf(best, sc[h]);
            if (sub == 0 && ch < c1) keys[ch] = desc_key(best);
        }
    }
}

// Decode, step 2: grid (row split, j, b).  Every workgroup of a (b, j)
// selects the same ksel chunks from the keys (exact radix select, ties to
// the lower chunk; the first workgroup reports them), then takes its share
// [r0, r1) of the kept rows: logits in the rank space, its own maximum per
// head, and a~_h = sum_t p_t,h A^V_t with z_h = sum_t p_t,h; the partial
// (a~, max, z) goes to the workspace.
template <int R, int G>
__global__ __launch_bounds__(XNT) void xkv_attend(XkvDecodeLaunch p) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ RadixSmem<XNT, 8> rs;
    __shared__ float red[XNW][MAXG];
    __shared__ float hm[MAXG];
    constexpr int LPR = R / 8;             // lanes per rank-space row
    constexpr int NGRP = XNT / LPR;        // rows per block pass
    constexpr int UNR = G <= 4 ? 16 : 8;   // logit rows in flight per lane group
    constexpr int CW = G <= 4 ? 16 : 8;    // value phase: columns per lane
    constexpr int CG = R / CW;             //              column groups
    constexpr int RGW = WAVE / CG;         //              row groups per wave
    constexpr int RGS = XNW * RGW;         //              row groups per block
    // The row splits of a pair read the same chunk scores and query
    // projection: contiguous runs of blocks per XCD share them in L2.
    const BlockXYZ blk = xcd_run_block(true);
    const int a = blk.x, j = blk.y, b = blk.z;
    const int slab = b * p.hkv + j, g = p.g;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int sub = lane % LPR, grp = tid / LPR;
    const int T = p.t_len, nch = (T + CHUNK - 1) / CHUNK;
    const int ksel = min(p.n_select, nch), nrows = ksel * CHUNK;
    const int r0 = min(nrows, a * p.rpw), r1 = min(nrows, r0 + p.rpw);
    uint32_t* keys = reinterpret_cast<uint32_t*>(smem);          // [nch]
    int32_t* sel = reinterpret_cast<int32_t*>(keys + nch);       // [ksel]
    float* lgt = reinterpret_cast<float*>(sel + ksel);           // [rpw][g]
    float* part = lgt + (size_t)p.rpw * g;                       // [XNW][MAXG][R + 1]
    float* out_part = p.ws_part + ((size_t)slab * p.nattend + a) * MAXG * (R + 2);

    if (r0 >= r1 && !(a == 0 && p.selected)) {
        // no rows here and nothing to report: an empty partial
        for (int h = tid; h < MAXG; h += XNT) {
            out_part[h * (R + 2) + R] = -INFINITY;
            out_part[h * (R + 2) + R + 1] = 0.f;
        }
        return;
    }
    const float* qtg = p.ws_qt + (size_t)slab * MAXG * R;
    float qr[G][8];                      // this lane's 8 columns of every q~_h
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) qr[h][e] = qtg[h * R + 8 * sub + e];
    const uint32_t* kg = p.ws_keys + (size_t)slab * nch;
    for (int ch = tid; ch < nch; ch += XNT) keys[ch] = kg[ch];
    __syncthreads();

    // the ksel best chunks, ascending (all of them when there are fewer):
    // thread t owns the contiguous chunks [t*per, (t+1)*per), so one block
    // scan places the equal keys in chunk order and another the kept ones
    if (ksel < nch) {
        uint32_t take;
        const uint32_t thr = radix_select<XNT>(nch, (uint32_t)ksel, [&](int t) { return keys[t]; },
                                               rs, &take);
        const int per = (nch + XNT - 1) / XNT;
        const int c0 = min(nch, tid * per), c1 = min(nch, c0 + per);
        uint32_t n_eq = 0;
        for (int ch = c0; ch < c1; ++ch) n_eq += keys[ch] == thr;
        uint32_t tot;
        uint32_t eq_rank = block_scan_u32<XNT>(n_eq, rs, &tot);
        uint32_t n_keep = 0;
        for (int ch = c0; ch < c1; ++ch) {
            const uint32_t u = keys[ch];
            n_keep += (u < thr) || (u == thr && eq_rank++ < take);
        }
        eq_rank -= n_eq;                           // back to this thread's first equal key
        uint32_t pos = block_scan_u32<XNT>(n_keep, rs, &tot);
        for (int ch = c0; ch < c1; ++ch) {
            const uint32_t u = keys[ch];
            if ((u < thr) || (u == thr && eq_rank++ < take)) {
                if (pos < (uint32_t)ksel) sel[pos] = ch;
                ++pos;
            }
        }
    } else {
        for (int ch = tid; ch < nch; ch += XNT) sel[ch] = ch;
    }
    __syncthreads();
    if (a == 0 && p.selected)
        for (int x = tid; x < p.n_select; x += XNT)
            p.selected[(size_t)slab * p.n_select + x] = x < ksel ? sel[x] : -1;

    // logits of this workgroup's rows in the rank space (LPR lanes per row,
    // UNR rows in flight) and its maximum per head
    const uint16_t* AK = reinterpret_cast<const uint16_t*>(p.ak) + (size_t)slab * p.x_tcap * R;
    const uint16_t* AV = reinterpret_cast<const uint16_t*>(p.av) + (size_t)slab * p.x_tcap * R;
    {
        float mh[G];
#pragma unroll
        for (int h = 0; h < G; ++h) mh[h] = -INFINITY;
        for (int base = r0; base < r1; base += UNR * NGRP) {
            u32x4 w[UNR];
            int tr[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int r = base + u * NGRP + grp;
                tr[u] = r < r1 ? sel[r / CHUNK] * CHUNK + r % CHUNK : T;
                w[u] = tr[u] < T ? load16(AK + (size_t)tr[u] * R + 8 * sub) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int r = base + u * NGRP + grp;
                float sc[G];
                rank_dots<R, G>(w[u], qr, sc);
                if (r < r1) {
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        if (h < g) {
                            const float l = tr[u] < T ? sc[h] * p.scale : -INFINITY;
                            mh[h] = fmaxf(mh[h], l);
                            if (sub == 0) lgt[(r - r0) * g + h] = l;
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float m = wave_max(mh[h]);
            if (lane == 0) red[wave][h] = m;
        }
        __syncthreads();
        if (tid < MAXG) {
            float m = red[0][tid];
            for (int w2 = 1; w2 < XNW; ++w2) m = fmaxf(m, red[w2][tid]);
            hm[tid] = m;
        }
        __syncthreads();
    }

    // a~ and z over this workgroup's rows: lane (row group, CW-column
    // group), 16-byte value reads, VR rows in flight; then sums over the row
    // groups (lanes, then waves)
    {
        const int cg = lane % CG, rgl = lane / CG;
        const int rg = wave * RGW + rgl;
        float mx[G];
#pragma unroll
        for (int h = 0; h < G; ++h) mx[h] = hm[h];
        float acc[G][CW], zs[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            zs[h] = 0.f;
#pragma unroll
            for (int e = 0; e < CW; ++e) acc[h][e] = 0.f;
        }
        constexpr int VR = 8;
        constexpr int NL = CW / 8;                 // 16-byte loads per row and lane
        for (int base = r0 + rg; base < r1; base += VR * RGS) {
            u32x4 w[VR][NL];
            int tr[VR];
#pragma unroll
            for (int u = 0; u < VR; ++u) {
                const int r = base + u * RGS;
                tr[u] = r < r1 ? sel[r / CHUNK] * CHUNK + r % CHUNK : T;
                const bool ok = tr[u] < T;
#pragma unroll
                for (int q2 = 0; q2 < NL; ++q2)
                    w[u][q2] = ok ? load16(AV + (size_t)tr[u] * R + CW * cg + 8 * q2)
                                  : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < VR; ++u) {
                const int r = base + u * RGS;
                if (tr[u] < T) {
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        if (h < g) {
                            const float pr = expf(lgt[(r - r0) * g + h] - mx[h]);
                            zs[h] += pr;
#pragma unroll
                            for (int q2 = 0; q2 < NL; ++q2)
#pragma unroll
                                for (int e = 0; e < 4; ++e) {
                                    acc[h][8 * q2 + 2 * e] =
                                        fmaf(pr, bf16lo(w[u][q2][e]), acc[h][8 * q2 + 2 * e]);
                                    acc[h][8 * q2 + 2 * e + 1] =
                                        fmaf(pr, bf16hi(w[u][q2][e]), acc[h][8 * q2 + 2 * e + 1]);
                                }
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            zs[h] = strided_sum<CG>(zs[h]);
#pragma unroll
            for (int e = 0; e < CW; ++e) acc[h][e] = strided_sum<CG>(acc[h][e]);
        }
        if (rgl == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
#pragma unroll
                for (int e = 0; e < CW; ++e) part[(wave * MAXG + h) * (R + 1) + CW * cg + e] = acc[h][e];
                if (cg == 0) part[(wave * MAXG + h) * (R + 1) + R] = zs[h];
            }
        }
    }
    __syncthreads();
    for (int x = tid; x < MAXG * (R + 1); x += XNT) {
        const int h = x / (R + 1), c = x % (R + 1);
        float s4 = 0.f;
        for (int w2 = 0; w2 < XNW; ++w2) s4 += part[(w2 * MAXG + h) * (R + 1) + c];
        out_part[h * (R + 2) + (c < R ? c : R + 1)] = s4;
        if (c == R) out_part[h * (R + 2) + R] = hm[h];
    }
}

// Decode, step 3: grid (j, b).  The row splits' partials merge with
// log-sum-exp weights; o_h = B_l^V a~_h / z_h, merged with the second part
// if given.  Thread (h, i) owns output channel i of heads h and h + 4.
// Every global read (its row of B_l^V, the second part, the partials) is
// issued before the first barrier, so the kernel waits on one round trip.
template <int R>
__global__ __launch_bounds__(XNT) void xkv_output(XkvDecodeLaunch p) {
    __shared__ float ps[XKV_MAX_ATTEND * MAXG * (R + 2)];
    __shared__ float at[MAXG * R];
    __shared__ float hz[MAXG], hmx[MAXG];
    __shared__ float wts[XKV_MAX_ATTEND * MAXG];
    constexpr int HPT = MAXG / (XNT / D);      // heads per thread
    const int j = blockIdx.x, b = blockIdx.y;
    const int slab = b * p.hkv + j, g = p.g, n = p.window * D, tid = threadIdx.x;
    const int na = p.nattend;
    const float* P = p.ws_part + (size_t)slab * na * MAXG * (R + 2);
    const float* BV = p.bv + (size_t)slab * n * R + (size_t)p.layer * D * R;
    const int oh = tid / D, i = tid % D;
    f32x4 bvv[R / 4];
#pragma unroll
    for (int c4 = 0; c4 < R / 4; ++c4) bvv[c4] = *reinterpret_cast<const f32x4*>(BV + i * R + 4 * c4);
    float o2[HPT], l2[HPT];
#pragma unroll
    for (int k = 0; k < HPT; ++k) {
        const int h = oh + k * (XNT / D);
        const size_t row = (size_t)b * p.hq + j * g + h;
        o2[k] = (p.o_in && h < g) ? p.o_in[row * D + i] : 0.f;
        l2[k] = (p.o_in && h < g) ? p.lse_in[row] : -INFINITY;
    }
    for (int x = tid; x < na * MAXG * (R + 2); x += XNT) ps[x] = P[x];
    __syncthreads();
    if (tid < MAXG) {
        float M = -INFINITY;
        for (int a = 0; a < na; ++a) M = fmaxf(M, ps[(a * MAXG + tid) * (R + 2) + R]);
        for (int a = 0; a < na; ++a) {
            const float ma = ps[(a * MAXG + tid) * (R + 2) + R];
            wts[a * MAXG + tid] = ma == -INFINITY ? 0.f : expf(ma - M);   // a split without rows
        }
        hmx[tid] = M;
    }
    __syncthreads();
    for (int x = tid; x < g * (R + 1); x += XNT) {
        const int h = x / (R + 1), c = x % (R + 1);
        float sum = 0.f;
        for (int a = 0; a < na; ++a) {
            const float w = wts[a * MAXG + h];
            const float v = ps[(a * MAXG + h) * (R + 2) + (c < R ? c : R + 1)];
            sum = w == 0.f ? sum : fmaf(w, v, sum);
        }
        if (c < R) at[h * R + c] = sum;
        else hz[h] = sum;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < HPT; ++k) {
        const int h = oh + k * (XNT / D);
        if (h >= g) break;
        float o = 0.f;
#pragma unroll
        for (int c4 = 0; c4 < R / 4; ++c4)
#pragma unroll
            for (int e = 0; e < 4; ++e) o = fmaf(bvv[c4][e], at[h * R + 4 * c4 + e], o);
        const float zz = hz[h];
        float l1 = zz > 0.f ? hmx[h] + logf(zz) : -INFINITY;
        o = zz > 0.f ? o / zz : 0.f;
        const size_t row = (size_t)b * p.hq + j * g + h;
        if (p.o_in) {
            const float mm = fmaxf(l1, l2[k]);
            if (mm != -INFINITY) {
                const float w1 = (l1 == -INFINITY) ? 0.f : expf(l1 - mm);
                const float w2 = (l2[k] == -INFINITY) ? 0.f : expf(l2[k] - mm);
                o = (o * w1 + o2[k] * w2) / (w1 + w2);
                l1 = mm + logf(w1 + w2);
            }
        }
        p.out[row * D + i] = o;
        if (i == 0 && p.lse) p.lse[row] = l1;
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

hipError_t launch_xkv_decode(const XkvDecodeLaunch& p, size_t lds, hipStream_t st) {
    const dim3 sgrid(p.nscore, p.hkv, p.nb), agrid(p.nattend, p.hkv, p.nb), ogrid(p.hkv, p.nb);
    auto go = [&](auto score, auto attend, auto output) {
        if (lds > 64 * 1024 &&
            hipFuncSetAttribute(reinterpret_cast<const void*>(attend),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL(score, sgrid, dim3(XNT), 0, st, p);
        hipLaunchKernelGGL(attend, agrid, dim3(XNT), lds, st, p);
        hipLaunchKernelGGL(output, ogrid, dim3(XNT), 0, st, p);
        return hipGetLastError();
    };
    if (p.rank == 32)
        return p.g <= 4 ? go(xkv_scores<32, 4>, xkv_attend<32, 4>, xkv_output<32>)
                        : go(xkv_scores<32, 8>, xkv_attend<32, 8>, xkv_output<32>);
    return p.g <= 4 ? go(xkv_scores<64, 4>, xkv_attend<64, 4>, xkv_output<64>)
                    : go(xkv_scores<64, 8>, xkv_attend<64, 8>, xkv_output<64>);
}

}  // namespace kvc
