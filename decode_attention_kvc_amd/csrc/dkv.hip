// VASE-DKV token scores: leverage of the Gaussian-sketched [K | V] rows.
//
// VASE summary (gist.science 2606.03928), §2.B: VASE-DKV adapts CurDKV, whose
// token scores are leverage scores from a CUR decomposition, and draws a new
// Gaussian projection G at every eviction pass.  Reading used here (the page
// gives no formula): score_t = y_t (Y^T Y)^+ y_t^T with Y = [K | V] G, G of
// shape (2d, R), i.e. the leverage of row t of the sketch; the pseudo-inverse
// goes through a Cholesky factorisation that drops every direction whose pivot
// is at most 1e-12 of the Gram matrix's trace.
//
// Three kernels per slot:
//  1. dkv_sketch: Y = [K | V] G on MFMA (v_mfma_f32_16x16x32_bf16, G staged in
//     LDS), one wave per 32-row tile.  K rows are row-major, so their operand
//     fragments come straight from HBM; the V tile is channel-major, so it is
//     written to a per-wave LDS buffer and read back one token per lane.  The
//     tile's Y (float32) goes to the workspace, and the Gram matrix Y^T Y
//     accumulates in float64 with v_mfma_f64_16x16x4_f64 on the Y fragments
//     as they are: in the 16x16 output layout lane l holds rows 4*(l/16)+i of
//     column l%16, which is exactly the A operand of Y^T (column l%16,
//     reduction index l/16) and the B operand of Y for register i.  Products
//     of two float32 values are exact in float64, so the Gram of the float32
//     sketch is accurate to float64 rounding; directions that the rows do not
//     span then show pivots far below the drop threshold (with a float32 Gram
//     they would sit at float32 rounding, ~1e-7 of the trace, and survive).
//     The value range of the tile is taken from the same V registers.  Each
//     workgroup writes its partial Gram (float64).
//  2. dkv_factor: one wave per slab sums the partial Grams in split order,
//     factors them (Cholesky with dropped pivots, float64, in registers) and
//     writes W = R^{-1} (zero rows for dropped directions) as float64.
//  3. dkv_leverage: score_t = ||y_t W||^2 in float64 (the float32 y_t widened
//     exactly), one thread per row, rounded to float32 once at the end; the
//     inverse factor and the quadratic form then add only float64 rounding
//     to what the float32 sketch carries.
// Ragged batches: sequence b sketches rows [0, T_b) of cache entry phys(b)
// (splits past its end contribute a zero Gram); Y and the scores keep the
// launch's t_len as their row stride.
#include <type_traits>

#include "common.h"
#include "kvc_internal.h"
#include "philox.h"

namespace kvc {

namespace {

constexpr int DT = 32;                 // rows per tile
constexpr int KV = 2 * D;              // sketched row length: key then value
constexpr int GPITCH = KV + 8;         // bf16 per staged sketch column (528 bytes)
constexpr int VPITCH = DT + 2;         // bf16 per channel in a wave's V buffer (68 bytes)
constexpr int NW = 4;

__device__ __forceinline__ bf16x8 as_bf(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Range of 32 rows from a channel-major V block in registers (lane (l16, lg):
// channels 16*dt + l16, rows 8*lg .. +8).  Max / min over the 16 lanes of a
// row with DPP moves.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
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
__device__ __forceinline__ void tile_range(const u32x4 (&x)[8], int t0, int T, float* range_out,
                                           int lane) {
    const int l16 = lane & 15, lg = lane >> 4;
    float mx[8], mn[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        mx[jj] = -INFINITY;
        mn[jj] = INFINITY;
    }
#pragma unroll
    for (int dt = 0; dt < 8; dt += 2)
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            const float a0 = bf16lo(x[dt][w2]), a1 = bf16lo(x[dt + 1][w2]);
            const float b0 = bf16hi(x[dt][w2]), b1 = bf16hi(x[dt + 1][w2]);
            mx[2 * w2] = fmaxf(mx[2 * w2], fmaxf(a0, a1));
            mn[2 * w2] = fminf(mn[2 * w2], fminf(a0, a1));
            mx[2 * w2 + 1] = fmaxf(mx[2 * w2 + 1], fmaxf(b0, b1));
            mn[2 * w2 + 1] = fminf(mn[2 * w2 + 1], fminf(b0, b1));
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

// Range of the 32 rows of a tile whose values were loaded as rows (the
// operand fragments va[rb][kc]: row t0 + 16*rb + l16, channels 32*kc + 8*lg
// .. +8): each lane reduces its 32 channels, the four lane groups of a row
// meet by lane exchanges.
__device__ __forceinline__ void tile_range_rows(const u32x4 (&va)[2][4], int t0, int T,
                                                float* range_out, int lane) {
    const int l16 = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        float mx = -INFINITY, mn = INFINITY;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                const float a = bf16lo(va[rb][kc][w2]), c = bf16hi(va[rb][kc][w2]);
                mx = fmaxf(mx, fmaxf(a, c));
                mn = fminf(mn, fminf(a, c));
            }
#pragma unroll
        for (int m = 16; m < 64; m <<= 1) {
            mx = fmaxf(mx, __shfl_xor(mx, m));
            mn = fminf(mn, __shfl_xor(mn, m));
        }
        const int t = t0 + 16 * rb + l16;
        if (lg == 0 && t < T) range_out[t] = mx - mn;
    }
}

// VROWS: the slab's values are [t][D] rows (a prefill's layout) and load as
// operand fragments exactly like the keys, with no transpose.
template <int R, bool RANGE, bool VROWS>
__global__ __launch_bounds__(256) void dkv_sketch(DkvLaunch p) {
    constexpr int CB = R / 16;                  // 16-column blocks of Y
    constexpr int NG = CB * (CB + 1) / 2;       // upper-triangle Gram blocks
    __shared__ __align__(16) uint16_t gs[R * GPITCH];
    __shared__ __align__(16) uint16_t vbuf[NW][D * VPITCH];
    static_assert(NG * 64 * 4 * sizeof(double) <= D * VPITCH * sizeof(uint16_t),
                  "a wave's Gram blocks fit in its V buffer");
    const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int slab = b * p.hkv + j;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int l16 = lane & 15, lg = lane >> 4;
    const int phys = seq_phys(p.sm, b);
    const int T = seq_rows(p.sm, b, phys);

    // Stage G: sketch column n is row n of g ([R][2d] bf16).
    const uint16_t* g = reinterpret_cast<const uint16_t*>(p.g);
    for (int x = tid; x < R * (KV / 8); x += blockDim.x) {
        const int n = x / (KV / 8), c = x % (KV / 8);
        *reinterpret_cast<u32x4*>(gs + n * GPITCH + 8 * c) = load16(g + (size_t)n * KV + 8 * c);
    }
    __syncthreads();

    const size_t cslab = (size_t)max(phys, 0) * p.hkv + j;
    const uint16_t* kslab = reinterpret_cast<const uint16_t*>(p.k) + cslab * p.t_cap * D;
    const uint16_t* vslab = reinterpret_cast<const uint16_t*>(p.v) + cslab * p.t_cap * D;
    float* ys = p.y + (size_t)slab * p.t_len * R;
    float* range = RANGE ? p.range + (size_t)slab * p.t_len : nullptr;
    uint16_t* vb = vbuf[wave];
    const int ntiles = (T + DT - 1) / DT;
    const int tile_begin = s * p.tps, tile_end = min(tile_begin + p.tps, ntiles);

    f64x4 gram[NG];
#pragma unroll
    for (int q = 0; q < NG; ++q) gram[q] = f64x4{0.0, 0.0, 0.0, 0.0};

    for (int tile = tile_begin + wave; tile < tile_end; tile += NW) {
        const int t0 = tile * DT;
        // K operand fragments: row t0 + 16*rb + l16, channels 32*kc + 8*lg .. +8.
        u32x4 ka[2][4], vt[8];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const uint16_t* kr = kslab + (size_t)(t0 + 16 * rb + l16) * D + 8 * lg;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) ka[rb][kc] = load_stream16(kr + 32 * kc);
        }
        u32x4 va[2][4];
        if constexpr (VROWS) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const uint16_t* vr = vslab + (size_t)(t0 + 16 * rb + l16) * D + 8 * lg;
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) va[rb][kc] = load_stream16(vr + 32 * kc);
            }
            if constexpr (RANGE) tile_range_rows(va, t0, T, range, lane);
        } else {
            // V block: channels 16*dt + l16, rows 8*lg .. +8.
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
                vt[dt] = load_stream16(vslab + vt_off(t0, 16 * dt + l16) + 8 * lg);

            // V block into the wave's buffer ([channel][row], 68-byte pitch),
            // then back out one row per lane: the previous tile's reads of
            // the buffer and these writes, and these writes and the reads
            // below, are ordered because one wave's LDS instructions execute
            // in issue order.
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                uint32_t* dst = reinterpret_cast<uint32_t*>(vb + (16 * dt + l16) * VPITCH + 8 * lg);
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) dst[w2] = vt[dt][w2];
            }
            __builtin_amdgcn_wave_barrier();
            if constexpr (RANGE) tile_range(vt, t0, T, range, lane);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
                    u16x8 e;
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj)
                        e[jj] = vb[(32 * kc + 8 * lg + jj) * VPITCH + 16 * rb + l16];
                    va[rb][kc] = __builtin_bit_cast(u32x4, e);
                }
        }

        // Y[rb][cb][i]: row t0 + 16*rb + 4*lg + i, sketch column 16*cb + l16.
        f32x4 Y[2][CB];
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const uint16_t* gcol = gs + (16 * cb + l16) * GPITCH + 8 * lg;
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) Y[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const bf16x8 gk = as_bf(*reinterpret_cast<const u32x4*>(gcol + 32 * kc));
                const bf16x8 gv = as_bf(*reinterpret_cast<const u32x4*>(gcol + D + 32 * kc));
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    Y[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(ka[rb][kc]), gk,
                                                                        Y[rb][cb], 0, 0, 0);
                    Y[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(va[rb][kc]), gv,
                                                                        Y[rb][cb], 0, 0, 0);
                }
            }
        }
        // Rows past t_len (arbitrary cache bits) become zero rows.
        if (t0 + DT > T) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int cb = 0; cb < CB; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Y[rb][cb][i] = (t0 + 16 * rb + 4 * lg + i < T) ? Y[rb][cb][i] : 0.f;
        }
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * rb + 4 * lg + i;
                if (t < T) {
#pragma unroll
                    for (int cb = 0; cb < CB; ++cb) ys[(size_t)t * R + 16 * cb + l16] = Y[rb][cb][i];
                }
            }
        // Gram blocks (a <= c): sum over the tile's rows.
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int q = 0;
#pragma unroll
                for (int a = 0; a < CB; ++a)
#pragma unroll
                    for (int c = a; c < CB; ++c, ++q)
                        gram[q] = __builtin_amdgcn_mfma_f64_16x16x4f64(
                            (double)Y[rb][a][i], (double)Y[rb][c][i], gram[q], 0, 0, 0);
            }
    }

    // Sum the four waves' Gram blocks in wave order and write this split's
    // partial: [R][R] float64, both triangles.  Each wave parks its blocks in
    // its own (no longer used) V buffer.
    __builtin_amdgcn_wave_barrier();
    {
        double* mine = reinterpret_cast<double*>(vb);
#pragma unroll
        for (int q = 0; q < NG; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) mine[(q * 64 + lane) * 4 + i] = gram[q][i];
    }
    __syncthreads();
    double* part = p.gram + ((size_t)slab * p.nsplit + s) * R * R;
    for (int x = tid; x < NG * 64 * 4; x += blockDim.x) {
        const int q = x / 256, ln = (x / 4) % 64, i = x % 4;
        double v = 0.0;
#pragma unroll
        for (int w = 0; w < NW; ++w) v += reinterpret_cast<const double*>(vbuf[w])[(q * 64 + ln) * 4 + i];
        int a = 0, c = 0, qq = q;
        for (a = 0; a < CB; ++a) {
            if (qq < CB - a) {
                c = a + qq;
                break;
            }
            qq -= CB - a;
        }
        // block (a, c), lane ln, register i: row ln/16 + 4*i, column ln%16
        // (the float64 16x16 output layout interleaves rows differently from
        // the float32 one, whose lane holds rows 4*(ln/16) + i)
        const int row = 16 * a + ln / 16 + 4 * i, col = 16 * c + ln % 16;
        part[row * R + col] = v;
        part[col * R + row] = v;
    }
}

// Broadcast of lane `src`'s double (src is a compile-time constant in the
// unrolled loops below, so this is two v_readlane into scalar registers).
__device__ __forceinline__ double lane_bcast(double v, int src) {
    const long long bits = __builtin_bit_cast(long long, v);
    const int lo = __builtin_amdgcn_readlane((int)(bits & 0xFFFFFFFF), src);
    const int hi = __builtin_amdgcn_readlane((int)(bits >> 32), src);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned int)lo);
}

// One wave per slab: merge, factor, invert.  Lane i (< R) keeps column i of
// the Gram matrix in registers and the factorisation is right-looking: at
// pivot j every lane turns its entry of row j into U[j][i] and updates its
// column of the Schur complement, with the row's entries broadcast from the
// lanes that own them.  The inverse is a back substitution per column, again
// with broadcast entries of U.  Everything is float64 and fully unrolled.
template <int R>
__global__ __launch_bounds__(64) void dkv_factor(DkvLaunch p) {
    const int slab = blockIdx.y * p.hkv + blockIdx.x;
    const int lane = threadIdx.x;
    const int col = lane < R ? lane : 0;
    const double* part = p.gram + (size_t)slab * p.nsplit * R * R;
    double m[R];
#pragma unroll
    for (int k = 0; k < R; ++k) m[k] = 0.0;
    for (int sp = 0; sp < p.nsplit; ++sp) {
#pragma unroll
        for (int k = 0; k < R; ++k) m[k] += part[((size_t)sp * R + k) * R + col];
    }
    double tr = 0.0;
#pragma unroll
    for (int k = 0; k < R; ++k) tr += lane_bcast(m[k], k);
    const double floor = 1e-12 * fmax(tr, 0.0);

    double u[R];          // column `col` of U: u[j] = U[j][col]
    bool keep[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const double piv = lane_bcast(m[j], j);      // Schur complement's M[j][j]
        keep[j] = piv > floor;
        const double r = keep[j] ? sqrt(piv) : 1.0;
        const double uj = (keep[j] && col >= j) ? m[j] / r : 0.0;
        u[j] = uj;
        // rows j+1.. of this column: m[k] -= U[j][k] * U[j][col], k <= col
#pragma unroll
        for (int k = j + 1; k < R; ++k) {
            const double ujk = lane_bcast(uj, k);
            if (k <= col) m[k] -= ujk * uj;
        }
    }
    // W = U^{-1} on the kept directions, column `col`: back substitution.
    double w[R];
#pragma unroll
    for (int i = 0; i < R; ++i) w[i] = 0.0;
#pragma unroll
    for (int i = R - 1; i >= 0; --i) {
        double acc = (i == col) ? 1.0 : 0.0;
#pragma unroll
        for (int k = i + 1; k < R; ++k) acc -= lane_bcast(u[i], k) * w[k];
        const double uii = lane_bcast(u[i], i);
        w[i] = (keep[i] && i <= col) ? acc / uii : 0.0;
    }
    if (lane < R) {
        double* wo = p.w + (size_t)slab * R * R;
#pragma unroll
        for (int i = 0; i < R; ++i) wo[i * R + col] = w[i];
    }
}

// score_t = ||y_t W||^2, W upper triangular; one thread per row.
template <int R>
__global__ __launch_bounds__(256) void dkv_leverage(DkvLaunch p) {
    __shared__ double ws[R][R];
    const int slab = blockIdx.z * p.hkv + blockIdx.y;
    const double* w = p.w + (size_t)slab * R * R;
    for (int x = threadIdx.x; x < R * R; x += blockDim.x) ws[x / R][x % R] = w[x];
    __syncthreads();
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    const int b = blockIdx.z;
    if (t >= seq_rows(p.sm, b, seq_phys(p.sm, b))) return;
    const float* y = p.y + ((size_t)slab * p.t_len + t) * R;
    double yv[R];
#pragma unroll
    for (int c = 0; c < R; c += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(y + c);
        yv[c] = v[0];
        yv[c + 1] = v[1];
        yv[c + 2] = v[2];
        yv[c + 3] = v[3];
    }
    double l = 0.0;
#pragma unroll
    for (int c = 0; c < R; ++c) {
        double z = 0.0;
#pragma unroll
        for (int i = 0; i <= c; ++i) z = fma(yv[i], ws[i][c], z);
        l = fma(z, z, l);
    }
    p.score[(size_t)slab * p.t_len + t] = (float)l;
}

// Box-Muller on Philox4x32-10 words; pair q -> elements 2q, 2q+1.
__global__ void gaussian_kernel(int64_t n, uint32_t c1, uint32_t c2, uint32_t k0, uint32_t k1,
                                uint16_t* out) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (2 * q >= n) return;
    const Philox4 r = philox4x32_10((uint32_t)q, c1, c2, 0u, k0, k1);
    const double u1 = ((double)r.x0 + 1.0) * 2.3283064365386963e-10;
    const double u2 = (double)r.x1 * 2.3283064365386963e-10;
    const double rad = sqrt(-2.0 * log(u1));
    double sn, cs;
    sincos(6.283185307179586 * u2, &sn, &cs);
    out[2 * q] = f32_to_bf16((float)(rad * cs));
    if (2 * q + 1 < n) out[2 * q + 1] = f32_to_bf16((float)(rad * sn));
}

}  // namespace

hipError_t launch_dkv(const DkvLaunch& p, hipStream_t st) {
    const dim3 grid(p.nsplit, p.hkv, p.nb);
    const dim3 sgrid(p.hkv, p.nb);
    const dim3 lgrid((p.t_len + 255) / 256, p.hkv, p.nb);
    auto sketch = [&](auto rank_tag) {
        constexpr int RK = decltype(rank_tag)::value;
        if (p.v_rows) {
            if (p.range)
                hipLaunchKernelGGL((dkv_sketch<RK, true, true>), grid, dim3(256), 0, st, p);
            else
                hipLaunchKernelGGL((dkv_sketch<RK, false, true>), grid, dim3(256), 0, st, p);
        } else {
            if (p.range)
                hipLaunchKernelGGL((dkv_sketch<RK, true, false>), grid, dim3(256), 0, st, p);
            else
                hipLaunchKernelGGL((dkv_sketch<RK, false, false>), grid, dim3(256), 0, st, p);
        }
        hipLaunchKernelGGL(dkv_factor<RK>, sgrid, dim3(64), 0, st, p);
        hipLaunchKernelGGL(dkv_leverage<RK>, lgrid, dim3(256), 0, st, p);
    };
    if (p.rank == 16)
        sketch(std::integral_constant<int, 16>{});
    else
        sketch(std::integral_constant<int, 32>{});
    return hipGetLastError();
}

hipError_t launch_gaussian(int64_t n, uint32_t c1, uint32_t c2, uint32_t k0, uint32_t k1,
                           void* out, hipStream_t st) {
    const int64_t pairs = (n + 1) / 2;
    const int64_t blocks = (pairs + 255) / 256;
    hipLaunchKernelGGL(gaussian_kernel, dim3((unsigned)blocks), dim3(256), 0, st, n, c1, c2, k0,
                       k1, (uint16_t*)out);
    return hipGetLastError();
}

}  // namespace kvc
