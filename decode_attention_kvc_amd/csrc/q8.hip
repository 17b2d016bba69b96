// Range-protected per-token int8 KV cache: quantization, append, decode
// attention.
//
// VASE summary (gist.science 2606.03928), §3 (third contribution) and §5:
// value states of large range dominate the reconstruction error of per-token
// KV quantization, so the high-magnitude states should keep full precision.
// Format used here (the page gives none): each key row and each value row is
// quantized on its own, symmetric int8 with a float32 scale
// max|x| / 127 and codes round-half-even(x / scale); the P rows of largest
// value range per slab keep bf16 keys and values in a side mini-slab, and
// their int8 slots are flagged by a negative key scale.  Codes are stored
// biased (code + 128, an unsigned byte) so that v_cvt_f32_ubyte turns each
// byte into an fp16 MFMA operand with one byte permute per two values: the
// halfword 0x64uu is the fp16 number 1024 + uu, i.e. 1152 + code.  The offset
// is removed after the products: q . (1152 + c) = q . (1152 + c) - 1152 sum(q),
// and likewise with the running sum of p * scale for the values.  Products
// of these integers with fp16 queries / P are exact in the float32
// accumulators.
//
// Layouts (per slab): codes K [t_cap][128] (row-major, 128 bytes a row),
// codes V [t_cap/32][128][32] (32-token tiles, channel-major, 4 KB a tile),
// scales sk, sv [t_cap] float32; protected rows K [p_cap][128] and V in
// 32-token tiles, bf16, like a cache slab.  A 32-row tile of codes and
// scales is 8448 bytes against 16384 for bf16.
//
// Decode attention follows the bf16 kernel (split-K, four waves per
// workgroup, S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16, P
// split into two bf16 halves, the same permuted K-row order) with two tile
// kinds in one online softmax: quantized tiles (fp16 MFMA on the code
// operands, fp16 queries, P split into two fp16 halves, row scales folded
// into the logits and into P) and the slab's protected rows from the bf16
// mini-slab (bf16 MFMA as in the bf16 kernel).  Queries go to fp16 exactly
// for any normal value above 2^-14 in magnitude.  A lane's 32 key channels are
// contiguous here (channels 32*lg .. +32, so one row fragment is two 16-byte
// loads of codes) and the query fragments use the same channel order.
#include <type_traits>

#include "common.h"
#include "kvc_internal.h"
#include "merge.h"

namespace kvc {

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr int QT = 32;                 // rows per tile
constexpr int QMAX = 127;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8v __attribute__((ext_vector_type(8)));

constexpr float CODE_OFFSET = 1152.f;
constexpr float M_FLOOR = -1e30f;      // below any logit of a finite cache   // fp16 0x64uu = 1024 + uu, uu = code + 128

// Four biased codes (one dword) -> two dwords of fp16 halfwords 0x64uu.
__device__ __forceinline__ uint32_t codes_lo_f16(uint32_t w) {
    return __builtin_amdgcn_perm(0x64646464u, w, 0x04010400u);
}
__device__ __forceinline__ uint32_t codes_hi_f16(uint32_t w) {
    return __builtin_amdgcn_perm(0x64646464u, w, 0x04030402u);
}
__device__ __forceinline__ f16x8 codes8_f16(uint32_t w0, uint32_t w1) {
    return __builtin_bit_cast(f16x8, u32x4{codes_lo_f16(w0), codes_hi_f16(w0), codes_lo_f16(w1),
                                           codes_hi_f16(w1)});
}

__device__ __forceinline__ bf16x8 as_bf(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// Code of x for a row of scale s > 0: round-half-even(x / s), clamped, biased.
__device__ __forceinline__ uint32_t quant_byte(float x, float s) {
    float c = rintf(x / s);
    c = fminf(fmaxf(c, -(float)QMAX), (float)QMAX);
    return (uint32_t)((int)c + 128);
}

__device__ __forceinline__ bool is_protected(const int32_t* prot, int n, int t) {
    int lo = 0, hi = n;            // first index with prot[i] >= t
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (prot[mid] < t) lo = mid + 1; else hi = mid;
    }
    return lo < n && prot[lo] == t;
}

// ---------------------------------------------------------------------------
// Quantization of a bf16 slot: one workgroup (256 threads) per 32-row tile.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void q8_quantize_kernel(Q8QuantLaunch p) {
    __shared__ float vabs[D][QT + 1];
    __shared__ float vscale[QT];
    __shared__ int prot_flag[QT];
    const int tile = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int slab = b * p.hkv + j;
    const int tid = threadIdx.x;
    const int T = p.t_len;
    const int t0 = tile * QT;
    const uint16_t* ks = reinterpret_cast<const uint16_t*>(p.k) + (size_t)slab * p.src_t_cap * D;
    const uint16_t* vs = reinterpret_cast<const uint16_t*>(p.v) + (size_t)slab * p.src_t_cap * D;
    uint8_t* kq = reinterpret_cast<uint8_t*>(p.kq) + (size_t)slab * p.dst_t_cap * D;
    uint8_t* vq = reinterpret_cast<uint8_t*>(p.vq) + (size_t)slab * p.dst_t_cap * D;
    float* sk = p.sk + (size_t)slab * p.dst_t_cap;
    float* sv = p.sv + (size_t)slab * p.dst_t_cap;
    if (tid < QT)
        prot_flag[tid] = t0 + tid < T &&
                         is_protected(p.protect + (size_t)slab * p.n_protect, p.n_protect, t0 + tid);

    // Keys: thread (row r = tid/8, chunk c = tid%8) holds 16 channels.
    {
        const int r = tid / 8, c = tid % 8, t = t0 + r;
        float x[16];
        float amax = 0.f;
        if (t < T) {
            const u32x4 a = load16(ks + (size_t)t * D + 16 * c);
            const u32x4 bq = load16(ks + (size_t)t * D + 16 * c + 8);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                x[2 * w] = bf16lo(a[w]);
                x[2 * w + 1] = bf16hi(a[w]);
                x[8 + 2 * w] = bf16lo(bq[w]);
                x[8 + 2 * w + 1] = bf16hi(bq[w]);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
        }
#pragma unroll
        for (int m = 1; m < 8; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
        __syncthreads();
        if (t < T) {
            const bool prot = prot_flag[r];
            const float s = amax / (float)QMAX;
            uint32_t w[4] = {0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
            if (!prot && s > 0.f) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w[q] = quant_byte(x[4 * q], s) | (quant_byte(x[4 * q + 1], s) << 8) |
                           (quant_byte(x[4 * q + 2], s) << 16) | (quant_byte(x[4 * q + 3], s) << 24);
            }
            *reinterpret_cast<u32x4*>(kq + (size_t)t * D + 16 * c) = u32x4{w[0], w[1], w[2], w[3]};
            if (c == 0) sk[t] = prot ? -1.f : s;
        }
    }
    // Values: thread (channel d = tid/2, half h = tid%2) holds tokens
    // 16h .. 16h+15 of the tile; per-token absolute maxima meet in LDS.
    {
        const int d = tid / 2, h = tid % 2;
        const uint16_t* src = vs + vt_off(t0, d) + 16 * h;
        const u32x4 a = load16(src), bq = load16(src + 8);
        float x[16];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            x[2 * w] = bf16lo(a[w]);
            x[2 * w + 1] = bf16hi(a[w]);
            x[8 + 2 * w] = bf16lo(bq[w]);
            x[8 + 2 * w + 1] = bf16hi(bq[w]);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) vabs[d][16 * h + e] = fabsf(x[e]);
        __syncthreads();
        if (tid < QT) {
            float amax = 0.f;
            for (int dd = 0; dd < D; ++dd) amax = fmaxf(amax, vabs[dd][tid]);
            const float s = amax / (float)QMAX;
            vscale[tid] = (prot_flag[tid] || t0 + tid >= T) ? 0.f : s;
            if (t0 + tid < T) sv[t0 + tid] = vscale[tid];
        }
        __syncthreads();
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tok = 16 * h + 4 * q + e;
                const float s = vscale[tok];
                const uint32_t byte = s > 0.f ? quant_byte(x[4 * q + e], s) : 0x80u;
                word |= byte << (8 * e);
            }
            w[q] = word;
        }
        if (t0 < T)
            *reinterpret_cast<u32x4*>(vq + (size_t)tile * QT * D + d * QT + 16 * h) =
                u32x4{w[0], w[1], w[2], w[3]};
    }
}

// Append: row t_len - 1 of every slab from bf16 [nb][hkv][D] rows; one wave
// per slab, two channels per lane.  Appended rows are never protected.
__global__ __launch_bounds__(64) void q8_append_kernel(Q8QuantLaunch p) {
    const int j = blockIdx.x, b = blockIdx.y;
    const int slab = b * p.hkv + j;
    const int lane = threadIdx.x;
    const int t = p.t_len - 1;
    const uint32_t kw = reinterpret_cast<const uint32_t*>(p.k_row)[(size_t)slab * (D / 2) + lane];
    const uint32_t vw = reinterpret_cast<const uint32_t*>(p.v_row)[(size_t)slab * (D / 2) + lane];
    const float k0 = bf16lo(kw), k1 = bf16hi(kw), v0 = bf16lo(vw), v1 = bf16hi(vw);
    float ka = fmaxf(fabsf(k0), fabsf(k1)), va = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        ka = fmaxf(ka, __shfl_xor(ka, m));
        va = fmaxf(va, __shfl_xor(va, m));
    }
    const float ssk = ka / (float)QMAX, ssv = va / (float)QMAX;
    uint8_t* kq = reinterpret_cast<uint8_t*>(p.kq) + (size_t)slab * p.dst_t_cap * D;
    uint8_t* vq = reinterpret_cast<uint8_t*>(p.vq) + (size_t)slab * p.dst_t_cap * D;
    const uint32_t kb0 = ssk > 0.f ? quant_byte(k0, ssk) : 0x80u;
    const uint32_t kb1 = ssk > 0.f ? quant_byte(k1, ssk) : 0x80u;
    *reinterpret_cast<uint16_t*>(kq + (size_t)t * D + 2 * lane) = (uint16_t)(kb0 | (kb1 << 8));
    const size_t vbase = (size_t)(t / QT) * QT * D + (t % QT);
    vq[vbase + (size_t)(2 * lane) * QT] = (uint8_t)(ssv > 0.f ? quant_byte(v0, ssv) : 0x80u);
    vq[vbase + (size_t)(2 * lane + 1) * QT] = (uint8_t)(ssv > 0.f ? quant_byte(v1, ssv) : 0x80u);
    if (lane == 0) {
        p.sk[(size_t)slab * p.dst_t_cap + t] = ssk;
        p.sv[(size_t)slab * p.dst_t_cap + t] = ssv;
    }
}

// Cache row that lane (l16) of column block c covers inside a 32-row tile
// (the S^T fragment of lane group lg then covers tile rows 8*lg .. 8*lg+7).
__device__ __forceinline__ int tile_row(int c, int l16) {
    return 8 * (l16 >> 2) + 4 * c + (l16 & 3);
}

struct Q8Regs {
    u32x4 k[2][2];      // codes: [column block c][16-byte half]
    uint32_t v[8][2];   // codes: [d tile] 8 tokens
    f32x4 sk[2], sv[2]; // scales of tile rows 8*lg .. 8*lg+7
};

__device__ __forceinline__ void load_q8(Q8Regs& R, const uint8_t* kq, const uint8_t* vq,
                                        const float* sk, const float* sv, int t0, int l16,
                                        int lg) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const uint8_t* kr = kq + (size_t)(t0 + tile_row(c, l16)) * D + 32 * lg;
        R.k[c][0] = load_stream16(kr);
        R.k[c][1] = load_stream16(kr + 16);
    }
    const uint8_t* vt = vq + (size_t)(t0 / QT) * QT * D + 8 * lg;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
        const u32x2 x = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2*>(vt + (16 * dt + l16) * QT));
        R.v[dt][0] = x[0];
        R.v[dt][1] = x[1];
    }
    R.sk[0] = *reinterpret_cast<const f32x4*>(sk + t0 + 8 * lg);
    R.sk[1] = *reinterpret_cast<const f32x4*>(sk + t0 + 8 * lg + 4);
    R.sv[0] = *reinterpret_cast<const f32x4*>(sv + t0 + 8 * lg);
    R.sv[1] = *reinterpret_cast<const f32x4*>(sv + t0 + 8 * lg + 4);
}

template <int NT>
__global__ __launch_bounds__(256) void attn_q8_kernel(Q8AttnLaunch P) {
    constexpr int W = 4;
    constexpr int RP = 16 * NT;
    const AttnLaunch& p = P.a;
    const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int slab = b * p.hkv + j;
    const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
    const int l16 = lane & 15, lg = lane >> 4;
    const int T = p.t_len;
    const int nq = P.nq_tiles;
    const int ntiles = nq + (P.p_len + QT - 1) / QT;
    const int tile_begin = s * p.tps;
    const int tile_end = min(tile_begin + p.tps, ntiles);

    const uint8_t* kq = reinterpret_cast<const uint8_t*>(p.k) + (size_t)slab * p.t_cap * D;
    const uint8_t* vq = reinterpret_cast<const uint8_t*>(p.v) + (size_t)slab * p.t_cap * D;
    const float* sk = P.sk + (size_t)slab * p.t_cap;
    const float* sv = P.sv + (size_t)slab * p.t_cap;
    const uint16_t* kp = reinterpret_cast<const uint16_t*>(P.kp) + (size_t)slab * P.p_cap * D;
    const uint16_t* vp = reinterpret_cast<const uint16_t*>(P.vp) + (size_t)slab * P.p_cap * D;

    // Query fragments, channel chunk kc of lane group lg = channels
    // 32*lg + 8*kc .. +8 (the codes' order), in bf16 (protected rows) and in
    // fp16 (codes); qsum = sum of the row's fp16 channels.
    bf16x8 qB[NT][4];
    f16x8 qH[NT][4];
    float qsum[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int r = nt * 16 + l16;
        float part = 0.f;
        if (r < p.rows) {
            const int qi = r / p.g, h = j * p.g + r % p.g;
            const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + p.q_off[qi] +
                                 ((size_t)b * p.hq + h) * D + 32 * lg;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const u32x4 x = load16(qp + 8 * kc);
                qB[nt][kc] = as_bf(x);
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    const _Float16 lo = (_Float16)bf16lo(x[w2]), hi = (_Float16)bf16hi(x[w2]);
                    qH[nt][kc][2 * w2] = lo;
                    qH[nt][kc][2 * w2 + 1] = hi;
                    part += (float)lo + (float)hi;
                }
            }
        } else {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                qB[nt][kc] = as_bf(u32x4{0u, 0u, 0u, 0u});
                qH[nt][kc] = __builtin_bit_cast(f16x8, u32x4{0u, 0u, 0u, 0u});
            }
        }
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        qsum[nt] = part;
    }

    // The running maxima start at a finite floor, so masked logits (-inf)
    // always give p = 0 without a guard, even before the first visible row.
    f32x4 acc[NT][8];
    float m[NT], lsum[NT], psum[NT];   // psum: sum of p * value scale (offset removal)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        m[nt] = M_FLOOR;
        lsum[nt] = 0.f;
        psum[nt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[nt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float scale = p.scale;

    // Online softmax step shared by both tile kinds: x[jj] are the logits of
    // tile rows 8*lg + jj, pv[jj] the factor each row's p is multiplied by
    // before the value product, V the value fragments.
    // F16: code tiles (fp16 P halves and value operands, offset mass
    // tracked in psum); otherwise bf16 protected rows.
    auto softmax_pv = [&](int nt, const float (&x)[8], const float (&pv)[8], const u32x4 (&V)[8],
                          auto f16_tag) {
        constexpr bool F16 = decltype(f16_tag)::value;
        float mx = x[0];
#pragma unroll
        for (int jj = 1; jj < 8; ++jj) mx = fmaxf(mx, x[jj]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // The reference maximum only moves when a logit exceeds it by more
        // than 2^8 in p (then p <= 256 against a stale reference, harmless in
        // float32 and in the fp16/bf16 halves); the accumulators are rescaled
        // only on the (wave-uniform) tiles where some row moved.
        const bool move = (mx - m[nt]) * LOG2E > 8.f;
        const float mnew = move ? mx : m[nt];
        const float alpha = exp2f((m[nt] - mnew) * LOG2E);
        const bool any_move = __ballot(move) != 0;
        m[nt] = mnew;
        float ps = 0.f, pss = 0.f;
        u16x8 hi, lo;
        f16x8 hh, ll;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const float pj = exp2f((x[jj] - mnew) * LOG2E);
            ps += pj;
            const float pw = pj * pv[jj];
            if constexpr (F16) {
                const _Float16 h = (_Float16)pw;
                hh[jj] = h;
                ll[jj] = (_Float16)(pw - (float)h);
                pss += pw;
            } else {
                const uint16_t h16 = f32_to_bf16(pw);
                hi[jj] = h16;
                lo[jj] = f32_to_bf16(pw - bf16_to_f32(h16));
            }
        }
        lsum[nt] = lsum[nt] * alpha + ps;
        psum[nt] = psum[nt] * alpha + pss;
        if (any_move) {
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) acc[nt][dt] *= alpha;
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            if constexpr (F16) {
                const f16x8 vf = __builtin_bit_cast(f16x8, V[dt]);
                acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, hh, acc[nt][dt], 0, 0, 0);
                acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, ll, acc[nt][dt], 0, 0, 0);
            } else {
                const bf16x8 pH = __builtin_bit_cast(bf16x8, hi);
                const bf16x8 pL = __builtin_bit_cast(bf16x8, lo);
                acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(V[dt]), pH, acc[nt][dt], 0, 0, 0);
                acc[nt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(V[dt]), pL, acc[nt][dt], 0, 0, 0);
            }
        }
    };
    using F16Tiles = std::integral_constant<bool, true>;
    using BF16Tiles = std::integral_constant<bool, false>;

    // A tile of codes.  TAIL: rows at or past t_len are masked.
    auto compute_q8 = [&](const Q8Regs& R, int t0, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        u32x4 KF[2][4], V[8];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
                KF[c][kc] = __builtin_bit_cast(
                    u32x4, codes8_f16(R.k[c][kc / 2][2 * (kc % 2)], R.k[c][kc / 2][2 * (kc % 2) + 1]));
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
            V[dt] = __builtin_bit_cast(u32x4, codes8_f16(R.v[dt][0], R.v[dt][1]));
        float skr[8], svr[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            skr[i] = R.sk[0][i];
            skr[4 + i] = R.sk[1][i];
            svr[i] = R.sv[0][i];
            svr[4 + i] = R.sv[1][i];
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 S[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                S[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kc = 0; kc < 4; ++kc)
                    S[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, KF[c][kc]),
                                                                   qH[nt][kc], S[c], 0, 0, 0);
            }
            // S[c][i]: tile row 8*lg + 4*c + i
            const float bias = CODE_OFFSET * qsum[nt];
            float x[8], pv[8];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int jj = 4 * c + i;
                    const float sc = skr[jj];
                    float v = (S[c][i] - bias) * sc * scale;
                    bool keep = sc >= 0.f;
                    float w = svr[jj];
                    if constexpr (TAIL) {
                        const bool in = t0 + 8 * lg + jj < T;
                        keep = keep && in;
                        w = in ? w : 0.f;
                    }
                    x[jj] = keep ? v : -INFINITY;
                    pv[jj] = w;
                }
            softmax_pv(nt, x, pv, V, F16Tiles{});
        }
    };

    // A tile of protected bf16 rows (always masked against p_len).
    auto compute_prot = [&](int tp) {
        const int r0 = tp * QT;
        u32x4 KF[2][4], V[8];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint16_t* kr = kp + (size_t)(r0 + tile_row(c, l16)) * D + 32 * lg;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) KF[c][kc] = load16(kr + 8 * kc);
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) V[dt] = load16(vp + vt_off(r0, 16 * dt + l16) + 8 * lg);
        // rows past p_len hold arbitrary bits: zero their values (0 * NaN)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            u16x8 e = __builtin_bit_cast(u16x8, V[dt]);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) e[jj] = (r0 + 8 * lg + jj < P.p_len) ? e[jj] : (uint16_t)0;
            V[dt] = __builtin_bit_cast(u32x4, e);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            f32x4 S[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                S[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kc = 0; kc < 4; ++kc)
                    S[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(KF[c][kc]), qB[nt][kc], S[c], 0, 0, 0);
            }
            float x[8], pv[8];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int jj = 4 * c + i;
                    x[jj] = (r0 + 8 * lg + jj < P.p_len) ? S[c][i] * scale : -INFINITY;
                    pv[jj] = 1.f;
                }
            softmax_pv(nt, x, pv, V, BF16Tiles{});
        }
    };
    using Interior = std::integral_constant<bool, false>;
    using Last = std::integral_constant<bool, true>;

    // Interior quantized tiles of this split, two tiles of loads in flight
    // per wave (unconditional loads inside the loop body).
    const int last_q = nq - 1;                  // the quantized tile that may be partial
    const int main_end = min(tile_end, last_q);
    const int n_main = max(0, main_end - tile_begin);
    const int n = wave < n_main ? (n_main - wave + W - 1) / W : 0;
    auto t0_of = [&](int k) { return (tile_begin + wave + k * W) * QT; };
    if (n > 0) {
        Q8Regs RA, RB;
        load_q8(RA, kq, vq, sk, sv, t0_of(0), l16, lg);
        int k = 0;
        for (; k + 2 < n; k += 2) {
            load_q8(RB, kq, vq, sk, sv, t0_of(k + 1), l16, lg);
            compute_q8(RA, t0_of(k), Interior{});
            load_q8(RA, kq, vq, sk, sv, t0_of(k + 2), l16, lg);
            compute_q8(RB, t0_of(k + 1), Interior{});
        }
        if (k + 1 < n) {
            load_q8(RB, kq, vq, sk, sv, t0_of(k + 1), l16, lg);
            compute_q8(RA, t0_of(k), Interior{});
            compute_q8(RB, t0_of(k + 1), Interior{});
        } else {
            compute_q8(RA, t0_of(k), Interior{});
        }
    }
    // The remaining tiles of the range (the last quantized tile and the
    // protected tiles), continuing the round-robin.
    for (int tile = max(tile_begin, main_end); tile < tile_end; ++tile) {
        if ((tile - tile_begin) % W != wave) continue;
        if (tile < nq) {
            Q8Regs R;
            load_q8(R, kq, vq, sk, sv, tile * QT, l16, lg);
            compute_q8(R, tile * QT, Last{});
        } else {
            compute_prot(tile - nq);
        }
    }

    // Row sums (and the biased value mass) over the four lane groups; remove
    // the code bias from the accumulators.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        lsum[nt] += __shfl_xor(lsum[nt], 16);
        lsum[nt] += __shfl_xor(lsum[nt], 32);
        psum[nt] += __shfl_xor(psum[nt], 16);
        psum[nt] += __shfl_xor(psum[nt], 32);
        const float corr = CODE_OFFSET * psum[nt];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[nt][dt] -= corr;
    }

    // Merge the four waves through LDS and write the partial (or, with one
    // split per slab, the finished rows).
    __shared__ float buf[W * 16 * D];
    __shared__ float wm[W][16], wl[W][16];
    constexpr int EPT = 2048 / (W * 64);
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
            const int nrow = tid / (D / EPT), d0 = (tid % (D / EPT)) * EPT;
            float M = wm[0][nrow];
#pragma unroll
            for (int w = 1; w < W; ++w) M = fmaxf(M, wm[w][nrow]);
            float f[W], L = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                f[w] = exp2f((wm[w][nrow] - M) * LOG2E);
                L += f[w] * wl[w][nrow];
            }
            float o[EPT];
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                float a = 0.f;
#pragma unroll
                for (int w = 0; w < W; ++w) a += f[w] * buf[(w * 16 + nrow) * D + d0 + e];
                o[e] = a;
            }
            const int r = nt * 16 + nrow;
            if (p.nsplit == 1) {
                if (r < p.rows) {
                    const float inv = 1.f / L;
                    const int qi = r / p.g, h = j * p.g + r % p.g;
                    float* dst = p.out + p.out_off[qi] + ((size_t)b * p.hq + h) * D + d0;
#pragma unroll
                    for (int e = 0; e < EPT; e += 4)
                        *reinterpret_cast<f32x4*>(dst + e) =
                            f32x4{o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv};
                    if (d0 == 0 && p.lse) p.lse[p.lse_off[qi] + (size_t)b * p.hq + h] = M + logf(L);
                }
            } else if (p.arrive) {
                if (r < p.rows) store_part_coh<EPT>(p, part_acc, part_ml, r, d0, o, M, L);
            } else {
                float* dst = part_acc + (size_t)r * D + d0;
#pragma unroll
                for (int e = 0; e < EPT; e += 4)
                    *reinterpret_cast<f32x4*>(dst + e) = f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]};
                if (d0 == 0) {
                    part_ml[r * 2] = M;
                    part_ml[r * 2 + 1] = L;
                }
            }
        }
        __syncthreads();
    }
    if (p.nsplit > 1 && p.arrive && arrive_last(p.arrive + slab, p.nsplit))
        combine_rows<W * 64, true>(p, j, b, 0, p.rows, buf);
}

}  // namespace

hipError_t launch_q8_quantize(const Q8QuantLaunch& p, hipStream_t st) {
    if (p.k_row) {
        hipLaunchKernelGGL(q8_append_kernel, dim3(p.hkv, p.nb), dim3(64), 0, st, p);
    } else {
        const dim3 grid((p.t_len + QT - 1) / QT, p.hkv, p.nb);
        hipLaunchKernelGGL(q8_quantize_kernel, grid, dim3(256), 0, st, p);
    }
    return hipGetLastError();
}

hipError_t launch_attn_q8(const Q8AttnLaunch& p, int nt, hipStream_t st) {
    const dim3 grid(p.a.nsplit, p.a.hkv, p.a.nb);
    if (nt == 1)
        hipLaunchKernelGGL(attn_q8_kernel<1>, grid, dim3(256), 0, st, p);
    else if (nt == 2)
        hipLaunchKernelGGL(attn_q8_kernel<2>, grid, dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL(attn_q8_kernel<4>, grid, dim3(256), 0, st, p);
    if (p.a.nsplit > 1 && !p.a.arrive) return launch_attn_combine(p.a, st);
    return hipGetLastError();
}

}  // namespace kvc
