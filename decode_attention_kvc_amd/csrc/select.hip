// VASE selection: which rows of a slab survive an eviction pass.
//
// VASE summary (gist.science 2606.03928): §2 keeps a persistent budget K plus
// a recent buffer B; §2.A always keeps the N_v rows of largest value range;
// §2.B fills the rest of the budget by weighted random sampling (here:
// without replacement, proportional to the observation-window score).
// Sampling without replacement proportional to w is realised with
// exponential keys (Efraimidis and Spirakis, 2006): with E_t ~ Exp(1), the
// k rows of smallest E_t / w_t are a draw of that law.  E_t comes from word
// 0 of Philox4x32-10 at counter (t, kv head, layer, batch) and key (seed
// low, seed high): E_t = -ln((x_t + 1) / 2^32), evaluated in double with
// log1p so that words near 2^32 keep full relative accuracy.
//
// One workgroup of 1024 threads per slab.  Both "k best" decisions are
// exact radix selections on 32-bit order-preserving keys: four passes of
// 8-bit digits with LDS histograms find the k-th key; rows strictly before
// it are in, rows equal to it are taken in ascending row order.  The kept
// rows are emitted in ascending order with block-wide ordered scans.
// The keys (first the range keys, then, in place, the sampling keys) live in
// LDS when the slab has at most LDS_KEYS rows, otherwise in the caller's
// workspace (one uint32 per row); all accesses stay inside one workgroup.
#include "common.h"
#include "kvc_internal.h"
#include "philox.h"
#include "radix.h"

namespace kvc {

namespace {

constexpr int NT = SELECT_THREADS;
constexpr int NWV = NT / WAVE;
constexpr uint32_t EXCLUDED = 0xFFFFFFFFu;   // above every float key
constexpr int LDS_KEYS = 36 * 1024;           // 144 KB of keys

using SelectSmem = RadixSmem<NT, 8>;   // 8 histogram copies: range keys share their top digit

__device__ __forceinline__ uint32_t range_key(float r) {
    // larger range first: invert the (non-negative) float's bits
    return ~__float_as_uint(r);
}

// Exponential key of row t; +inf when the weight is not positive.
__device__ __forceinline__ uint32_t sample_key(const SelectLaunch& p, int t, int j, uint32_t seq,
                                               float score) {
    if (!(score > 0.f)) return 0x7F800000u;
    const Philox4 r = philox4x32_10((uint32_t)t, (uint32_t)j, p.layer_id, seq, p.seed_lo,
                                    p.seed_hi);
    const double m = 4294967295.0 - (double)r.x0;          // 2^32 - 1 - x
    const double e = -log1p(-m * 2.3283064365386963e-10);  // -ln((x + 1) / 2^32)
    const float kappa = (float)(e / (double)score);
    return __float_as_uint(kappa);
}

template <bool IN_LDS>
__global__ __launch_bounds__(NT) void select_kernel(SelectLaunch p) {
    __shared__ SelectSmem sm;
    __shared__ uint32_t lds_keys[IN_LDS ? LDS_KEYS : 1];
    const int slab = blockIdx.x;
    const int b = slab / p.hkv, j = slab % p.hkv;
    const int tid = threadIdx.x;
    // Ragged batches: the slab's own row count T (at most t_len, which is
    // the row stride of score / range / keys) and kept stride min(t_len, K+B);
    // kept entries past the slab's min(T, K+B) are -1.
    const int T = p.len ? min(max(p.len[b], 0), p.t_len) : p.t_len;
    const uint32_t seq = p.seq_id ? (uint32_t)p.seq_id[b] : (uint32_t)b;
    const int kb = p.budget_k + p.recent_b;
    const int stride = min(p.t_len, kb);
    int32_t* kept = p.kept + (size_t)slab * stride;
    if (T <= kb) {
        for (int t = tid; t < stride; t += NT) kept[t] = t < T ? t : -1;
        return;
    }
    const int n_keep = kb;
    const float* score = p.score + (size_t)slab * p.t_len;
    const float* range = p.range + (size_t)slab * p.t_len;
    uint32_t* keys = IN_LDS ? lds_keys : p.keys + (size_t)slab * p.t_len;
    const int ncand = T - p.recent_b;

    // 1. N_v candidates of largest range (ties to the lower row).
    uint32_t rthr = 0, rtake = 0;
    if (p.n_v > 0) {
        for (int t = tid; t < ncand; t += NT) keys[t] = range_key(range[t]);
        __syncthreads();
        rthr = radix_select<NT>(ncand, (uint32_t)p.n_v, [&](int t) { return keys[t]; }, sm, &rtake);
    }

    // 2. Sampling keys for the remaining candidates, written over the range
    //    keys; protected rows are marked EXCLUDED.  Ordered pass: equal-range
    //    rows are protected in row order.
    uint32_t eq_seen = 0;
    for (int base = 0; base < ncand; base += NT) {
        const int t = base + tid;
        const bool valid = t < ncand;
        const uint32_t rk = (valid && p.n_v > 0) ? keys[t] : 0xFFFFFFFFu;
        const bool eq = valid && p.n_v > 0 && rk == rthr;
        uint32_t tot;
        const uint32_t rank = eq_seen + block_scan_flag<NT>(eq, sm, &tot);
        eq_seen += tot;
        if (valid) {
            const bool prot = p.n_v > 0 && (rk < rthr || (eq && rank < rtake));
            keys[t] = prot ? EXCLUDED : sample_key(p, t, j, seq, score[t]);
        }
    }
    __syncthreads();

    // 3. K - N_v smallest sampling keys.
    const uint32_t ns = (uint32_t)(p.budget_k - p.n_v);
    uint32_t kthr = 0, ktake = 0;
    if (ns > 0) kthr = radix_select<NT>(
        ncand, ns, [&](int t) { return keys[t]; }, sm, &ktake);

    // 4. Emit kept rows in ascending order.
    uint32_t written = 0, keq_seen = 0;
    for (int base = 0; base < T; base += NT) {
        const int t = base + tid;
        const bool valid = t < T;
        bool keep = false, eq = false;
        uint32_t u = 0;
        if (valid) {
            if (t >= ncand) {
                keep = true;
            } else {
                u = keys[t];
                eq = ns > 0 && u == kthr && u != EXCLUDED;
                keep = (u == EXCLUDED) || (ns > 0 && u < kthr);
            }
        }
        uint32_t tot;
        const uint32_t rank = keq_seen + block_scan_flag<NT>(eq, sm, &tot);
        keq_seen += tot;
        if (eq && rank < ktake) keep = true;
        const uint32_t pos = written + block_scan_flag<NT>(keep, sm, &tot);
        written += tot;
        if (keep && pos < (uint32_t)n_keep) kept[pos] = t;
    }
}

__global__ void philox_kernel(int64_t n, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                              uint32_t k1, uint32_t* out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const Philox4 r = philox4x32_10((uint32_t)i, c1, c2, c3, k0, k1);
    u32x4 v = u32x4{r.x0, r.x1, r.x2, r.x3};
    *reinterpret_cast<u32x4*>(out + 4 * i) = v;
}

}  // namespace

hipError_t launch_select(const SelectLaunch& p, hipStream_t st) {
    if (p.t_len <= LDS_KEYS)
        hipLaunchKernelGGL(select_kernel<true>, dim3(p.nb * p.hkv), dim3(NT), 0, st, p);
    else
        hipLaunchKernelGGL(select_kernel<false>, dim3(p.nb * p.hkv), dim3(NT), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_philox(int64_t n, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                         uint32_t k1, uint32_t* out, hipStream_t st) {
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(philox_kernel, dim3((unsigned)blocks), dim3(256), 0, st, n, c1, c2, c3, k0,
                       k1, out);
    return hipGetLastError();
}

}  // namespace kvc
