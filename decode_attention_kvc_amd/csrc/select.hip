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
// Two launches.  select_keys_kernel computes the sampling key of every
// candidate row of every slab (Philox + log1p in double: the only heavy
// arithmetic, spread over the whole chip) into the workspace.  Then one
// workgroup of 1024 threads per slab makes both "k best" decisions as exact
// radix selections on 32-bit order-preserving keys: 8-bit digits with LDS
// histograms (the first counted while the keys are stored, further ones only
// while the bin holding the k-th key is not taken whole) find the cut; rows
// strictly before it are in, rows at it are taken in ascending row order.  The row-ordered
// steps (which of the rows tied at a threshold are taken, and the ascending
// emission of the kept rows) give each thread a contiguous run of rows and
// need one block-wide scan of per-thread counts each, not one per 1024 rows.
// The keys (first the range keys, then, in place, the sampling keys) live in
// LDS when the slab has at most LDS_KEYS rows, otherwise in the caller's
// workspace; all accesses stay inside one workgroup.
#include "common.h"
#include "kvc_internal.h"
#include "philox.h"
#include "radix.h"

namespace kvc {

namespace {

constexpr int NT = SELECT_THREADS;
constexpr int NWV = NT / WAVE;
constexpr uint32_t EXCLUDED = 0xFFFFFFFFu;   // above every float key: a protected row
constexpr uint32_t TIE_R = 0xFFFFFFFEu;      // range key at the threshold, order not yet decided
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

// Sampling key of every candidate row [0, T - B) of every evicting slab.
__global__ __launch_bounds__(256) void select_keys_kernel(SelectLaunch p) {
    const int slab = blockIdx.y;
    const int b = slab / p.hkv, j = slab % p.hkv;
    const int T = p.len ? min(max(p.len[b], 0), p.t_len) : p.t_len;
    if (T <= p.budget_k + p.recent_b) return;       // keeps everything
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T - p.recent_b) return;
    const uint32_t seq = p.seq_id ? (uint32_t)p.seq_id[b] : (uint32_t)b;
    p.kappa[(size_t)slab * p.t_len + t] = sample_key(p, t, j, seq, p.score[(size_t)slab * p.t_len + t]);
}

template <bool IN_LDS>
__global__ __launch_bounds__(NT) void select_kernel(SelectLaunch p) {
    __shared__ SelectSmem sm;
    __shared__ uint32_t lds_keys[IN_LDS ? LDS_KEYS : 1];
    const int slab = blockIdx.x;
    const int b = slab / p.hkv;
    const int tid = threadIdx.x;
    // Ragged batches: the slab's own row count T (at most t_len, which is
    // the row stride of score / range / keys) and kept stride min(t_len, K+B);
    // kept entries past the slab's min(T, K+B) are -1.
    const int T = p.len ? min(max(p.len[b], 0), p.t_len) : p.t_len;
    const int kb = p.budget_k + p.recent_b;
    const int stride = min(p.t_len, kb);
    int32_t* kept = p.kept + (size_t)slab * stride;
    if (T <= kb) {
        for (int t = tid; t < stride; t += NT) kept[t] = t < T ? t : -1;
        return;
    }
    const int n_keep = kb;
    const float* range = p.range + (size_t)slab * p.t_len;
    const uint32_t* kap = p.kappa + (size_t)slab * p.t_len;
    uint32_t* keys = IN_LDS ? lds_keys : p.keys + (size_t)slab * p.t_len;
    const int ncand = T - p.recent_b;

    // First-digit histograms are counted while the keys are stored.  Keys of
    // one magnitude share their top byte, so a wave whose active lanes all
    // fall in one bin adds them with a single atomic.
    constexpr int PITCH = SelectSmem::PITCH;
    uint32_t* hist = sm.hist + (tid % 8) * PITCH;
    auto count_top8 = [&](uint32_t u, bool add) {
        const uint32_t bin = u >> 24;
        const unsigned long long want = __ballot(add);
        if (want == 0) return;
        const int first = __ffsll((long long)want) - 1;
        const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
        const unsigned long long same = __ballot(add && bin == b0);
        if (same == want) {
            if ((tid % WAVE) == first) atomicAdd(&hist[b0], (uint32_t)__popcll(want));
        } else if (add) {
            atomicAdd(&hist[bin], 1u);
        }
    };
    auto clear_hist = [&]() {
        for (int i = tid; i < 8 * PITCH; i += NT) sm.hist[i] = 0;
        __syncthreads();
    };

    // 1. N_v candidates of largest range (ties to the lower row): the range
    //    keys below rpre under rmask, and the first rtake of those equal to
    //    it (all rcnt of them when rtake == rcnt).
    uint32_t rpre = 0, rmask = 0, rtake = 0, rcnt = 0;
    if (p.n_v > 0) {
        clear_hist();
        for (int t = tid; t < ncand; t += NT) {
            const uint32_t u = range_key(range[t]);
            keys[t] = u;
            count_top8(u, true);
        }
        __syncthreads();
        rpre = radix_select<NT>(ncand, (uint32_t)p.n_v, [&](int t) { return keys[t]; }, sm,
                                &rmask, &rtake, &rcnt);
    }
    const bool split_r = p.n_v > 0 && rtake != rcnt;   // some rows at the range cut are left out

    // 2. Sampling keys over the range keys; rows before the range cut are
    //    protected (EXCLUDED), rows at it too when the cut keeps them all,
    //    else they are marked and then protected in row order (the first
    //    rtake of them); the others get their key.
    clear_hist();
    for (int t = tid; t < ncand; t += NT) {
        uint32_t u = kap[t];
        if (p.n_v > 0) {
            const uint32_t rm = keys[t] & rmask;
            if (rm < rpre) u = EXCLUDED;
            else if (rm == rpre) u = split_r ? TIE_R : EXCLUDED;
        }
        keys[t] = u;
        count_top8(u, u != TIE_R);        // a marked row is counted once it is resolved
    }
    __syncthreads();
    if (split_r) {
        const int c = (ncand + NT - 1) / NT, lo = min(ncand, tid * c), hi = min(ncand, lo + c);
        uint32_t n = 0;
        for (int t = lo; t < hi; ++t) n += keys[t] == TIE_R;
        uint32_t tot;
        uint32_t rank = block_scan_u32<NT>(n, sm, &tot);
        for (int t = lo; t < hi; ++t)
            if (keys[t] == TIE_R) {
                const uint32_t u = rank++ < rtake ? EXCLUDED : kap[t];
                keys[t] = u;
                atomicAdd(&hist[u >> 24], 1u);
            }
        __syncthreads();
    }

    // 3. K - N_v smallest sampling keys: below kpre under kmask, and the
    //    first ktake of those equal to it (all kcnt when ktake == kcnt).
    const uint32_t ns = (uint32_t)(p.budget_k - p.n_v);
    uint32_t kpre = 0, kmask = 0, ktake = 0, kcnt = 0;
    if (ns > 0)
        kpre = radix_select<NT>(ncand, ns, [&](int t) { return keys[t]; }, sm, &kmask, &ktake, &kcnt);

    // 4. Emit the kept rows in ascending order: each thread owns a run of
    //    rows; its offset is the kept rows before the run (the sure ones, and
    //    the first ktake rows at the sampling cut, in row order).
    {
        const int c = (T + NT - 1) / NT, lo = min(T, tid * c), hi = min(T, lo + c);
        auto sure = [&](int t, uint32_t u) {
            return t >= ncand || u == EXCLUDED || (ns > 0 && (u & kmask) < kpre);
        };
        auto at_cut = [&](uint32_t u) { return ns > 0 && u != EXCLUDED && (u & kmask) == kpre; };
        const bool split_k = ktake != kcnt;   // some rows at the cut are left out
        uint32_t nsure = 0, neq = 0;
        for (int t = lo; t < hi; ++t) {
            const uint32_t u = t < ncand ? keys[t] : 0u;
            if (sure(t, u) || (!split_k && at_cut(u))) ++nsure;
            else if (at_cut(u)) ++neq;
        }
        uint32_t tot;
        const uint32_t sure_off = block_scan_u32<NT>(nsure, sm, &tot);
        uint32_t eq_rank = split_k ? block_scan_u32<NT>(neq, sm, &tot) : 0u;
        uint32_t pos = sure_off + min(eq_rank, ktake);
        for (int t = lo; t < hi; ++t) {
            const uint32_t u = t < ncand ? keys[t] : 0u;
            bool keep = sure(t, u) || (!split_k && at_cut(u));
            if (split_k && at_cut(u)) keep = eq_rank++ < ktake;
            if (keep) {
                if (pos < (uint32_t)n_keep) kept[pos] = t;
                ++pos;
            }
        }
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
    if (p.t_len > p.budget_k + p.recent_b) {
        const dim3 kgrid((p.t_len - p.recent_b + 255) / 256, p.nb * p.hkv);
        hipLaunchKernelGGL(select_keys_kernel, kgrid, dim3(256), 0, st, p);
    }
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
