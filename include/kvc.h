/*
 * libkvc — decode attention over a compressed KV cache, for AMD MI355X
 * (gfx950).  Plain C ABI: every argument is a host value, a host pointer or a
 * device pointer; no C++ or framework types cross it.
 *
 * What the calls compute comes from three pages:
 *   [RCLA]  "Stochastic KV Routing" (aitrends.kr article on R-CLA),
 *           inference and implementation paragraphs: a fixed sharing set S of
 *           leader layers; every other layer reuses the KV of the nearest
 *           earlier leader, and only leaders store or update KV.
 *   [VASE]  "VASE: value-aware stochastic KV-cache eviction"
 *           (gist.science 2606.03928), §2 (periodic eviction with a
 *           persistent budget K and a recent buffer B), §2.A
 *           (Range(v) = max(v) - min(v); the N_v rows of largest range are
 *           always kept), §2.B (weighted random sampling on SnapKV-style
 *           observation-window attention scores), §1 (evicted pairs are
 *           discarded for good, giving a static footprint).
 *   [XKV]   "xKV: cross-layer KV-cache compression" (gist.science
 *           2503.18893), §2.2 (cross-layer factorisation of windows of W
 *           layers), §2.3 (selective reconstruction with landmark chunk
 *           selection).
 *   Decode attention itself is standard softmax attention, one query row
 *   per head, with grouped-query heads (GQA, named in [XKV] §4).
 *
 * Conventions shared by every call
 *   - Status: every call returns KVC_OK (0) or a negative kvc_status.  All
 *     arguments are validated on the host before anything is enqueued; on
 *     an error nothing is enqueued and no output is touched.  KVC_EHIP
 *     reports a launch failure seen right after enqueueing.
 *   - Streams: device work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream) and runs asynchronously; the call returns before
 *     it finishes.  Host outputs (kvc_share_map, *_ws_bytes) are ready on
 *     return.
 *   - Ownership: the caller allocates and owns all memory.  The library
 *     allocates nothing and keeps no state between calls; calls are
 *     reentrant.  Calls that share a workspace must be ordered on one stream.
 *     (The one exception, kvc_decode_attn_noalloc, uses a device array the
 *     library owns; see there.)
 *   - Alignment: cache, query and output pointers must be 16-byte aligned
 *     (KVC_EALIGN otherwise).
 *   - Sizes are element counts unless a name ends in _bytes.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t* kvc_stream_t;

typedef enum kvc_status {
    KVC_OK = 0,
    KVC_EINVAL = -1,      /* a size, index or set is out of range          */
    KVC_EDTYPE = -2,      /* unknown or mismatched element type            */
    KVC_EALIGN = -3,      /* a pointer is NULL or not 16-byte aligned      */
    KVC_EWORKSPACE = -4,  /* workspace missing or smaller than required    */
    KVC_EALIAS = -5,      /* source and destination memory overlap         */
    KVC_EHIP = -6,        /* the HIP runtime reported a launch error       */
    KVC_ESCRATCH = -7     /* the call needs more than the library's own
                             scratch array (no-allocation entry point)     */
} kvc_status;

typedef enum kvc_dtype {
    KVC_F32 = 0,          /* IEEE float32                                  */
    KVC_BF16 = 1          /* bfloat16 (upper half of a float32)            */
} kvc_dtype;

/* Head dimension the kernels are built for. */
#define KVC_HEAD_DIM 128
/* t_cap must be a multiple of this (keeps every vector access in bounds). */
#define KVC_T_ALIGN 64
/* Tokens per value tile. */
#define KVC_V_TILE 32

/*
 * A KV cache of n_slots leader slots (one per layer in S), nb_cap batch
 * entries, n_kv_heads heads and head_dim = 128.  One slab = one (slot, batch
 * entry, kv head).
 *   k: [n_slots][nb_cap][n_kv_heads][t_cap][head_dim]        row-major rows
 *   v: [n_slots][nb_cap][n_kv_heads][t_cap/32][head_dim][32] tiles of 32
 *      tokens, each tile channel-major: value V[t][c] of a slab sits at
 *      element (t/32)*head_dim*32 + c*32 + t%32.  A tile's values are one
 *      contiguous block, and the token-contiguous operand of the P*V product
 *      loads with one 16-byte access per lane.
 * dtype is a kvc_dtype; both k and v hold that type.
 *
 * v_layout (kvc_v_layout) says how v is stored:
 *   KVC_V_TILES (0, the default of a zero-initialised descriptor): the
 *     tiled layout above, which decode attention, appends, the int8 and
 *     sketch paths and compaction destinations use;
 *   KVC_V_ROWS (1): v stored like k, [n_slots][nb_cap][n_kv_heads][t_cap]
 *     [head_dim] rows -- the layout a prefill writes.  A rows cache is an
 *     input of the prompt compression: kvc_value_range, kvc_score (with the
 *     fused range), kvc_dkv_score and kvc_compact (as the source) read it, and kvc_compact
 *     re-lays the rows it gathers into a tiled destination (with kept =
 *     NULL it copies rows [0, n_keep): a bulk ingest).  Every other call
 *     returns KVC_EINVAL for it.
 *
 * A call addresses nb sequences.  Uniform batches (batch_idx = seq_len =
 * NULL, nb_cap = 0 or nb): sequence b is batch entry b and rows [0, t_len)
 * are valid in every slot.
 * Ragged batches (per-sequence lengths, and eviction passes that run on
 * each sequence's own steps):
 *   batch_idx: NULL or device int32 [nb]: sequence b is stored in batch
 *              entry batch_idx[b] (an entry outside [0, nb_cap) makes the
 *              sequence empty).  Lets a call address any subset of the
 *              entries, and lets a sequence move between entries (an
 *              eviction pass compacts it into a free entry).
 *   seq_len:   NULL or device int32 [nb]: sequence b holds rows
 *              [0, seq_len[b]) (entries are clamped to [0, t_len]).  t_len
 *              is then the bound that sizes launches and workspaces and the
 *              row stride of per-row outputs (score, range).
 * Per-sequence inputs and outputs (queries, new rows, out, lse, score,
 * range, kept) are indexed by b, the sequence's position in the call.  An
 * empty sequence reads and writes no cache row; its attention output is zero
 * with lse = -inf.  Both arrays are read on the device, in stream order.
 */
typedef struct kvc_cache {
    void* k;
    void* v;
    int32_t dtype;
    int32_t n_slots;
    int32_t nb;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t t_len;
    int32_t t_cap;
    int32_t nb_cap;              /* batch entries of k / v; 0 means nb     */
    const int32_t* batch_idx;    /* device [nb] or NULL                    */
    const int32_t* seq_len;      /* device [nb] or NULL                    */
    int32_t v_layout;            /* kvc_v_layout; 0 = KVC_V_TILES          */
} kvc_cache;

typedef enum kvc_v_layout {
    KVC_V_TILES = 0,      /* [t_cap/32][head_dim][32] tiles (decode layout) */
    KVC_V_ROWS = 1        /* [t_cap][head_dim] rows, like k (prefill)       */
} kvc_v_layout;

/*
 * A range-protected int8 cache [VASE §3, §5: large-range value states
 * dominate per-token quantization error, so they keep full precision].
 * Per slot, per (batch entry b, KV head j):
 *   kq: uint8 [t_cap][head_dim]      key codes + 128 (code = round-half-even
 *                                     of x / scale, clamped to +-127)
 *   vq: uint8 [t_cap/32][head_dim][32] value codes + 128, 32-token tiles
 *   sk: float32 [t_cap]               key row scale max|k| / 127; a negative
 *                                     scale marks a protected row (its codes
 *                                     are ignored)
 *   sv: float32 [t_cap]               value row scale max|v| / 127
 *   kp: bf16 [p_cap][head_dim]        keys of the p_len protected rows
 *   vp: bf16 [p_cap/32][head_dim][32] values of the protected rows
 * Slots follow each other in every array; t_cap and p_cap are multiples of
 * 64, p_len <= t_len, every pointer is 16-byte aligned.  A quantized row
 * reconstructs as code * scale; attention sees every row once (protected
 * rows through kp / vp only).
 */
typedef struct kvc_qcache {
    void* kq;
    void* vq;
    float* sk;
    float* sv;
    void* kp;
    void* vp;
    int32_t n_slots;
    int32_t nb;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t t_len;
    int32_t t_cap;
    int32_t p_len;
    int32_t p_cap;
} kvc_qcache;

/* Library version as major*10000 + minor*100 + patch. */
int kvc_version(void);

/* Static description of a status code (never NULL). */
const char* kvc_strerror(int status);

/*
 * Sharing map [RCLA, inference paragraph].  Host only, synchronous.
 *   leaders[n_leaders]: the sorted set S; must start at layer 0, be strictly
 *   increasing and lie in [0, n_layers).
 *   src_layer[n_layers] (out): max{s in S : s <= l}.
 *   src_slot[n_layers]  (out): index of src_layer[l] in S (the cache slot).
 * KVC_EINVAL for a bad set, KVC_EALIGN for a NULL pointer.
 */
int kvc_share_map(int n_layers, const int32_t* leaders, int n_leaders,
                  int32_t* src_layer, int32_t* src_slot);

/*
 * Leader append [RCLA, implementation paragraph]: write one new row per
 * (b, kv head) at row t_len - 1 of `slot` (ragged: row seq_len[b] - 1; the
 * caller has already counted the row).  k_new, v_new: device
 * [nb][n_kv_heads][head_dim], same dtype as the cache.  Followers never
 * call this.
 */
int kvc_append(const kvc_cache* c, int slot, const void* k_new,
               const void* v_new, kvc_stream_t stream);

/* Workspace bytes kvc_decode_attn needs for caches of this shape, for any
 * t_len <= c->t_cap and any n_q_layers up to the given count: a head of
 * KVC_ATTN_COUNTERS 32-bit arrival counters, then the split partials. */
#define KVC_ATTN_COUNTERS 16384
int kvc_decode_attn_ws_bytes(const kvc_cache* c, int n_q_layers,
                             int n_q_heads, size_t* bytes);

/*
 * Grouped-query decode attention over leader KV [RCLA; standard softmax].
 * For q-layer i, batch b, query head h, with g = n_q_heads / n_kv_heads and
 * kv head j = h / g (contiguous groups):
 *     out[i][b][h] = softmax_t(scale * q[i][b][h] . K[s][b][j][t]) V[s][b][j][t]
 *     lse[i][b][h] = log sum_t exp(scale * q[i][b][h] . K[s][b][j][t])
 * over t in [0, c->t_len) (ragged: [0, seq_len[b])), where s = q_slot[i]
 * (a host array; normally the src_slot of the layer).  Several q-layers
 * that read one slot are served by one pass over that slot's KV (all
 * followers of a leader in one call), or the caller makes one call per
 * layer.
 *   q:   device [n_q_layers][nb][n_q_heads][head_dim], cache dtype; q-layer
 *        i starts q_layer_stride elements after q-layer i-1 (0 = packed).
 *   scale: 0 means 1/sqrt(head_dim).
 *   append_slot >= 0: row t_len-1 (ragged: seq_len[b]-1) of that slot is
 *        taken from k_new/v_new
 *        (device [nb][n_kv_heads][head_dim]) and also written into the
 *        cache, as kvc_append does; -1: no append, k_new/v_new ignored.
 *   out: device float32 [n_q_layers][nb][n_q_heads][head_dim], layer stride
 *        out_layer_stride (0 = packed).
 *   lse: device float32 [n_q_layers][nb][n_q_heads] or NULL, layer stride
 *        lse_layer_stride (0 = packed).
 *   ws:  device workspace of at least kvc_decode_attn_ws_bytes bytes: a head
 *        of KVC_ATTN_COUNTERS arrival counters, which must be zero before
 *        the first call that uses the workspace (allocate it zeroed) and
 *        which every completed call leaves zero, so that one workspace may
 *        serve calls of any shape; then the split partials (no
 *        initialisation needed).  Calls that share a workspace must be
 *        ordered (one stream).  A launch whose slabs have several splits
 *        has its partials merged by the last workgroup of each slab to
 *        finish, counted in the head, or by a second kernel when a slab has
 *        many splits per query row.
 * Requires t_len >= 1, n_q_heads a multiple of n_kv_heads, head_dim 128.
 */
int kvc_decode_attn(const kvc_cache* c, const void* q, int64_t q_layer_stride,
                    int n_q_layers, const int32_t* q_slot, int n_q_heads,
                    float scale, const void* k_new, const void* v_new,
                    int append_slot, float* out, int64_t out_layer_stride,
                    float* lse, int64_t lse_layer_stride, void* ws,
                    size_t ws_bytes, kvc_stream_t stream);

/*
 * kvc_decode_attn for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, results and kernels as kvc_decode_attn,
 * without ws / ws_bytes: the split partials go to a device array the library
 * owns, KVC_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, which each GPU the
 * library runs on holds until the process ends.  The caller still passes
 * and owns the inputs and outputs.  The call allocates nothing (no
 * hipMalloc, no allocating library routine); its first call on a device
 * looks up that device's copy of the array (hipGetSymbolAddress), with the
 * device current.
 *   - KVC_ESCRATCH when the call needs more than KVC_NOALLOC_SCRATCH_BYTES
 *     (the kvc_decode_attn_ws_bytes of the same arguments); nothing is
 *     enqueued.  Every call on at most 256 (batch entry, kv head) slabs fits,
 *     and so does every call with at most 16 query rows per slab (q-layers
 *     x g) on at most 2048 slabs.
 *   - The stream must belong to the current device (KVC_EHIP otherwise).
 *   - Every call on one GPU shares that GPU's array and leaves its partials
 *     there; calls that overlap on one GPU (different streams, or different
 *     host threads without ordering) race and may return wrong results.
 *     Calls ordered on one stream are safe.  The array's counter head is
 *     zero when the library is loaded (static storage) and every completed
 *     call leaves it zero; the partials need no clearing: every launch
 *     writes what it reads.
 */
#define KVC_NOALLOC_SCRATCH_BYTES (32u << 20)
int kvc_decode_attn_noalloc(const kvc_cache* c, const void* q,
                            int64_t q_layer_stride, int n_q_layers,
                            const int32_t* q_slot, int n_q_heads, float scale,
                            const void* k_new, const void* v_new,
                            int append_slot, float* out,
                            int64_t out_layer_stride, float* lse,
                            int64_t lse_layer_stride, kvc_stream_t stream);

/*
 * Value range [VASE §2.A]: range[b][j][t] = max_c V[slot][b][j][t][c]
 *                                         - min_c V[slot][b][j][t][c]
 * over the head_dim channels of each value row, t in [0, t_len) (ragged:
 * [0, seq_len[b]); rows past it are not written), computed in float32
 * (exact rounding of the true difference).
 *   range: device float32 [nb][n_kv_heads][t_len].
 */
int kvc_value_range(const kvc_cache* c, int slot, float* range,
                    kvc_stream_t stream);

/* Workspace bytes kvc_score needs without lse_obs (two passes). */
int kvc_score_ws_bytes(const kvc_cache* c, int n_q_heads, int w,
                       size_t* bytes);

/*
 * Observation-window score [VASE §2.B, SnapKV-derived], one pass over the
 * slot's KV.  For slab (b, j) the rows are (h in the group of j, i < w) with
 * queries q_obs[i][b][h]; window row i sees cache rows t <= t_len - w + i
 * (it was issued when the cache held t_len - w + i + 1 rows).  Ragged:
 * t <= seq_len[b] - w + i, and a window row that sees no row adds nothing
 * (its lse_obs entry is ignored); rows past seq_len[b] are
 * not written.
 *     score[b][j][t] = sum_{h,i} softmax_t(scale * q_obs[i][b][h] . K[t])
 *   q_obs:   device [w][nb][n_q_heads][head_dim], cache dtype, oldest first.
 *   lse_obs: device float32 [w][nb][n_q_heads] holding the log-normaliser of
 *            each window row over its visible rows (as kvc_decode_attn
 *            returned it when the query was decoded, valid when no
 *            compaction happened inside the window), or NULL: then a first
 *            pass computes it and ws (kvc_score_ws_bytes bytes, no
 *            initialisation needed) is required.
 *   score:   device float32 [nb][n_kv_heads][t_len].
 *   range:   NULL or device float32 [nb][n_kv_heads][t_len]: the value range
 *            of kvc_value_range, fused into the same pass over the cache.
 * Requires 1 <= w <= t_len and g*w <= 512.
 */
int kvc_score(const kvc_cache* c, int slot, const void* q_obs, int n_q_heads,
              int w, float scale, const float* lse_obs, float* score,
              float* range, void* ws, size_t ws_bytes, kvc_stream_t stream);

/*
 * Observation-window score [VASE §2.B] for a pass over some of a batch's
 * sequences [VASE §2: each sequence evicts on its own period, so a pass
 * covers the sequences due after a step] whose window queries sit in the
 * whole batch's arrays:
 * call sequence b reads q_obs[i][q_idx[b]][h] and lse_obs[i][q_idx[b]][h].
 *   q_obs:   device [w][q_nb][n_q_heads][head_dim]; lse_obs [w][q_nb][n_q_heads]
 *            or NULL.
 *   q_idx:   device int32 [c->nb], entries in [0, q_nb) (read on the
 *            device, not checked), or NULL: sequence b reads row b (then
 *            q_nb >= c->nb).
 * Everything else is kvc_score's (which is this call with q_nb = c->nb and
 * q_idx = NULL).
 */
int kvc_score_seq(const kvc_cache* c, int slot, const void* q_obs, int q_nb,
                  const int32_t* q_idx, int n_q_heads, int w, float scale,
                  const float* lse_obs, float* score, float* range, void* ws,
                  size_t ws_bytes, kvc_stream_t stream);

/* Workspace bytes kvc_select needs for nb * n_kv_heads slabs of t_len rows
 * (two uint32 per row: the sampling key of every candidate row, and the
 * selection keys of slabs too long for LDS). */
int kvc_select_ws_bytes(int nb, int n_kv_heads, int t_len, size_t* bytes);

/*
 * kvc_select for ragged batches: slab (b, j) has T_b = seq_len[b] rows
 * (clamped to [0, t_len]; NULL: t_len each) and keeps min(T_b, K + B) of
 * them; kept keeps the stride n_keep = min(t_len, K + B) and its entries
 * past min(T_b, K + B) are -1.  The Philox counter's batch word is
 * seq_id[b] (NULL: b), so that a sequence draws the same keys whatever its
 * position in the call.  score / range rows keep the stride t_len.
 */
int kvc_select_seq(const float* score, const float* range, int nb, int n_kv_heads,
                   int t_len, const int32_t* seq_len, const int32_t* seq_id,
                   int budget_k, int recent_b, int n_v, uint64_t seed, int layer_id,
                   int32_t* kept, void* ws, size_t ws_bytes, kvc_stream_t stream);

/*
 * VASE selection [VASE §2, §2.A, §2.B], per slab (b, j):
 *   if t_len <= K + B every row is kept; otherwise
 *   1. the last B rows [t_len - B, t_len) are kept;
 *   2. among candidate rows [0, t_len - B) the N_v of largest range are
 *      kept (ties to the lower row);
 *   3. K - N_v more candidates are sampled without replacement with
 *      probability proportional to score: row t gets the key
 *      kappa_t = E_t / score_t (infinite when score_t <= 0), where
 *      E_t = -ln((x_t + 1) / 2^32) and x_t is word 0 of Philox4x32-10 at
 *      counter (t, j, layer_id, b) and key (seed mod 2^32, seed >> 32); the
 *      K - N_v smallest keys are kept (ties to the lower row).
 *   score, range: device float32 [nb][n_kv_heads][t_len].
 *   kept (out):   device int32 [nb][n_kv_heads][n_keep], ascending, with
 *                 n_keep = min(t_len, K + B).
 *   ws: device workspace of kvc_select_ws_bytes bytes (no zeroing needed).
 * Requires 0 <= N_v <= K, B >= 0, K + B >= 1.  The result is a pure
 * function of its inputs; a driver that evicts repeatedly passes a new seed
 * each pass.
 */
int kvc_select(const float* score, const float* range, int nb, int n_kv_heads,
               int t_len, int budget_k, int recent_b, int n_v, uint64_t seed,
               int layer_id, int32_t* kept, void* ws, size_t ws_bytes,
               kvc_stream_t stream);

/*
 * Compaction [VASE §1: evicted pairs are dropped for good].  For every slab
 * of `slot`: dst row i <- src row kept[b][j][i], i < n_keep, for K and V,
 * written into the same slot of dst.  Out of place: the slot's K and V
 * regions of src and dst must not overlap (KVC_EALIAS).  dst must have the
 * same dtype, nb, n_kv_heads and head_dim, and dst->t_cap >= n_keep; the
 * caller sets dst->t_len = n_keep afterwards.  kept: device int32
 * [nb][n_kv_heads][n_keep] with entries in [0, src->t_len); a row whose
 * index is out of that range is written as zeros.
 * Ragged batches: sequence b is read from its src entry and written to its
 * dst entry (each side's batch_idx) and keeps min(T_b, n_keep) rows, T_b its
 * src length; the caller then sets its dst length to that.  With a batch
 * map on either side, src and dst may be one cache: the caller keeps every
 * sequence's src and dst entries apart (not checked, the maps are device
 * data); a shared entry gives unspecified rows, never an access outside the
 * buffers.
 * kept may be NULL: dst row i <- src row i for i < n_keep (ragged: i <
 * min(T_b, n_keep)), a bulk copy.
 * Layouts: dst must be KVC_V_TILES; src may be either.  From a KVC_V_ROWS
 * src the gather reads exactly the kept value rows and writes them as
 * tiles, so a prefill's [t][head_dim] cache enters the decode layout in the
 * prompt compression itself (or, with kept = NULL, in one copy).
 */
int kvc_compact(const kvc_cache* src, int slot, const int32_t* kept,
                int n_keep, const kvc_cache* dst, kvc_stream_t stream);

/* Workspace bytes kvc_dkv_score needs for any t_len <= max(t_len, t_cap). */
int kvc_dkv_ws_bytes(const kvc_cache* c, int rank, size_t* bytes);

/*
 * VASE-DKV token scores [VASE §2.B: CurDKV's leverage scores, with a
 * Gaussian projection G drawn afresh at every eviction pass].  The page gives
 * no formula; this library scores token t of slab (b, j) by the leverage of
 * row t of the sketch Y = [K | V] G (key row then value row, T x 2d, times
 * G of shape 2d x rank):
 *   score_t = y_t (Y^T Y)^+ y_t^T,
 * the squared norm of row t of an orthonormal basis of Y's column space
 * (sum over t = rank(Y)).  The pseudo-inverse is taken through a Cholesky
 * factorisation of Y^T Y in float64 that drops every direction whose pivot
 * is at most 1e-12 of the trace.  Y is accumulated in float32 from the bf16
 * cache and G, Y^T Y in float64.  The scores are sampling weights for
 * kvc_select, which runs
 * unchanged (value-range protection, recent buffer, exponential keys).
 *   g:     device bf16 [rank][2 * head_dim]; row n is sketch column n
 *          (entries 0..d-1 multiply the key channels, d..2d-1 the value
 *          channels).  Draw it per pass, e.g. with kvc_gaussian_bf16.
 *   rank:  16 or 32.
 *   score: device float32 [nb][n_kv_heads][t_len].
 *   range: NULL or device float32 [nb][n_kv_heads][t_len]: the value range
 *          of kvc_value_range, fused into the same pass over the cache.
 *   ws:    kvc_dkv_ws_bytes bytes, 16-byte aligned, no initialisation needed.
 * bf16 caches only (KVC_EDTYPE otherwise).
 */
int kvc_dkv_score(const kvc_cache* c, int slot, const void* g, int rank,
                  float* score, float* range, void* ws, size_t ws_bytes,
                  kvc_stream_t stream);

/*
 * N(0, 1) draws rounded to bf16, for the Gaussian projection of
 * kvc_dkv_score: Box-Muller (1958) on Philox4x32-10.  Elements 2p and 2p+1
 * come from words x0, x1 at counter (p, c1, c2, 0) under key
 * (seed mod 2^32, seed >> 32):
 *   u1 = (x0 + 1) / 2^32,  u2 = x1 / 2^32,
 *   out[2p] = sqrt(-2 ln u1) cos(2 pi u2), out[2p+1] = ... sin(2 pi u2),
 * evaluated in float64, rounded to float32, then to bf16 (nearest even).
 *   out: device bf16 [n], 4-byte aligned; n <= 2^32.
 */
int kvc_gaussian_bf16(int64_t n, uint64_t seed, uint32_t c1, uint32_t c2,
                      void* out, kvc_stream_t stream);

/*
 * Range-protected quantization of one bf16 slot into the same slot of an
 * int8 cache [VASE §3, §5].  protect: device int32 [nb][n_kv_heads]
 * [n_protect], each list ascending with entries in [0, src->t_len) -- the
 * rows that keep bf16 (typically the n_protect largest value ranges:
 * kvc_value_range, then kvc_select with K = N_v = n_protect, B = 0).  Every
 * other row's key and value are quantized per row.  The caller sets
 * dst->t_len = src->t_len and dst->p_len = n_protect before the call;
 * n_protect <= dst->p_cap.  src must be bf16 (KVC_EDTYPE), with the same nb
 * and n_kv_heads as dst, and a uniform batch (no batch_idx / seq_len,
 * nb_cap 0 or nb; KVC_EINVAL otherwise).
 */
int kvc_q8_quantize(const kvc_cache* src, int slot, const int32_t* protect,
                    int n_protect, const kvc_qcache* dst, kvc_stream_t stream);

/*
 * Leader append into an int8 cache [R-CLA implementation paragraph]: row
 * t_len - 1 of every slab of `slot` becomes the per-row quantization of
 * k_new, v_new (device bf16 [nb][n_kv_heads][head_dim]); appended rows are
 * not protected.  The caller has already bumped t_len.
 */
int kvc_q8_append(const kvc_qcache* c, int slot, const void* k_new,
                  const void* v_new, kvc_stream_t stream);

/* Workspace bytes kvc_q8_decode_attn needs (any t_len <= t_cap): the same
 * head of KVC_ATTN_COUNTERS arrival counters as kvc_decode_attn's (zero
 * before the first call, left zero by every call), then the partials. */
int kvc_q8_decode_attn_ws_bytes(const kvc_qcache* c, int n_q_layers,
                                int n_q_heads, size_t* bytes);

/*
 * Decode attention over an int8 range-protected cache: exactly
 * kvc_decode_attn's contract (same q / out / lse layouts and strides, GQA,
 * q-layer grouping; no fused append -- use kvc_q8_append first), with each
 * row's key and value taken as code * scale, or as the bf16 protected row.
 * q: bf16.  Requires g = n_q_heads / n_kv_heads <= 64.  ws: as for
 * kvc_decode_attn (allocated zeroed; one workspace may serve both calls).
 */
int kvc_q8_decode_attn(const kvc_qcache* c, const void* q,
                       int64_t q_layer_stride, int n_q_layers,
                       const int32_t* q_slot, int n_q_heads, float scale,
                       float* out, int64_t out_layer_stride, float* lse,
                       int64_t lse_layer_stride, void* ws, size_t ws_bytes,
                       kvc_stream_t stream);

/*
 * Cross-layer factorisation store for one window of W consecutive layers
 * [XKV §2.2: the window's caches concatenated side by side, a rank-r SVD,
 * one token basis A shared by the window and one matrix B_l per layer].
 * Per (batch entry b, KV head j), keys and values separately:
 *   ak:     bf16 [nb][n_kv_heads][t_cap][rank]      key token basis A_K
 *   av:     bf16 [nb][n_kv_heads][t_cap/chunk][rank][chunk]  value token
 *           basis A_V, chunk-transposed: A_V[t][c] at [t/chunk][c][t%chunk]
 *           (the chunk's rows side by side for each rank, the operand
 *           layout of the rank-space value product)
 *   bk, bv: float32 [nb][n_kv_heads][window*head_dim][rank]: rows
 *           l*head_dim .. l*head_dim + head_dim - 1 hold B_l^T, so layer l's
 *           row t is rebuilt as A[t] B_l
 *   lk:     bf16 [nb][n_kv_heads][t_cap/chunk][rank]  key landmarks: the
 *           mean of each chunk's rows of the key basis [XKV §2.3]
 * window 1..4, rank 32 or 64 (<= window*head_dim), chunk 8, t_cap a
 * multiple of 64, rows [0, t_len) valid, every pointer 16-byte aligned.
 * Memory: t_cap*rank + window*head_dim*rank numbers per basis instead of
 * window*t_cap*head_dim.
 */
typedef struct kvc_xkv {
    void* ak;
    void* av;
    void* lk;
    float* bk;
    float* bv;
    int32_t nb;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t window;
    int32_t rank;
    int32_t chunk;
    int32_t t_len;
    int32_t t_cap;
} kvc_xkv;

/* Workspace bytes kvc_xkv_factor needs for stores of this shape. */
int kvc_xkv_factor_ws_bytes(const kvc_xkv* x, size_t* bytes);

/*
 * Cross-layer factorisation [XKV §2.2] of slots [slot0, slot0 + window) of
 * a bf16 cache (uniform batch: no batch_idx / seq_len, nb_cap 0 or nb) into
 * x, for keys and values.  The rank-r truncated SVD of X = [X_1 | ... | X_W]
 * (T x window*head_dim, T = c->t_len = x->t_len) is computed by `iters`
 * steps of subspace iteration on X^T X (float32) from a Gaussian start drawn
 * with `seed`, modified Gram-Schmidt after every step: the bases' columns
 * are orthonormal and converge to the top-r right singular subspace, so A B_l
 * is the rank-r truncation up to that convergence (exact when X has rank
 * <= r).  A = X V is rounded to bf16; the landmarks are the chunk means of
 * the stored key rows.  iters 1..64.  ws: kvc_xkv_factor_ws_bytes bytes, no
 * initialisation needed.
 */
int kvc_xkv_factor(const kvc_cache* c, int slot0, int iters, uint64_t seed,
                   const kvc_xkv* x, void* ws, size_t ws_bytes, kvc_stream_t stream);

/*
 * Selective-reconstruction decode attention [XKV §2.3] for layer `layer`
 * (0..window-1) of the window x stores.  For batch entry b and KV head j with
 * query heads h of its group (g = n_q_heads / n_kv_heads <= 8):
 *   chunk score s_c = max_h q_h . (lk[c] B_layer)       (landmark key)
 *   kept chunks    = the n_select largest s_c (ties to the lower chunk; all
 *                    chunks when there are fewer), ascending
 *   out[b][h]      = softmax(scale * q_h . K^_t) V^_t over the rows t of the
 *                    kept chunks, K^_t = ak[t] B^K_layer, V^_t = av[t] B^V_layer
 * computed in the rank space (the rebuilt rows are never stored).  With o_in
 * and lse_in (float32 [nb][n_q_heads][head_dim] and [nb][n_q_heads], e.g.
 * kvc_decode_attn over the rows appended after the factorisation) the two
 * parts merge into attention over their union; lse (optional) is the
 * union's log-normaliser.  q: bf16 [nb][n_q_heads][head_dim]; out: float32
 * like o_in; selected: NULL or int32 [nb][n_kv_heads][n_select] (-1 past the
 * kept count).  n_select >= 1 (KVC_EINVAL otherwise).  Two launches of
 * one to eight workgroups per (b, j): the chunk scores, then the top-k and
 * the kept rows, whose partials the last workgroup of each (b, j) merges.
 * ws: kvc_xkv_decode_ws_bytes bytes for the same store shape, head count and
 * n_select (16-byte aligned; KVC_EWORKSPACE if NULL or smaller).  It starts
 * with one arrival counter per (b, j), then holds the chunk keys, q~ and the
 * partials: the counters must be zero before the first call that uses the
 * workspace (allocate it zeroed) and every completed call leaves them zero,
 * so one workspace may serve stores of several shapes.  Calls that share a
 * workspace must be ordered (one stream).
 */
int kvc_xkv_decode_attn(const kvc_xkv* x, int layer, const void* q, int n_q_heads, float scale,
                        int n_select, const float* o_in, const float* lse_in, float* out,
                        float* lse, int32_t* selected, void* ws, size_t ws_bytes,
                        kvc_stream_t stream);

/* Workspace bytes kvc_xkv_decode_attn needs for this store shape, query head
 * count and n_select (same argument checks as the call). */
int kvc_xkv_decode_ws_bytes(const kvc_xkv* x, int n_q_heads, int n_select, size_t* bytes);

/*
 * Diagnostic: the device Philox4x32-10 stream that kvc_select draws from.
 * out[i][0..3] = Philox4x32-10(counter (i, c1, c2, c3),
 *                              key (seed mod 2^32, seed >> 32)), i < n.
 *   out: device uint32 [n][4].
 */
int kvc_philox_words(int64_t n, uint32_t c1, uint32_t c2, uint32_t c3,
                     uint64_t seed, uint32_t* out, kvc_stream_t stream);

/*
 * Diagnostic: the read rate this device sustains for a pure stream, the
 * ceiling for the decode kernels (HBM-bound: every cache byte is read once).
 * Streams buf once with the 16-byte non-temporal loads those kernels use;
 * out[i] (i < KVC_PROBE_BLOCKS) is the XOR of the 32-bit words that
 * workgroup i read, so the XOR of all of out is the XOR of every word of
 * buf.  buf: device, 16-byte aligned, bytes a multiple of 16 (KVC_EALIGN /
 * KVC_EINVAL otherwise; bytes 0 writes zeros); out: device uint32
 * [KVC_PROBE_BLOCKS], 4-byte aligned.  Stream-ordered.
 */
#define KVC_PROBE_BLOCKS 256
int kvc_read_probe(const void* buf, size_t bytes, uint32_t* out, kvc_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
