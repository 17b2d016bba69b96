// Internal launch descriptors shared by the host dispatcher (abi.cpp) and the
// kernels.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvc {

constexpr int MAX_QL = 64;       // q-layers served by one attention launch
constexpr int ATTN_TILE = 32;    // cache rows per attention step (bf16 path)
constexpr int ATTN_TILE_F32 = 64;
constexpr int ATTN_WAVES = 4;    // waves per attention workgroup
constexpr int ATTN_TARGET_WGS = 256;  // partial workgroups an attention launch aims for
constexpr int MAX_SPLIT_ROWS = 4096;  // bound on nsplit * padded rows (workspace size)
constexpr int SCORE_TILE = 32;
constexpr int SCORE_MAX_TPS = 64;     // tiles per score-statistics workgroup
constexpr int SCORE_QPITCH = 136;     // bf16 per window-query row staged in LDS (272 bytes)
constexpr int CU_COUNT = 256;         // compute units of the part
constexpr int XCD_COUNT = 8;          // accelerator dies; workgroups are dealt to them in turn
constexpr int LDS_PER_CU = 160 * 1024;

// LDS of one bf16 score-pass workgroup: the window queries (16-row blocks)
// plus one float (lse term) and one int (last visible row) per row.
// bf16 windows of up to 256 rows run the statistics pass on the score
// pass's grid and tiling (its splits then size the statistics workspace).
inline bool score_stats_tiled(int rows) { return rows <= 256; }
inline size_t score_main_lds_bytes(int rows) {
    return (size_t)((rows + 15) / 16) * 16 * (SCORE_QPITCH * 2 + 8);
}
constexpr int SELECT_THREADS = 1024;

// Workgroups are dealt to the XCDs in turn (linear id modulo XCD_COUNT).
// With `runs`, the block coordinates are renumbered so that each XCD takes a
// contiguous run of linear blocks (x fastest) when the grid divides evenly:
// neighbouring blocks that read the same data then share one XCD's L2.
struct BlockXYZ {
    int x, y, z;
};
__device__ __forceinline__ BlockXYZ xcd_run_block(bool runs) {
    const int gx = gridDim.x, gy = gridDim.y;
    const int nwg = gx * gy * gridDim.z;
    int blk = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    if (runs && nwg % XCD_COUNT == 0) blk = (blk % XCD_COUNT) * (nwg / XCD_COUNT) + blk / XCD_COUNT;
    return BlockXYZ{blk % gx, (blk / gx) % gy, blk / (gx * gy)};
}

// Ragged batches.  A launch addresses nb sequences; sequence b is stored in
// batch entry phys(b) of buffers that hold nb_cap entries and has rows(b)
// rows.  Per-sequence inputs and outputs are indexed by b.  Both arrays live
// on the device and are not trusted: an entry index outside [0, nb_cap)
// makes the sequence empty and lengths are clamped to [0, t_len].
struct SeqMap {
    const int32_t* idx;     // [nb] batch entry per sequence, or null (entry b)
    const int32_t* len;     // [nb] rows per sequence, or null (t_len each)
    int nb_cap;             // batch entries of the buffers
    int t_len;              // bound on every length
};
__device__ __forceinline__ int seq_phys(const SeqMap& m, int b) {
    if (!m.idx) return b;
    const int c = m.idx[b];
    return (c >= 0 && c < m.nb_cap) ? c : -1;
}
__device__ __forceinline__ int seq_rows(const SeqMap& m, int b, int phys) {
    if (phys < 0) return 0;
    if (!m.len) return m.t_len;
    return min(max(m.len[b], 0), m.t_len);
}

// Batch row of q_obs / lse_obs that sequence b of a score launch reads.
__device__ __forceinline__ int score_qrow(const int32_t* q_idx, int b) {
    return q_idx ? q_idx[b] : b;
}

// One attention launch: a set of q-layers that all read one cache slot.
struct AttnLaunch {
    const void* k;          // slot base of K: [nb][hkv][t_cap][D]
    const void* v;          // slot base of V: [nb][hkv][D][t_cap]
    int nb, hkv, g, hq;
    int t_len, t_cap;
    int nql, rows;          // q-layers in this launch, rows = nql * g
    int rp;                 // padded rows per slab in the workspace
    const void* q;
    int64_t q_off[MAX_QL];  // element offset of q-layer i
    float* out;
    int64_t out_off[MAX_QL];
    float* lse;             // may be null
    int64_t lse_off[MAX_QL];
    float scale;
    const void* k_new;      // [nb][hkv][D], read when append_read
    const void* v_new;
    int append_read;        // row t_len-1 comes from k_new / v_new
    int append_write;       // and is written into the cache
    int nsplit, tps;        // splits per slab, tiles per split
    int xcd_runs;           // workgroups renumbered into contiguous runs per XCD
    float* part;            // partial accumulators, then (m, l) pairs
    unsigned* arrive;       // per-slab arrival counters (zero between launches), or null:
                            // then a separate kernel merges the partials
    SeqMap sm;              // cache entry and rows of each sequence
};

// One observation-window score launch over one cache slot.
struct ScoreLaunch {
    const void* k;          // slot base of K
    const void* v;          // slot base of V (for the fused range)
    int nb, hkv, g, hq, w;
    int t_len, t_cap;
    int rows;               // g * w
    const void* q_obs;      // [w][q_nb][hq][D]
    const float* lse_obs;   // [w][q_nb][hq] or null (then `lse_ws` is used)
    const int32_t* q_idx;   // [nb]: q_obs / lse_obs batch row of each sequence, or null (b)
    int q_nb;               // batch rows of q_obs / lse_obs
    float scale;
    float* score;           // [nb][hkv][t_len]
    float* range;           // [nb][hkv][t_len] or null
    int nsplit, tps;        // statistics pass (and the float32 path): splits, tiles per split
    int main_nsplit, main_tps;   // bf16 score pass
    float* stats;           // [slabs][nsplit][rows_pad][2] partial (m, z)
    float* lse_ws;          // [slabs][rows_pad] merged log-normalisers
    int rows_pad;
    SeqMap sm;
};

// Decode attention over a range-protected int8 slot.  `a` carries the
// attention fields (a.k / a.v are the code slot bases, a.t_len / a.t_cap the
// quantized rows); the protected rows are a bf16 mini-slab per (b, j).
struct Q8AttnLaunch {
    AttnLaunch a;
    const float* sk;        // [nb][hkv][t_cap] key scales; < 0: the row is protected
    const float* sv;        // [nb][hkv][t_cap] value scales
    const void* kp;         // bf16 [nb][hkv][p_cap][D]
    const void* vp;         // bf16 [nb][hkv][p_cap/32][D][32]
    int p_len, p_cap;
    int nq_tiles;           // 32-row tiles of quantized rows; protected tiles follow
};

// Quantization of one bf16 slot into a range-protected int8 slot.
struct Q8QuantLaunch {
    const void* k;          // bf16 slot bases of the source
    const void* v;
    int nb, hkv, t_len, src_t_cap;
    const int32_t* protect; // [nb][hkv][n_protect], ascending
    int n_protect;
    void* kq;               // uint8 code slot bases of the destination (code + 128)
    void* vq;
    float* sk;
    float* sv;
    int dst_t_cap;
    int row0, nrows;        // rows [row0, row0 + nrows) are quantized (an append: one row)
    const void* k_row;      // append: bf16 [nb][hkv][D] new rows instead of the source slot
    const void* v_row;
};

// VASE-DKV scores of one cache slot (bf16).
struct DkvLaunch {
    const void* k;          // slot base of K
    const void* v;          // slot base of V
    int nb, hkv, t_len, t_cap;
    const void* g;          // bf16 [rank][2*D]: row n is sketch column n
    int rank;               // 16 or 32
    float* score;           // [nb][hkv][t_len]
    float* range;           // [nb][hkv][t_len] or null
    int nsplit, tps;        // sketch pass: splits per slab, tiles per split
    float* y;               // workspace [slabs][t_len][rank]
    double* gram;           // workspace [slabs][nsplit][rank][rank]
    double* w;              // workspace [slabs][rank][rank]: the inverse factor
    SeqMap sm;
    int v_rows;             // values stored as [t][D] rows (else tiles)
};

struct SelectLaunch {
    const float* score;
    const float* range;
    int nb, hkv, t_len, budget_k, recent_b, n_v;
    uint32_t seed_lo, seed_hi;
    uint32_t layer_id;
    int32_t* kept;
    uint32_t* keys;         // workspace [slabs][t_len]: selection keys of slabs past LDS_KEYS rows
    uint32_t* kappa;        // workspace [slabs][t_len]: sampling keys of the candidate rows
    const int32_t* len;     // [nb] rows per slab's sequence, or null (t_len)
    const int32_t* seq_id;  // [nb] sequence word of the Philox counter, or null (b)
};

struct CompactLaunch {
    const void* sk;
    const void* sv;
    void* dk;
    void* dv;
    int nb, hkv;
    int src_t_cap, dst_t_cap;
    const int32_t* kept;
    int n_keep;             // stride of kept; sequence b keeps min(rows(b), n_keep)
    int elem;               // bytes per element
    SeqMap src_sm, dst_sm;  // src_sm.len gives the source rows
    int src_rows;           // source values stored as [t][D] rows (else tiles)
};

// Cross-layer factorisation of one window of W slots (bf16, uniform batch).
struct XkvLaunch {
    const void* k;          // K of the window's first slot
    const void* v;          // V of the window's first slot
    size_t slot_stride;     // elements from one slot to the next
    int nb, hkv, t_len, t_cap, window, rank;
    float* gram;            // workspace [2][nb][hkv][n][n], n = window * D (keys, then values)
    uint16_t* vt;           // workspace [2][nb][hkv][rank][n]: bf16 transpose of the bases
    void* ak;               // bf16 [nb][hkv][x_tcap][rank]
    void* av;
    void* lk;               // bf16 [nb][hkv][x_tcap / 8][rank]
    float* bk;              // [nb][hkv][n][rank]
    float* bv;
    int x_tcap;
    int iters;
    uint32_t seed_lo, seed_hi;
    int nsplit, tps;        // projection: splits per slab, 32-row tiles per split
};

// Selective-reconstruction decode attention for one layer of a window.
struct XkvDecodeLaunch {
    const void* ak;
    const void* av;
    const void* lk;
    const float* bk;
    const float* bv;
    int nb, hkv, g, hq, t_len, x_tcap, window, rank, layer, n_select;
    const void* q;          // bf16 [nb][hq][D]
    float scale;
    const float* o_in;      // float32 [nb][hq][D] or null: a second part to merge
    const float* lse_in;
    float* out;
    float* lse;             // may be null
    int32_t* selected;      // [nb][hkv][n_select] or null
    int ns;                 // workgroups per (b, j) in each of the two launches
    uint32_t* ws_keys;      // [nb][hkv][nch] chunk score keys
    float* ws_qt;           // [nb][hkv][8][rank] q~ of the first launch
    float* ws_part;         // [nb][hkv][ns][8][rank + 2] the splits' partials
    unsigned* ws_arrive;    // [nb][hkv] arrival counters, zero between launches
};

// Host-side launchers (defined next to their kernels).  Each returns
// hipSuccess or the launch error.
// Launches the partial kernel and the merge kernel.
hipError_t launch_attn(const AttnLaunch& p, int dtype, int nt, hipStream_t s);
// Device address of the current device's no-allocation scratch array
// (KVC_NOALLOC_SCRATCH_BYTES); `stream` (may be NULL) must be on that device.
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);
hipError_t launch_attn_combine(const AttnLaunch& p, hipStream_t s);
// Read-bandwidth probe: PROBE_BLOCKS workgroups stream `bytes` (a multiple of
// 16) and write one XOR checksum word each to out[PROBE_BLOCKS].
constexpr int PROBE_BLOCKS = 256;
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t s);
hipError_t launch_attn_q8(const Q8AttnLaunch& p, int nt, hipStream_t s);
hipError_t launch_q8_quantize(const Q8QuantLaunch& p, hipStream_t s);
hipError_t launch_append(const void* k, const void* v, int nb, int hkv, int t_cap,
                         const SeqMap& sm, const void* k_new, const void* v_new, int elem,
                         hipStream_t s);
hipError_t launch_value_range(const void* v, bool v_rows, int nb, int hkv, int t_cap, const SeqMap& sm,
                              int dtype, float* range, hipStream_t s);
hipError_t launch_score(const ScoreLaunch& p, int dtype, hipStream_t s);
hipError_t launch_select(const SelectLaunch& p, hipStream_t s);
hipError_t launch_dkv(const DkvLaunch& p, hipStream_t s);
hipError_t launch_gaussian(int64_t n, uint32_t c1, uint32_t c2, uint32_t k0, uint32_t k1,
                           void* out, hipStream_t s);
hipError_t launch_compact(const CompactLaunch& p, hipStream_t s);
hipError_t launch_xkv_factor(const XkvLaunch& p, hipStream_t s);
// The decode (one workgroup per (b, j)): dynamic LDS bytes for nch chunks
// and ksel kept ones, with the chunk keys in LDS or (gkeys) in ws_keys.
// LDS bytes of the decode's second launch (the first needs xkv_scores_lds).
size_t xkv_scores_lds(int rank);
size_t xkv_rows_lds(int rank, int nch, int ksel, bool gkeys);
hipError_t launch_xkv_decode(const XkvDecodeLaunch& p, bool gkeys, size_t rows_lds, hipStream_t s);
hipError_t launch_philox(int64_t n, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                         uint32_t k1, uint32_t* out, hipStream_t s);

}  // namespace kvc
