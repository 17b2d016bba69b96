// libkvc C ABI: argument validation, launch planning and error mapping.
// Every entry point checks all of its arguments on the host before it
// enqueues anything; on an error it returns a negative kvc_status and
// leaves every output untouched.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/kvc.h"
#include "kvc_internal.h"

using namespace kvc;

namespace {

constexpr int VERSION = 10000;   // 1.0.0

bool aligned16(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
size_t elem_size(int dtype) { return dtype == KVC_F32 ? 4 : 2; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Batch entries the buffers hold (0 means nb).
int nb_cap_of(const kvc_cache* c) { return c->nb_cap ? c->nb_cap : c->nb; }

int check_cache(const kvc_cache* c) {
    if (!c) return KVC_EALIGN;
    if (c->dtype != KVC_F32 && c->dtype != KVC_BF16) return KVC_EDTYPE;
    if (c->head_dim != KVC_HEAD_DIM) return KVC_EINVAL;
    if (c->n_slots < 1 || c->nb < 0 || c->n_kv_heads < 1) return KVC_EINVAL;
    if (c->t_cap < 0 || c->t_len < 0 || c->t_len > c->t_cap) return KVC_EINVAL;
    if (c->t_cap % KVC_T_ALIGN) return KVC_EINVAL;
    if (c->nb_cap < 0) return KVC_EINVAL;
    // without a map, sequence b is entry b
    if (!c->batch_idx && c->nb > nb_cap_of(c)) return KVC_EINVAL;
    if (c->v_layout != KVC_V_TILES && c->v_layout != KVC_V_ROWS) return KVC_EINVAL;
    if (!aligned16(c->k) || !aligned16(c->v)) return KVC_EALIGN;
    if ((c->batch_idx && !aligned4(c->batch_idx)) || (c->seq_len && !aligned4(c->seq_len)))
        return KVC_EALIGN;
    return KVC_OK;
}

bool is_ragged(const kvc_cache* c) { return c->batch_idx || c->seq_len; }

// A cache whose values are [t][D] rows (a prefill's layout): only the prompt
// compression's calls (range, score, compaction source) read it.
bool v_rows(const kvc_cache* c) { return c->v_layout == KVC_V_ROWS; }

// check_cache, then require the tiled value layout.
int check_tiled(const kvc_cache* c) {
    const int st = check_cache(c);
    if (st) return st;
    return v_rows(c) ? KVC_EINVAL : KVC_OK;
}

SeqMap seq_map(const kvc_cache* c) {
    SeqMap m;
    m.idx = c->batch_idx;
    m.len = c->seq_len;
    m.nb_cap = nb_cap_of(c);
    m.t_len = c->t_len;
    return m;
}

size_t slot_elems(const kvc_cache* c) {
    return (size_t)nb_cap_of(c) * c->n_kv_heads * c->t_cap * KVC_HEAD_DIM;
}
const char* slot_k(const kvc_cache* c, int slot) {
    return static_cast<const char*>(c->k) + (size_t)slot * slot_elems(c) * elem_size(c->dtype);
}
const char* slot_v(const kvc_cache* c, int slot) {
    return static_cast<const char*>(c->v) + (size_t)slot * slot_elems(c) * elem_size(c->dtype);
}

int hip_status() { return hipGetLastError() == hipSuccess ? KVC_OK : KVC_EHIP; }

// ---- attention planning ----------------------------------------------------
struct AttnPlan {
    int nt, rp, nsplit, tps;
};

AttnPlan plan_attn(int dtype, int rows, int t_len, int slabs) {
    AttnPlan pl;
    int tile, min_tps;
    if (dtype == KVC_F32) {
        pl.nt = 1;
        pl.rp = 16;
        tile = ATTN_TILE_F32;
        min_tps = 1;
    } else {
        pl.nt = rows <= 16 ? 1 : rows <= 32 ? 2 : 4;
        pl.rp = 16 * pl.nt;
        tile = ATTN_TILE;
        min_tps = ATTN_WAVES;   // at least one tile per wave
    }
    const int ntiles = std::max(1, (t_len + tile - 1) / tile);
    const long long work = (long long)ntiles * std::max(1, slabs);
    int tps = (int)std::max<long long>(min_tps, (work + ATTN_TARGET_WGS - 1) / ATTN_TARGET_WGS);
    int nsplit = (ntiles + tps - 1) / tps;
    const int cap = MAX_SPLIT_ROWS / pl.rp;
    if (nsplit > cap) {
        tps = (ntiles + cap - 1) / cap;
        nsplit = (ntiles + tps - 1) / tps;
    }
    pl.tps = tps;
    pl.nsplit = nsplit;
    return pl;
}

int max_rows_per_chunk(int dtype, int g) {
    const int cap_rows = dtype == KVC_F32 ? 16 : 64;
    const int ql = std::min(MAX_QL, cap_rows / g);
    return ql * g;
}

size_t attn_ws_for(int dtype, int rows, int t_len, int slabs) {
    const AttnPlan pl = plan_attn(dtype, rows, t_len, slabs);
    return (size_t)slabs * pl.nsplit * pl.rp * (KVC_HEAD_DIM + 2) * sizeof(float);
}

size_t attn_ws_total(const kvc_cache* c, int rows) {
    const int slabs = c->nb * c->n_kv_heads;
    size_t part = 0;
    for (int t = 1; t <= std::max(1, c->t_cap); t += (c->dtype == KVC_F32 ? ATTN_TILE_F32 : ATTN_TILE))
        part = std::max(part, attn_ws_for(c->dtype, rows, t, slabs));
    part = std::max(part, attn_ws_for(c->dtype, rows, std::max(1, c->t_cap), slabs));
    return part;
}

// The workspace of kvc_decode_attn starts with a fixed head of arrival
// counters (one per slab of a launch whose last workgroup per slab merges),
// then holds the split partials.  The head's place and size do not depend on
// the cache's shape, so a workspace shared by calls of several shapes keeps
// its counters where every call left them: at zero.
constexpr size_t ATTN_COUNTER_HEAD = (size_t)KVC_ATTN_COUNTERS * sizeof(unsigned);

size_t attn_ws_with_counters(const kvc_cache* c, int rows) {
    return ATTN_COUNTER_HEAD + attn_ws_total(c, rows);
}

// Whether the last workgroup of each slab merges the launch's partials (in
// place of the merge kernel): 256 threads share a slab's (row, 8 channels)
// items, split groups sharing an item, so each thread folds at most eight
// splits; and the launch's slabs have counters in the head.
bool fuse_merge(int rows, int nsplit, int slabs) {
    if (nsplit < 2 || slabs > KVC_ATTN_COUNTERS) return false;
    const int items = rows * (KVC_HEAD_DIM / 8);
    const int sg = std::max(1, std::min(nsplit, 256 / std::max(items, 1)));
    return (nsplit + sg - 1) / sg <= 8;
}

// ---- score planning --------------------------------------------------------
struct ScorePlan {
    int nsplit, tps, rows_pad;
    int main_nsplit, main_tps;
};

ScorePlan plan_score(int dtype, int rows, int t_len, int slabs) {
    ScorePlan pl;
    const int tile = dtype == KVC_F32 ? 64 : SCORE_TILE;
    const int ntiles = std::max(1, (t_len + tile - 1) / tile);
    const long long work = (long long)ntiles * std::max(1, slabs);
    int tps = (int)std::max<long long>(1, (work + 2047) / 2048);
    if (dtype != KVC_F32) tps = std::min(tps, SCORE_MAX_TPS);
    pl.tps = tps;
    pl.nsplit = (ntiles + tps - 1) / tps;
    pl.rows_pad = dtype == KVC_F32 ? rows : (rows + 31) / 32 * 32;
    // bf16 score pass: one round of workgroups, as many per CU as registers
    // (four) and the staged queries' LDS allow, and at least two tiles per
    // wave so that staging the window queries stays a small overhead.
    const long long per_cu = std::max<long long>(
        1, std::min<long long>(4, LDS_PER_CU / (long long)score_main_lds_bytes(rows)));
    const long long target = per_cu * CU_COUNT;
    pl.main_tps = (int)std::max<long long>(8, (work + target - 1) / target);
    pl.main_nsplit = (ntiles + pl.main_tps - 1) / pl.main_tps;
    if (dtype != KVC_F32 && score_stats_tiled(rows)) {
        // the statistics pass runs on the score pass's grid
        pl.tps = pl.main_tps;
        pl.nsplit = pl.main_nsplit;
    }
    return pl;
}

struct ScoreWs {
    size_t lse_off, stats_off, total;
};

ScoreWs score_ws_layout(int dtype, int rows, int t_len, int slabs) {
    const ScorePlan pl = plan_score(dtype, rows, t_len, slabs);
    ScoreWs w;
    w.lse_off = 0;
    w.stats_off = w.lse_off + align_up((size_t)slabs * pl.rows_pad * sizeof(float), 256);
    w.total = w.stats_off + (size_t)slabs * pl.nsplit * pl.rows_pad * 2 * sizeof(float);
    return w;
}

// ---- attention launches ----------------------------------------------------
// Group the q-layers by slot (first-appearance order) and cut each group into
// launches of at most chunk_ql q-layers: fn(slot, q-layer ids, count).
template <typename F>
int for_each_attn_chunk(int n_slots, int n_q_layers, const int32_t* q_slot, int chunk_ql, F&& fn) {
    std::vector<char> done(n_slots, 0);
    for (int i = 0; i < n_q_layers; ++i) {
        const int slot = q_slot[i];
        if (done[slot]) continue;
        done[slot] = 1;
        std::vector<int> members;
        for (int k = i; k < n_q_layers; ++k)
            if (q_slot[k] == slot) members.push_back(k);
        for (size_t m0 = 0; m0 < members.size(); m0 += chunk_ql) {
            const int nql = (int)std::min<size_t>(chunk_ql, members.size() - m0);
            const int st = fn(slot, members.data() + m0, nql);
            if (st) return st;
        }
    }
    return KVC_OK;
}

// The fields every attention launch of one chunk shares.
void fill_attn(AttnLaunch& p, int nb, int hkv, int g, int hq, int t_len, int t_cap,
               const int* members, int nql, int64_t qs, int64_t os, int64_t ls, const void* q,
               float* out, float* lse, float scale) {
    memset(&p, 0, sizeof(p));
    p.nb = nb;
    p.hkv = hkv;
    p.g = g;
    p.hq = hq;
    p.t_len = t_len;
    p.t_cap = t_cap;
    p.nql = nql;
    p.rows = nql * g;
    for (int x = 0; x < nql; ++x) {
        p.q_off[x] = members[x] * qs;
        p.out_off[x] = members[x] * os;
        p.lse_off[x] = members[x] * ls;
    }
    p.q = q;
    p.out = out;
    p.lse = lse;
    p.scale = scale;
}

// ---- int8 range-protected caches --------------------------------------------
int check_qcache(const kvc_qcache* c) {
    if (!c) return KVC_EALIGN;
    if (c->head_dim != KVC_HEAD_DIM) return KVC_EINVAL;
    if (c->n_slots < 1 || c->nb < 0 || c->n_kv_heads < 1) return KVC_EINVAL;
    if (c->t_cap < 0 || c->t_len < 0 || c->t_len > c->t_cap || c->t_cap % KVC_T_ALIGN)
        return KVC_EINVAL;
    if (c->p_cap < 0 || c->p_len < 0 || c->p_len > c->p_cap || c->p_cap % KVC_T_ALIGN)
        return KVC_EINVAL;
    if (c->p_len > c->t_len) return KVC_EINVAL;
    if (!aligned16(c->kq) || !aligned16(c->vq) || !aligned16(c->sk) || !aligned16(c->sv))
        return KVC_EALIGN;
    if (c->p_cap > 0 && (!aligned16(c->kp) || !aligned16(c->vp))) return KVC_EALIGN;
    return KVC_OK;
}
size_t q_slot_rows(const kvc_qcache* c) { return (size_t)c->nb * c->n_kv_heads * c->t_cap; }
size_t p_slot_rows(const kvc_qcache* c) { return (size_t)c->nb * c->n_kv_heads * c->p_cap; }
uint8_t* q_kq(const kvc_qcache* c, int slot) {
    return static_cast<uint8_t*>(c->kq) + (size_t)slot * q_slot_rows(c) * KVC_HEAD_DIM;
}
uint8_t* q_vq(const kvc_qcache* c, int slot) {
    return static_cast<uint8_t*>(c->vq) + (size_t)slot * q_slot_rows(c) * KVC_HEAD_DIM;
}
float* q_sk(const kvc_qcache* c, int slot) { return c->sk + (size_t)slot * q_slot_rows(c); }
float* q_sv(const kvc_qcache* c, int slot) { return c->sv + (size_t)slot * q_slot_rows(c); }
uint16_t* q_kp(const kvc_qcache* c, int slot) {
    return static_cast<uint16_t*>(c->kp) + (size_t)slot * p_slot_rows(c) * KVC_HEAD_DIM;
}
uint16_t* q_vp(const kvc_qcache* c, int slot) {
    return static_cast<uint16_t*>(c->vp) + (size_t)slot * p_slot_rows(c) * KVC_HEAD_DIM;
}

// Quantized and protected tiles are planned together as one tile range.
int q8_virtual_rows(const kvc_qcache* c) {
    const int nq = (c->t_len + ATTN_TILE - 1) / ATTN_TILE;
    const int np = (c->p_len + ATTN_TILE - 1) / ATTN_TILE;
    return (nq + np) * ATTN_TILE;
}

// ---- VASE-DKV planning -----------------------------------------------------
constexpr int DKV_TILE = 32;

struct DkvWs {
    int nsplit, tps;
    size_t y_off, gram_off, w_off, total;
};

DkvWs dkv_layout(int rank, int t_len, int slabs) {
    DkvWs w;
    const int ntiles = std::max(1, (t_len + DKV_TILE - 1) / DKV_TILE);
    const long long work = (long long)ntiles * std::max(1, slabs);
    // one round of workgroups (rank 16: three per CU, bounded by LDS;
    // rank 32: two, bounded by registers), at least two tiles per wave
    const long long target = (rank == 16 ? 3LL : 2LL) * CU_COUNT;
    w.tps = (int)std::max<long long>(8, (work + target - 1) / target);
    w.nsplit = (ntiles + w.tps - 1) / w.tps;
    w.y_off = 0;
    w.gram_off = align_up((size_t)slabs * t_len * rank * sizeof(float), 256);
    w.w_off = w.gram_off + align_up((size_t)slabs * w.nsplit * rank * rank * sizeof(double), 256);
    w.total = w.w_off + (size_t)slabs * rank * rank * sizeof(double);
    return w;
}

// ---- cross-layer factorisation ---------------------------------------------
constexpr int XKV_MAXG = 8;          // query heads per KV head on the decode path
constexpr int XKV_CHUNK = 8;
// dynamic LDS of one decode workgroup (it also holds ~8.4 KB of static LDS,
// the selection histograms)
constexpr size_t XKV_DECODE_LDS_LIMIT = LDS_PER_CU - 12 * 1024;

int check_xkv(const kvc_xkv* x) {
    if (!x) return KVC_EALIGN;
    if (x->head_dim != KVC_HEAD_DIM) return KVC_EINVAL;
    if (x->nb < 0 || x->n_kv_heads < 1) return KVC_EINVAL;
    if (x->window < 1 || x->window > 4) return KVC_EINVAL;
    if (x->rank != 32 && x->rank != 64) return KVC_EINVAL;
    if (x->chunk != XKV_CHUNK) return KVC_EINVAL;
    if (x->t_cap < 0 || x->t_cap % KVC_T_ALIGN || x->t_len < 0 || x->t_len > x->t_cap)
        return KVC_EINVAL;
    if (!aligned16(x->ak) || !aligned16(x->av) || !aligned16(x->lk) || !aligned16(x->bk) ||
        !aligned16(x->bv))
        return KVC_EALIGN;
    return KVC_OK;
}

struct XkvWs {
    size_t gram_off, vt_off, total;
};

XkvWs xkv_ws(const kvc_xkv* x) {
    const size_t n = (size_t)x->window * KVC_HEAD_DIM;
    const size_t probs = 2 * (size_t)x->nb * x->n_kv_heads;
    XkvWs w;
    w.gram_off = 0;
    w.vt_off = align_up(probs * n * n * sizeof(float), 256);
    w.total = w.vt_off + probs * x->rank * n * sizeof(uint16_t);
    return w;
}

// Decode plan: two launches of `ns` workgroups per (b, j) (scores, then
// top-k and the kept rows), enough to give every compute unit a workgroup.
// The workspace holds one arrival counter per (b, j), the chunk keys, q~
// and the splits' partials; the second launch keeps the keys in LDS when
// they fit beside the rest of its work.
constexpr int XKV_MAX_SPLIT = 8;

struct XkvDecodePlan {
    int nch, ksel, ns;
    bool gkeys;
    size_t keys_off, qt_off, part_off, arrive_off, ws_bytes, lds;
};

XkvDecodePlan plan_xkv_decode(const kvc_xkv* x, int n_select) {
    XkvDecodePlan pl;
    const size_t slabs = (size_t)x->nb * x->n_kv_heads;
    pl.nch = (x->t_len + XKV_CHUNK - 1) / XKV_CHUNK;
    pl.ksel = std::min(n_select, pl.nch);
    pl.ns = (int)std::min<size_t>(XKV_MAX_SPLIT, std::max<size_t>(1, (CU_COUNT + slabs - 1) / std::max<size_t>(slabs, 1)));
    pl.lds = xkv_rows_lds(x->rank, pl.nch, pl.ksel, false);
    pl.gkeys = pl.lds > XKV_DECODE_LDS_LIMIT;
    if (pl.gkeys) pl.lds = xkv_rows_lds(x->rank, pl.nch, pl.ksel, true);
    // the counters first: a workspace shared by stores of other shapes keeps
    // them at the same place (every completed call leaves them zero)
    pl.arrive_off = 0;
    pl.keys_off = align_up(slabs * 4, 256);
    pl.qt_off = pl.keys_off + align_up(slabs * pl.nch * 4, 256);
    pl.part_off = pl.qt_off + align_up(slabs * XKV_MAXG * x->rank * 4, 256);
    pl.ws_bytes = pl.part_off + slabs * pl.ns * XKV_MAXG * (x->rank + 2) * 4;
    return pl;
}

}  // namespace

extern "C" {

int kvc_version(void) { return VERSION; }

const char* kvc_strerror(int status) {
    switch (status) {
        case KVC_OK: return "success";
        case KVC_EINVAL: return "invalid argument: a size, index or set is out of range";
        case KVC_EDTYPE: return "unknown or mismatched element type";
        case KVC_EALIGN: return "pointer is NULL or not 16-byte aligned";
        case KVC_EWORKSPACE: return "workspace missing or too small";
        case KVC_EALIAS: return "source and destination memory overlap";
        case KVC_EHIP: return "HIP runtime error at launch";
        case KVC_ESCRATCH:
            return "the call needs more scratch than the no-allocation entry point's "
                   "32 MiB device array holds; use the call with a caller workspace";
        default: return "unknown status";
    }
}

int kvc_share_map(int n_layers, const int32_t* leaders, int n_leaders, int32_t* src_layer,
                  int32_t* src_slot) {
    if (!leaders || !src_layer || !src_slot) return KVC_EALIGN;
    if (n_layers < 1 || n_leaders < 1 || n_leaders > n_layers) return KVC_EINVAL;
    if (leaders[0] != 0) return KVC_EINVAL;
    for (int i = 1; i < n_leaders; ++i)
        if (leaders[i] <= leaders[i - 1]) return KVC_EINVAL;
    if (leaders[n_leaders - 1] >= n_layers) return KVC_EINVAL;
    int slot = 0;
    for (int l = 0; l < n_layers; ++l) {
        while (slot + 1 < n_leaders && leaders[slot + 1] <= l) ++slot;
        src_layer[l] = leaders[slot];
        src_slot[l] = slot;
    }
    return KVC_OK;
}

int kvc_append(const kvc_cache* c, int slot, const void* k_new, const void* v_new,
               kvc_stream_t stream) {
    int st = check_tiled(c);
    if (st) return st;
    if (slot < 0 || slot >= c->n_slots || c->t_len < 1) return KVC_EINVAL;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVC_EALIGN;
    if (c->nb == 0) return KVC_OK;
    if (launch_append(slot_k(c, slot), slot_v(c, slot), c->nb, c->n_kv_heads, c->t_cap,
                      seq_map(c), k_new, v_new, (int)elem_size(c->dtype),
                      (hipStream_t)stream) != hipSuccess)
        return KVC_EHIP;
    return hip_status();
}

int kvc_decode_attn_ws_bytes(const kvc_cache* c, int n_q_layers, int n_q_heads, size_t* bytes) {
    int st = check_tiled(c);
    if (st) return st;
    if (!bytes) return KVC_EALIGN;
    if (n_q_layers < 0 || n_q_heads < 1 || n_q_heads % c->n_kv_heads) return KVC_EINVAL;
    const int g = n_q_heads / c->n_kv_heads;
    if (g > (c->dtype == KVC_F32 ? 16 : 64)) return KVC_EINVAL;
    const int rows = std::min(n_q_layers * g, max_rows_per_chunk(c->dtype, g));
    *bytes = (n_q_layers == 0 || c->nb == 0) ? 0 : attn_ws_with_counters(c, std::max(rows, 1));
    return KVC_OK;
}

int kvc_decode_attn(const kvc_cache* c, const void* q, int64_t q_layer_stride, int n_q_layers,
                    const int32_t* q_slot, int n_q_heads, float scale, const void* k_new,
                    const void* v_new, int append_slot, float* out, int64_t out_layer_stride,
                    float* lse, int64_t lse_layer_stride, void* ws, size_t ws_bytes,
                    kvc_stream_t stream) {
    int st = check_tiled(c);
    if (st) return st;
    if (n_q_layers < 0 || n_q_heads < 1 || n_q_heads % c->n_kv_heads) return KVC_EINVAL;
    const int g = n_q_heads / c->n_kv_heads;
    if (g > (c->dtype == KVC_F32 ? 16 : 64)) return KVC_EINVAL;
    if (append_slot < -1 || append_slot >= c->n_slots) return KVC_EINVAL;
    if (!isfinite(scale) || scale < 0.f) return KVC_EINVAL;
    const int64_t packed_q = (int64_t)c->nb * n_q_heads * KVC_HEAD_DIM;
    const int64_t packed_l = (int64_t)c->nb * n_q_heads;
    if (q_layer_stride < 0 || out_layer_stride < 0 || lse_layer_stride < 0) return KVC_EINVAL;
    if (q_layer_stride && q_layer_stride < packed_q) return KVC_EINVAL;
    if (out_layer_stride && out_layer_stride < packed_q) return KVC_EINVAL;
    if (lse_layer_stride && lse_layer_stride < packed_l) return KVC_EINVAL;
    if (n_q_layers == 0 || c->nb == 0) {
        if (append_slot < 0 || c->nb == 0) return KVC_OK;
    }
    if (c->t_len < 1) return KVC_EINVAL;
    if (n_q_layers > 0) {
        if (!q_slot) return KVC_EALIGN;
        for (int i = 0; i < n_q_layers; ++i)
            if (q_slot[i] < 0 || q_slot[i] >= c->n_slots) return KVC_EINVAL;
        if (!aligned16(q) || !aligned16(out)) return KVC_EALIGN;
        if (q_layer_stride % (16 / (int64_t)elem_size(c->dtype))) return KVC_EALIGN;
        if (lse && !aligned4(lse)) return KVC_EALIGN;
    }
    if (append_slot >= 0 && (!aligned16(k_new) || !aligned16(v_new))) return KVC_EALIGN;
    size_t need = 0;
    if (n_q_layers > 0) {
        const int rows = std::min(n_q_layers * g, max_rows_per_chunk(c->dtype, g));
        need = attn_ws_with_counters(c, rows);
        if (!ws || ws_bytes < need || !aligned16(ws)) return KVC_EWORKSPACE;
    }
    if (scale == 0.f) scale = 1.0f / sqrtf((float)KVC_HEAD_DIM);
    const hipStream_t s = (hipStream_t)stream;
    const int slabs = c->nb * c->n_kv_heads;

    bool append_done = false;
    const int64_t qs = q_layer_stride ? q_layer_stride : packed_q;
    const int64_t os = out_layer_stride ? out_layer_stride : packed_q;
    const int64_t ls = lse_layer_stride ? lse_layer_stride : packed_l;
    const int chunk_ql = max_rows_per_chunk(c->dtype, g) / g;
    st = for_each_attn_chunk(c->n_slots, n_q_layers, q_slot, chunk_ql,
                             [&](int slot, const int* members, int nql) {
        AttnLaunch p;
        fill_attn(p, c->nb, c->n_kv_heads, g, n_q_heads, c->t_len, c->t_cap, members, nql, qs,
                  os, ls, q, out, lse, scale);
        p.k = slot_k(c, slot);
        p.v = slot_v(c, slot);
        p.append_read = (slot == append_slot);
        p.append_write = (slot == append_slot) && !append_done;
        if (p.append_read) {
            p.k_new = k_new;
            p.v_new = v_new;
        }
        const AttnPlan pl = plan_attn(c->dtype, p.rows, c->t_len, slabs);
        p.rp = pl.rp;
        p.nsplit = pl.nsplit;
        p.tps = pl.tps;
        p.xcd_runs = pl.nsplit >= 8;
        p.part = reinterpret_cast<float*>(static_cast<char*>(ws) + ATTN_COUNTER_HEAD);
        if (c->dtype == KVC_BF16 && fuse_merge(p.rows, pl.nsplit, slabs))
            p.arrive = static_cast<unsigned*>(ws);
        p.sm = seq_map(c);
        if (launch_attn(p, c->dtype, pl.nt, s) != hipSuccess) return (int)KVC_EHIP;
        if (p.append_write) append_done = true;
        return (int)KVC_OK;
    });
    if (st) return st;
    if (append_slot >= 0 && !append_done) {
        if (launch_append(slot_k(c, append_slot), slot_v(c, append_slot), c->nb, c->n_kv_heads,
                          c->t_cap, seq_map(c), k_new, v_new, (int)elem_size(c->dtype),
                          s) != hipSuccess)
            return KVC_EHIP;
    }
    return hip_status();
}

int kvc_decode_attn_noalloc(const kvc_cache* c, const void* q, int64_t q_layer_stride,
                            int n_q_layers, const int32_t* q_slot, int n_q_heads, float scale,
                            const void* k_new, const void* v_new, int append_slot, float* out,
                            int64_t out_layer_stride, float* lse, int64_t lse_layer_stride,
                            kvc_stream_t stream) {
    size_t need = 0;
    int st = kvc_decode_attn_ws_bytes(c, n_q_layers, n_q_heads, &need);
    if (st) return st;
    if (need > (size_t)KVC_NOALLOC_SCRATCH_BYTES) return KVC_ESCRATCH;
    void* ws = nullptr;
    if (noalloc_scratch((hipStream_t)stream, &ws) != hipSuccess) return KVC_EHIP;
    return kvc_decode_attn(c, q, q_layer_stride, n_q_layers, q_slot, n_q_heads, scale, k_new,
                           v_new, append_slot, out, out_layer_stride, lse, lse_layer_stride, ws,
                           (size_t)KVC_NOALLOC_SCRATCH_BYTES, stream);
}

int kvc_value_range(const kvc_cache* c, int slot, float* range, kvc_stream_t stream) {
    int st = check_cache(c);
    if (st) return st;
    if (slot < 0 || slot >= c->n_slots) return KVC_EINVAL;
    if (!aligned4(range)) return KVC_EALIGN;
    if (c->nb == 0 || c->t_len == 0) return KVC_OK;
    if (launch_value_range(slot_v(c, slot), v_rows(c), c->nb, c->n_kv_heads, c->t_cap,
                           seq_map(c), c->dtype, range, (hipStream_t)stream) != hipSuccess)
        return KVC_EHIP;
    return hip_status();
}

int kvc_score_ws_bytes(const kvc_cache* c, int n_q_heads, int w, size_t* bytes) {
    int st = check_cache(c);
    if (st) return st;
    if (!bytes) return KVC_EALIGN;
    if (n_q_heads < 1 || n_q_heads % c->n_kv_heads || w < 1) return KVC_EINVAL;
    const int rows = (n_q_heads / c->n_kv_heads) * w;
    const int slabs = c->nb * c->n_kv_heads;
    size_t tot = 0;
    const int tile = c->dtype == KVC_F32 ? 64 : SCORE_TILE;
    for (int t = w; t <= std::max(w, c->t_cap); t += tile)
        tot = std::max(tot, score_ws_layout(c->dtype, rows, t, slabs).total);
    tot = std::max(tot, score_ws_layout(c->dtype, rows, std::max(w, c->t_cap), slabs).total);
    *bytes = slabs ? tot : 0;
    return KVC_OK;
}

int kvc_score(const kvc_cache* c, int slot, const void* q_obs, int n_q_heads, int w, float scale,
              const float* lse_obs, float* score, float* range, void* ws, size_t ws_bytes,
              kvc_stream_t stream) {
    return kvc_score_seq(c, slot, q_obs, c ? c->nb : 0, nullptr, n_q_heads, w, scale, lse_obs,
                         score, range, ws, ws_bytes, stream);
}

int kvc_score_seq(const kvc_cache* c, int slot, const void* q_obs, int q_nb, const int32_t* q_idx,
                  int n_q_heads, int w, float scale, const float* lse_obs, float* score,
                  float* range, void* ws, size_t ws_bytes, kvc_stream_t stream) {
    int st = check_cache(c);
    if (st) return st;
    if (slot < 0 || slot >= c->n_slots) return KVC_EINVAL;
    if (n_q_heads < 1 || n_q_heads % c->n_kv_heads || w < 1) return KVC_EINVAL;
    const int g = n_q_heads / c->n_kv_heads;
    const int rows = g * w;
    if (rows > (c->dtype == KVC_F32 ? 128 : 512)) return KVC_EINVAL;
    if (!isfinite(scale) || scale < 0.f) return KVC_EINVAL;
    if (q_nb < 0 || (!q_idx && q_nb < c->nb)) return KVC_EINVAL;
    if (c->nb == 0) return KVC_OK;
    if (w > c->t_len) return KVC_EINVAL;
    if (!aligned16(q_obs) || !aligned4(score)) return KVC_EALIGN;
    if (q_idx && !aligned4(q_idx)) return KVC_EALIGN;
    if ((lse_obs && !aligned4(lse_obs)) || (range && !aligned4(range))) return KVC_EALIGN;
    const int slabs = c->nb * c->n_kv_heads;
    const ScoreWs lay = score_ws_layout(c->dtype, rows, c->t_len, slabs);
    if (!lse_obs && (!ws || ws_bytes < lay.total || !aligned16(ws))) return KVC_EWORKSPACE;
    if (scale == 0.f) scale = 1.0f / sqrtf((float)KVC_HEAD_DIM);
    const ScorePlan pl = plan_score(c->dtype, rows, c->t_len, slabs);
    ScoreLaunch p;
    memset(&p, 0, sizeof(p));
    p.k = slot_k(c, slot);
    p.v = slot_v(c, slot);
    p.nb = c->nb;
    p.hkv = c->n_kv_heads;
    p.g = g;
    p.hq = n_q_heads;
    p.w = w;
    p.t_len = c->t_len;
    p.t_cap = c->t_cap;
    p.rows = rows;
    p.q_obs = q_obs;
    p.lse_obs = lse_obs;
    p.q_idx = q_idx;
    p.q_nb = q_nb;
    p.scale = scale;
    p.score = score;
    // Values stored as rows: the score pass reads the keys only and the
    // range comes from the rows kernel (the same bytes, one launch more).
    p.range = v_rows(c) ? nullptr : range;
    p.nsplit = pl.nsplit;
    p.tps = pl.tps;
    p.main_nsplit = pl.main_nsplit;
    p.main_tps = pl.main_tps;
    p.rows_pad = pl.rows_pad;
    p.sm = seq_map(c);
    if (!lse_obs) {
        char* base = static_cast<char*>(ws);
        p.lse_ws = reinterpret_cast<float*>(base + lay.lse_off);
        p.stats = reinterpret_cast<float*>(base + lay.stats_off);
    }
    if (launch_score(p, c->dtype, (hipStream_t)stream) != hipSuccess) return KVC_EHIP;
    if (range && v_rows(c) &&
        launch_value_range(slot_v(c, slot), true, c->nb, c->n_kv_heads, c->t_cap, seq_map(c),
                           c->dtype, range, (hipStream_t)stream) != hipSuccess)
        return KVC_EHIP;
    return hip_status();
}

int kvc_select_ws_bytes(int nb, int n_kv_heads, int t_len, size_t* bytes) {
    if (!bytes) return KVC_EALIGN;
    if (nb < 0 || n_kv_heads < 1 || t_len < 0) return KVC_EINVAL;
    *bytes = 2 * (size_t)nb * n_kv_heads * t_len * sizeof(uint32_t);
    return KVC_OK;
}

int kvc_select(const float* score, const float* range, int nb, int n_kv_heads, int t_len,
               int budget_k, int recent_b, int n_v, uint64_t seed, int layer_id, int32_t* kept,
               void* ws, size_t ws_bytes, kvc_stream_t stream) {
    return kvc_select_seq(score, range, nb, n_kv_heads, t_len, nullptr, nullptr, budget_k,
                          recent_b, n_v, seed, layer_id, kept, ws, ws_bytes, stream);
}

int kvc_select_seq(const float* score, const float* range, int nb, int n_kv_heads, int t_len,
                   const int32_t* seq_len, const int32_t* seq_id, int budget_k, int recent_b,
                   int n_v, uint64_t seed, int layer_id, int32_t* kept, void* ws,
                   size_t ws_bytes, kvc_stream_t stream) {
    if (nb < 0 || n_kv_heads < 1 || t_len < 0) return KVC_EINVAL;
    if (budget_k < 0 || recent_b < 0 || n_v < 0 || n_v > budget_k) return KVC_EINVAL;
    if ((long long)budget_k + recent_b < 1 || (long long)budget_k + recent_b > INT32_MAX)
        return KVC_EINVAL;
    if (layer_id < 0) return KVC_EINVAL;
    if (nb == 0 || t_len == 0) return KVC_OK;
    if (!aligned4(score) || !aligned4(kept)) return KVC_EALIGN;
    if (n_v > 0 && !aligned4(range)) return KVC_EALIGN;
    if ((seq_len && !aligned4(seq_len)) || (seq_id && !aligned4(seq_id))) return KVC_EALIGN;
    const size_t need = 2 * (size_t)nb * n_kv_heads * t_len * sizeof(uint32_t);
    const bool evicts = t_len > budget_k + recent_b;
    if (evicts && (!ws || ws_bytes < need || !aligned4(ws))) return KVC_EWORKSPACE;
    SelectLaunch p;
    memset(&p, 0, sizeof(p));
    p.score = score;
    p.range = range ? range : score;
    p.nb = nb;
    p.hkv = n_kv_heads;
    p.t_len = t_len;
    p.budget_k = budget_k;
    p.recent_b = recent_b;
    p.n_v = n_v;
    p.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
    p.seed_hi = (uint32_t)(seed >> 32);
    p.layer_id = (uint32_t)layer_id;
    p.kept = kept;
    p.keys = static_cast<uint32_t*>(ws);
    p.kappa = p.keys + (size_t)nb * n_kv_heads * t_len;
    p.len = seq_len;
    p.seq_id = seq_id;
    if (launch_select(p, (hipStream_t)stream) != hipSuccess) return KVC_EHIP;
    return hip_status();
}

int kvc_compact(const kvc_cache* src, int slot, const int32_t* kept, int n_keep,
                const kvc_cache* dst, kvc_stream_t stream) {
    int st = check_cache(src);
    if (st) return st;
    st = check_tiled(dst);
    if (st) return st;
    if (src->dtype != dst->dtype) return KVC_EDTYPE;
    if (src->nb != dst->nb || src->n_kv_heads != dst->n_kv_heads) return KVC_EINVAL;
    if (slot < 0 || slot >= src->n_slots || slot >= dst->n_slots) return KVC_EINVAL;
    if (n_keep < 0 || n_keep > src->t_len || n_keep > dst->t_cap) return KVC_EINVAL;
    if (src->nb == 0 || n_keep == 0) return KVC_OK;
    if (kept && !aligned4(kept)) return KVC_EALIGN;
    const size_t es = elem_size(src->dtype);
    const size_t sb = slot_elems(src) * es, db = slot_elems(dst) * es;
    const char* sr[2] = {slot_k(src, slot), slot_v(src, slot)};
    const char* dr[2] = {slot_k(dst, slot), slot_v(dst, slot)};
    // With batch maps the two sides may share buffers (other entries of one
    // cache); the maps themselves live on the device and keeping the
    // entries apart is the caller's part.  Without maps the regions must
    // not overlap at all.
    const bool mapped = src->batch_idx || dst->batch_idx;
    for (int a = 0; a < 2; ++a)
        for (int b2 = 0; b2 < 2; ++b2)
            if (!mapped && sr[a] < dr[b2] + db && dr[b2] < sr[a] + sb) return KVC_EALIAS;
    if (dr[0] < dr[1] + db && dr[1] < dr[0] + db) return KVC_EALIAS;
    CompactLaunch p;
    memset(&p, 0, sizeof(p));
    p.sk = sr[0];
    p.sv = sr[1];
    p.dk = const_cast<char*>(dr[0]);
    p.dv = const_cast<char*>(dr[1]);
    p.nb = src->nb;
    p.hkv = src->n_kv_heads;
    p.src_t_cap = src->t_cap;
    p.dst_t_cap = dst->t_cap;
    p.kept = kept;
    p.n_keep = n_keep;
    p.elem = (int)es;
    p.src_sm = seq_map(src);
    p.dst_sm = seq_map(dst);
    p.src_rows = v_rows(src);
    if (launch_compact(p, (hipStream_t)stream) != hipSuccess) return KVC_EHIP;
    return hip_status();
}

int kvc_q8_quantize(const kvc_cache* src, int slot, const int32_t* protect, int n_protect,
                    const kvc_qcache* dst, kvc_stream_t stream) {
    int st = check_tiled(src);
    if (st) return st;
    st = check_qcache(dst);
    if (st) return st;
    if (src->dtype != KVC_BF16) return KVC_EDTYPE;
    if (is_ragged(src) || nb_cap_of(src) != src->nb) return KVC_EINVAL;   // uniform batches only
    if (src->nb != dst->nb || src->n_kv_heads != dst->n_kv_heads) return KVC_EINVAL;
    if (slot < 0 || slot >= src->n_slots || slot >= dst->n_slots) return KVC_EINVAL;
    if (dst->t_len != src->t_len || dst->p_len != n_protect) return KVC_EINVAL;
    if (n_protect < 0 || n_protect > dst->p_cap || n_protect > src->t_len) return KVC_EINVAL;
    if (src->nb == 0 || src->t_len == 0) return KVC_OK;
    if (n_protect > 0 && !aligned4(protect)) return KVC_EALIGN;
    const hipStream_t s = (hipStream_t)stream;
    Q8QuantLaunch p;
    memset(&p, 0, sizeof(p));
    p.k = slot_k(src, slot);
    p.v = slot_v(src, slot);
    p.nb = src->nb;
    p.hkv = src->n_kv_heads;
    p.t_len = src->t_len;
    p.src_t_cap = src->t_cap;
    p.protect = protect;
    p.n_protect = n_protect;
    p.kq = q_kq(dst, slot);
    p.vq = q_vq(dst, slot);
    p.sk = q_sk(dst, slot);
    p.sv = q_sv(dst, slot);
    p.dst_t_cap = dst->t_cap;
    if (launch_q8_quantize(p, s) != hipSuccess) return KVC_EHIP;
    if (n_protect > 0) {
        // the protected rows, gathered into the bf16 mini-slabs
        CompactLaunch cp;
        memset(&cp, 0, sizeof(cp));
        cp.sk = slot_k(src, slot);
        cp.sv = slot_v(src, slot);
        cp.dk = q_kp(dst, slot);
        cp.dv = q_vp(dst, slot);
        cp.nb = src->nb;
        cp.hkv = src->n_kv_heads;
        cp.src_sm.t_len = src->t_len;
        cp.src_sm.nb_cap = cp.dst_sm.nb_cap = src->nb;
        cp.src_t_cap = src->t_cap;
        cp.dst_t_cap = dst->p_cap;
        cp.kept = protect;
        cp.n_keep = n_protect;
        cp.elem = 2;
        if (launch_compact(cp, s) != hipSuccess) return KVC_EHIP;
    }
    return hip_status();
}

int kvc_q8_append(const kvc_qcache* c, int slot, const void* k_new, const void* v_new,
                  kvc_stream_t stream) {
    int st = check_qcache(c);
    if (st) return st;
    if (slot < 0 || slot >= c->n_slots || c->t_len < 1) return KVC_EINVAL;
    if (!aligned16(k_new) || !aligned16(v_new)) return KVC_EALIGN;
    if (c->nb == 0) return KVC_OK;
    Q8QuantLaunch p;
    memset(&p, 0, sizeof(p));
    p.nb = c->nb;
    p.hkv = c->n_kv_heads;
    p.t_len = c->t_len;
    p.kq = q_kq(c, slot);
    p.vq = q_vq(c, slot);
    p.sk = q_sk(c, slot);
    p.sv = q_sv(c, slot);
    p.dst_t_cap = c->t_cap;
    p.k_row = k_new;
    p.v_row = v_new;
    if (launch_q8_quantize(p, (hipStream_t)stream) != hipSuccess) return KVC_EHIP;
    return hip_status();
}

int kvc_q8_decode_attn_ws_bytes(const kvc_qcache* c, int n_q_layers, int n_q_heads,
                                size_t* bytes) {
    int st = check_qcache(c);
    if (st) return st;
    if (!bytes) return KVC_EALIGN;
    if (n_q_layers < 0 || n_q_heads < 1 || n_q_heads % c->n_kv_heads) return KVC_EINVAL;
    const int g = n_q_heads / c->n_kv_heads;
    if (g > 64) return KVC_EINVAL;
    const int rows = std::min(std::max(1, n_q_layers) * g, max_rows_per_chunk(KVC_BF16, g));
    const int slabs = c->nb * c->n_kv_heads;
    const int vmax = ((c->t_cap + ATTN_TILE - 1) / ATTN_TILE +
                      (c->p_cap + ATTN_TILE - 1) / ATTN_TILE) * ATTN_TILE;
    size_t part = 0;
    for (int t = ATTN_TILE; t <= std::max(ATTN_TILE, vmax); t += ATTN_TILE)
        part = std::max(part, attn_ws_for(KVC_BF16, rows, t, slabs));
    *bytes = ATTN_COUNTER_HEAD + part;
    return KVC_OK;
}

int kvc_q8_decode_attn(const kvc_qcache* c, const void* q, int64_t q_layer_stride,
                       int n_q_layers, const int32_t* q_slot, int n_q_heads, float scale,
                       float* out, int64_t out_layer_stride, float* lse, int64_t lse_layer_stride,
                       void* ws, size_t ws_bytes, kvc_stream_t stream) {
    int st = check_qcache(c);
    if (st) return st;
    if (n_q_layers < 0 || n_q_heads < 1 || n_q_heads % c->n_kv_heads) return KVC_EINVAL;
    const int g = n_q_heads / c->n_kv_heads;
    if (g > 64) return KVC_EINVAL;
    if (!isfinite(scale) || scale < 0.f) return KVC_EINVAL;
    const int64_t packed_q = (int64_t)c->nb * n_q_heads * KVC_HEAD_DIM;
    const int64_t packed_l = (int64_t)c->nb * n_q_heads;
    if (q_layer_stride < 0 || out_layer_stride < 0 || lse_layer_stride < 0) return KVC_EINVAL;
    if (q_layer_stride && q_layer_stride < packed_q) return KVC_EINVAL;
    if (out_layer_stride && out_layer_stride < packed_q) return KVC_EINVAL;
    if (lse_layer_stride && lse_layer_stride < packed_l) return KVC_EINVAL;
    if (n_q_layers == 0 || c->nb == 0) return KVC_OK;
    if (c->t_len < 1) return KVC_EINVAL;
    if (!q_slot) return KVC_EALIGN;
    for (int i = 0; i < n_q_layers; ++i)
        if (q_slot[i] < 0 || q_slot[i] >= c->n_slots) return KVC_EINVAL;
    if (!aligned16(q) || !aligned16(out)) return KVC_EALIGN;
    if (q_layer_stride % 8) return KVC_EALIGN;
    if (lse && !aligned4(lse)) return KVC_EALIGN;
    size_t need = 0;
    st = kvc_q8_decode_attn_ws_bytes(c, n_q_layers, n_q_heads, &need);
    if (st) return st;
    if (!ws || ws_bytes < need || !aligned16(ws)) return KVC_EWORKSPACE;
    if (scale == 0.f) scale = 1.0f / sqrtf((float)KVC_HEAD_DIM);
    const hipStream_t s = (hipStream_t)stream;
    const int slabs = c->nb * c->n_kv_heads;
    const int64_t qs = q_layer_stride ? q_layer_stride : packed_q;
    const int64_t os = out_layer_stride ? out_layer_stride : packed_q;
    const int64_t ls = lse_layer_stride ? lse_layer_stride : packed_l;
    const int chunk_ql = max_rows_per_chunk(KVC_BF16, g) / g;
    const int vrows = q8_virtual_rows(c);
    st = for_each_attn_chunk(c->n_slots, n_q_layers, q_slot, chunk_ql,
                             [&](int slot, const int* members, int nql) {
        Q8AttnLaunch p;
        memset(&p, 0, sizeof(p));
        fill_attn(p.a, c->nb, c->n_kv_heads, g, n_q_heads, c->t_len, c->t_cap, members, nql, qs,
                  os, ls, q, out, lse, scale);
        p.a.k = q_kq(c, slot);
        p.a.v = q_vq(c, slot);
        const AttnPlan pl = plan_attn(KVC_BF16, p.a.rows, vrows, slabs);
        p.a.rp = pl.rp;
        p.a.nsplit = pl.nsplit;
        p.a.tps = pl.tps;
        p.a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + ATTN_COUNTER_HEAD);
        if (fuse_merge(p.a.rows, pl.nsplit, slabs)) p.a.arrive = static_cast<unsigned*>(ws);
        p.sk = q_sk(c, slot);
        p.sv = q_sv(c, slot);
        p.kp = q_kp(c, slot);
        p.vp = q_vp(c, slot);
        p.p_len = c->p_len;
        p.p_cap = c->p_cap;
        p.nq_tiles = (c->t_len + ATTN_TILE - 1) / ATTN_TILE;
        if (launch_attn_q8(p, pl.nt, s) != hipSuccess) return (int)KVC_EHIP;
        return (int)KVC_OK;
    });
    if (st) return st;
    return hip_status();
}

int kvc_dkv_ws_bytes(const kvc_cache* c, int rank, size_t* bytes) {
    int st = check_cache(c);
    if (st) return st;
    if (!bytes) return KVC_EALIGN;
    if (rank != 16 && rank != 32) return KVC_EINVAL;
    const int slabs = c->nb * c->n_kv_heads;
    *bytes = dkv_layout(rank, std::max(c->t_len, c->t_cap), slabs).total;
    return KVC_OK;
}

int kvc_dkv_score(const kvc_cache* c, int slot, const void* g, int rank, float* score,
                  float* range, void* ws, size_t ws_bytes, kvc_stream_t stream) {
    int st = check_cache(c);
    if (st) return st;
    if (c->dtype != KVC_BF16) return KVC_EDTYPE;
    if (slot < 0 || slot >= c->n_slots) return KVC_EINVAL;
    if (rank != 16 && rank != 32) return KVC_EINVAL;
    if (c->nb == 0 || c->t_len == 0) return KVC_OK;
    if (!aligned16(g) || !aligned4(score) || (range && !aligned4(range))) return KVC_EALIGN;
    const int slabs = c->nb * c->n_kv_heads;
    const DkvWs lay = dkv_layout(rank, c->t_len, slabs);
    if (!ws || ws_bytes < lay.total || !aligned16(ws)) return KVC_EWORKSPACE;
    DkvLaunch p;
    memset(&p, 0, sizeof(p));
    p.k = slot_k(c, slot);
    p.v = slot_v(c, slot);
    p.nb = c->nb;
    p.hkv = c->n_kv_heads;
    p.t_len = c->t_len;
    p.t_cap = c->t_cap;
    p.g = g;
    p.rank = rank;
    p.score = score;
    p.range = range;
    p.nsplit = lay.nsplit;
    p.tps = lay.tps;
    char* base = static_cast<char*>(ws);
    p.y = reinterpret_cast<float*>(base + lay.y_off);
    p.gram = reinterpret_cast<double*>(base + lay.gram_off);
    p.w = reinterpret_cast<double*>(base + lay.w_off);
    p.sm = seq_map(c);
    p.v_rows = v_rows(c);
    if (launch_dkv(p, (hipStream_t)stream) != hipSuccess) return KVC_EHIP;
    return hip_status();
}

int kvc_xkv_factor_ws_bytes(const kvc_xkv* x, size_t* bytes) {
    int st = check_xkv(x);
    if (st) return st;
    if (!bytes) return KVC_EALIGN;
    *bytes = xkv_ws(x).total;
    return KVC_OK;
}

int kvc_xkv_factor(const kvc_cache* c, int slot0, int iters, uint64_t seed, const kvc_xkv* x,
                   void* ws, size_t ws_bytes, kvc_stream_t stream) {
    int st = check_tiled(c);
    if (st) return st;
    st = check_xkv(x);
    if (st) return st;
    if (c->dtype != KVC_BF16) return KVC_EDTYPE;
    if (is_ragged(c) || nb_cap_of(c) != c->nb) return KVC_EINVAL;   // uniform batches only
    if (slot0 < 0 || slot0 + x->window > c->n_slots) return KVC_EINVAL;
    if (x->nb != c->nb || x->n_kv_heads != c->n_kv_heads) return KVC_EINVAL;
    if (x->t_len != c->t_len) return KVC_EINVAL;
    if (iters < 1 || iters > 64) return KVC_EINVAL;
    if (c->nb == 0 || c->t_len == 0) return KVC_OK;
    const XkvWs lay = xkv_ws(x);
    if (!ws || ws_bytes < lay.total || !aligned16(ws)) return KVC_EWORKSPACE;
    XkvLaunch p;
    memset(&p, 0, sizeof(p));
    p.k = slot_k(c, slot0);
    p.v = slot_v(c, slot0);
    p.slot_stride = slot_elems(c);
    p.nb = c->nb;
    p.hkv = c->n_kv_heads;
    p.t_len = c->t_len;
    p.t_cap = c->t_cap;
    p.window = x->window;
    p.rank = x->rank;
    char* base = static_cast<char*>(ws);
    p.gram = reinterpret_cast<float*>(base + lay.gram_off);
    p.vt = reinterpret_cast<uint16_t*>(base + lay.vt_off);
    p.ak = x->ak;
    p.av = x->av;
    p.lk = x->lk;
    p.bk = x->bk;
    p.bv = x->bv;
    p.x_tcap = x->t_cap;
    p.iters = iters;
    p.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
    p.seed_hi = (uint32_t)(seed >> 32);
    // projection: about two workgroups per CU, at least four tiles per wave
    const int ntiles = (c->t_len + 31) / 32;
    const long long work = (long long)ntiles * c->nb * c->n_kv_heads;
    p.tps = (int)std::max<long long>(16, (work + 2 * CU_COUNT - 1) / (2 * CU_COUNT));
    p.nsplit = (ntiles + p.tps - 1) / p.tps;
    if (launch_xkv_factor(p, (hipStream_t)stream) != hipSuccess) return KVC_EHIP;
    return hip_status();
}

int kvc_xkv_decode_ws_bytes(const kvc_xkv* x, int n_q_heads, int n_select, size_t* bytes) {
    int st = check_xkv(x);
    if (st) return st;
    if (!bytes) return KVC_EINVAL;
    if (n_q_heads < 1 || n_q_heads % x->n_kv_heads) return KVC_EINVAL;
    const int g = n_q_heads / x->n_kv_heads;
    if (g > XKV_MAXG) return KVC_EINVAL;
    if (n_select < 1) return KVC_EINVAL;
    *bytes = plan_xkv_decode(x, n_select).ws_bytes;
    return KVC_OK;
}

int kvc_xkv_decode_attn(const kvc_xkv* x, int layer, const void* q, int n_q_heads, float scale,
                        int n_select, const float* o_in, const float* lse_in, float* out,
                        float* lse, int32_t* selected, void* ws, size_t ws_bytes,
                        kvc_stream_t stream) {
    int st = check_xkv(x);
    if (st) return st;
    if (layer < 0 || layer >= x->window) return KVC_EINVAL;
    if (n_q_heads < 1 || n_q_heads % x->n_kv_heads) return KVC_EINVAL;
    const int g = n_q_heads / x->n_kv_heads;
    if (g > XKV_MAXG) return KVC_EINVAL;
    if (n_select < 1) return KVC_EINVAL;
    if (!isfinite(scale) || scale < 0.f) return KVC_EINVAL;
    if ((o_in == nullptr) != (lse_in == nullptr)) return KVC_EINVAL;
    if (x->nb == 0) return KVC_OK;
    if (!aligned16(q) || !aligned4(out)) return KVC_EALIGN;
    if ((lse && !aligned4(lse)) || (o_in && (!aligned4(o_in) || !aligned4(lse_in))) ||
        (selected && !aligned4(selected)))
        return KVC_EALIGN;
    const XkvDecodePlan pl = plan_xkv_decode(x, n_select);
    if (pl.lds > XKV_DECODE_LDS_LIMIT) return KVC_EINVAL;
    if (!ws || ws_bytes < pl.ws_bytes || !aligned16(ws)) return KVC_EWORKSPACE;
    if (scale == 0.f) scale = 1.0f / sqrtf((float)KVC_HEAD_DIM);
    XkvDecodeLaunch p;
    memset(&p, 0, sizeof(p));
    p.ak = x->ak;
    p.av = x->av;
    p.lk = x->lk;
    p.bk = x->bk;
    p.bv = x->bv;
    p.nb = x->nb;
    p.hkv = x->n_kv_heads;
    p.g = g;
    p.hq = n_q_heads;
    p.t_len = x->t_len;
    p.x_tcap = x->t_cap;
    p.window = x->window;
    p.rank = x->rank;
    p.layer = layer;
    p.n_select = n_select;
    p.q = q;
    p.scale = scale;
    p.o_in = o_in;
    p.lse_in = lse_in;
    p.out = out;
    p.lse = lse;
    p.selected = selected;
    char* w = static_cast<char*>(ws);
    p.ns = pl.ns;
    p.ws_keys = reinterpret_cast<uint32_t*>(w + pl.keys_off);
    p.ws_qt = reinterpret_cast<float*>(w + pl.qt_off);
    p.ws_part = reinterpret_cast<float*>(w + pl.part_off);
    p.ws_arrive = reinterpret_cast<unsigned*>(w + pl.arrive_off);
    if (launch_xkv_decode(p, pl.gkeys, pl.lds, (hipStream_t)stream) != hipSuccess) return KVC_EHIP;
    return hip_status();
}

int kvc_gaussian_bf16(int64_t n, uint64_t seed, uint32_t c1, uint32_t c2, void* out,
                      kvc_stream_t stream) {
    if (n < 0 || n > (int64_t)1 << 32) return KVC_EINVAL;
    if (n == 0) return KVC_OK;
    if (!aligned4(out)) return KVC_EALIGN;
    if (launch_gaussian(n, c1, c2, (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32), out,
                        (hipStream_t)stream) != hipSuccess)
        return KVC_EHIP;
    return hip_status();
}

int kvc_read_probe(const void* buf, size_t bytes, uint32_t* out, kvc_stream_t stream) {
    static_assert(KVC_PROBE_BLOCKS == PROBE_BLOCKS, "probe grid");
    if (bytes % 16) return KVC_EINVAL;
    if (!aligned4(out) || (bytes && !aligned16(buf))) return KVC_EALIGN;
    if (launch_read_probe(buf, bytes, out, (hipStream_t)stream) != hipSuccess) return KVC_EHIP;
    return hip_status();
}

int kvc_philox_words(int64_t n, uint32_t c1, uint32_t c2, uint32_t c3, uint64_t seed,
                     uint32_t* out, kvc_stream_t stream) {
    if (n < 0 || n > (int64_t)1 << 32) return KVC_EINVAL;
    if (n == 0) return KVC_OK;
    if (!aligned16(out)) return KVC_EALIGN;
    if (launch_philox(n, c1, c2, c3, (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32), out,
                      (hipStream_t)stream) != hipSuccess)
        return KVC_EHIP;
    return hip_status();
}

}  // extern "C"
