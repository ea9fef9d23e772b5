// C entry points of libpa: argument checks, workspace layout, split policy and launches.
// Every check runs before anything is enqueued; device-resident index contents are the
// caller's contract (see include/pa.h).
#include <math.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <numeric>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace pa {

// ---------------------------------------------------------------------------------------------
// Timing hooks
// ---------------------------------------------------------------------------------------------
namespace {
struct TimingRec {
    std::string name;
    hipEvent_t start, stop;
};
std::atomic<int> g_timing{0};
std::mutex g_timing_mu;
std::vector<TimingRec> g_pending;
std::vector<hipEvent_t> g_free;  // recycled events
std::map<std::string, std::pair<double, int64_t>> g_done;

hipEvent_t take_event() {  // caller holds g_timing_mu
    if (!g_free.empty()) {
        hipEvent_t e = g_free.back();
        g_free.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}
}  // namespace

LaunchScope::LaunchScope(const char *name, hipStream_t stream, int launches)
    : name_(name), stream_(stream), start_(nullptr), stop_(nullptr), n_(launches), idx_(0) {
    if (!g_timing.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lk(g_timing_mu);
    start_ = take_event();
    stop_ = take_event();
    if (!start_ || !stop_) {
        if (start_) g_free.push_back(start_);
        if (stop_) g_free.push_back(stop_);
        start_ = stop_ = nullptr;
    }
}

LaunchScope::~LaunchScope() {
    if (!start_) return;
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (idx_ == n_) {
        g_pending.push_back(TimingRec{name_, start_, stop_});
    } else {  // not every planned kernel was launched (error or early exit): drop the record
        g_free.push_back(start_);
        g_free.push_back(stop_);
    }
}

int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
        v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

// ---------------------------------------------------------------------------------------------
// Paged attention planning (host side of the split policy and workspace layout)
// ---------------------------------------------------------------------------------------------
namespace {

constexpr size_t kAlign = 256;
constexpr int kSplitMinKeys = 128;      // manifest tunable SPLIT_MIN_KEYS
constexpr int kMaxSplits = 16;          // manifest tunable MAX_SPLITS
constexpr int kSplitTargetWg = 1024;    // manifest tunable SPLIT_TARGET_WORKGROUPS
constexpr int kWavesPerCu = 8;          // resident decode waves per CU (2 per SIMD)
// Stream-K decode shares: one per resident workgroup on 7/8 of the CUs. Plain reads of the
// cache's random blocks reach the same rate from 192 workgroups up, and fewer shares mean fewer
// pieces, partials and start-up chains: 224 shares on 256 CUs 182.5 -> 179.4 us (208: 180.0,
// 240: 181.2) on the batch-64 decode.
constexpr int kDecodeCusNum = 7, kDecodeCusDen = 8;
// Waves of a decode workgroup that runs beside a prefill workgroup on each CU (the prefill
// workgroup's shape). Measured on the batch-64 decode: one such workgroup per CU (1024 waves)
// reads the cache in 190.8 us against 179.4 us for 224 workgroups of 8 waves.
constexpr int kFusedDecodeWaves = kPrefillCols / 32;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct PagedPlan {
    int Q, ncb_dec, tpi_dec, tpi_pre;
    int kv_div, Gv;  // query-head groups per cache head, and groups in all (Gv = G * kv_div)
    bool fused;  // decode and prefill items in one launch (decode_prefill)
    int mode, splits, gw, slots;
    int cap_dec, cap_pre, cap_comb, unit_cap;
    size_t off_dec, off_pre, off_comb, off_slot, off_first, off_o, off_m, off_l, total;
};

pa_status check_shape(const pa_paged_shape *s) {
    if (!s) return PA_ERR_NULL;
    if (s->batch < 1 || s->num_tokens < 0 || s->num_heads <= 0 || s->kv_num_heads <= 0 ||
        s->num_heads % s->kv_num_heads != 0 || s->head_size <= 0 || s->num_blocks < 1 ||
        s->block_size < 1 || s->max_blocks < 1 || (s->packed_qkv != 0 && s->packed_qkv != 1))
        return PA_ERR_SHAPE;
    if (s->head_size != 64 && s->head_size != 128 && s->head_size != 256)
        return PA_ERR_UNSUPPORTED;
    if ((long long)s->kv_num_heads * s->head_size >= (1LL << 24)) return PA_ERR_UNSUPPORTED;
    // the kernels form in-block row offsets with 24 x 24-bit multiplies: a block's elements
    // must fit in 32 bits
    if ((long long)s->block_size * s->kv_num_heads * s->head_size >= (1LL << 32))
        return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

int page_rule_splits(const pa_paged_shape *s) {
    const long long ceiling = (long long)s->max_blocks * s->block_size;
    const long long cap = std::max(1LL, std::min((long long)kMaxSplits, ceiling / kSplitMinKeys));
    const long long base = std::max(1LL, (long long)s->num_tokens * s->kv_num_heads);
    const long long want = (kSplitTargetWg + base - 1) / base;
    return (int)std::max(1LL, std::min(cap, want));
}

bool make_plan(const pa_paged_shape *s, int num_splits, PagedPlan &p) {
    if (check_shape(s) != PA_OK || num_splits < PA_SPLITS_PAGE_RULE) return false;
    const int T = s->num_tokens, B = s->batch, H = s->num_heads;
    const int D = s->head_size;
    // A kv head with more query heads than the decode waves take (64; 16 at D = 256, where one
    // column block fills a wave's registers) is served as kv_div groups of at most 16 heads
    // (the smallest such divisor of H / G_cache), each group reading the same cache head.
    const int Qc = H / s->kv_num_heads;
    p.kv_div = 1;
    if (Qc > (D == 256 ? 16 : 64))
        for (p.kv_div = 2; Qc % p.kv_div != 0 || Qc / p.kv_div > 16; ++p.kv_div) {}
    p.Gv = s->kv_num_heads * p.kv_div;
    const int G = p.Gv;
    p.Q = H / G;
    p.gw = 0;  // set below from the decode kernel's column blocks
    p.ncb_dec = p.Q <= 16 ? 1 : (p.Q <= 32 ? 2 : 4);
    p.tpi_dec = 16 * p.ncb_dec / p.Q;
    // decode waves per workgroup (kv heads of an item side by side) and resident per CU: at
    // D = 256 one wave per SIMD (its tiles need the whole register file)
    const int dec_waves = D == 256 ? 4 : 8;
    p.gw = p.ncb_dec == 1 ? std::gcd(G, dec_waves) : 1;
    p.tpi_pre = std::max(1, kPrefillCols / p.Q);  // one prefill workgroup: kPrefillCols columns
    // Decode and prefill run in one launch when the call surely has prefill items (more tokens
    // than B decode items hold, so some sequence has more new tokens than a decode item) and the
    // decode workgroups can take the prefill workgroups' shape (kPrefillCols / 32 waves, one kv
    // head each): then every CU holds one decode and one prefill workgroup, and the prefill's
    // matrix work hides under the decode's memory time. Otherwise the decode kernel runs alone
    // with its own layout and the prefill follows it.
    p.fused = p.ncb_dec == 1 && G % kFusedDecodeWaves == 0 && D <= 128 &&
              (long long)T > (long long)B * p.tpi_dec;
    if (p.fused) p.gw = kFusedDecodeWaves;
    if (num_splits == PA_SPLITS_AUTO) {
        p.mode = 0;
        p.splits = 0;
        // one share per resident decode workgroup (gw waves each, kWavesPerCu waves per CU) on
        // kDecodeCusNum / kDecodeCusDen of the CUs; beside the prefill, one per CU
        p.slots = p.fused ? device_cu_count()
                          : std::max(1, device_cu_count() * kDecodeCusNum / kDecodeCusDen *
                                            (D == 256 ? 4 : kWavesPerCu) / p.gw);
        p.cap_dec = p.slots + B;   // each share boundary adds at most one piece
        p.unit_cap = p.tpi_dec * p.cap_dec;
    } else {
        p.mode = 1;
        p.splits = num_splits == PA_SPLITS_PAGE_RULE ? page_rule_splits(s) : num_splits;
        p.slots = 0;
        const long long cd = (long long)p.splits * B;
        if (cd > (1LL << 30)) return false;
        p.cap_dec = (int)cd;
        const long long uc = p.splits >= 2 ? (long long)p.splits * T : 0;
        if (uc > (1LL << 30)) return false;
        p.unit_cap = (int)uc;
    }
    p.cap_pre = T / p.tpi_pre + T / (p.tpi_dec + 1) + 1;
    p.cap_comb = std::max(1, T);
    size_t off = align_up(sizeof(PlanHeader));
    p.off_dec = off;
    off = align_up(off + sizeof(AttnItem) * (size_t)p.cap_dec);
    p.off_pre = off;
    off = align_up(off + sizeof(AttnItem) * (size_t)p.cap_pre);
    p.off_comb = off;
    off = align_up(off + sizeof(CombItem) * (size_t)p.cap_comb);
    p.off_slot = off;
    off = align_up(off + sizeof(int32_t) * (size_t)(p.slots + 1));
    p.off_first = off;
    off = align_up(off + sizeof(AttnItem) * (size_t)p.slots);
    p.off_o = off;
    off = align_up(off + sizeof(float) * (size_t)p.unit_cap * H * D);
    p.off_m = off;
    off = align_up(off + sizeof(float) * (size_t)p.unit_cap * H);
    p.off_l = off;
    off = align_up(off + sizeof(float) * (size_t)p.unit_cap * H);
    p.total = off;
    return true;
}

int log2_pow2_ge8(int bs) {
    if (bs < 8 || (bs & (bs - 1))) return -1;
    int l = 0;
    while ((1 << l) < bs) ++l;
    return l;
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" {

const char *pa_status_string(pa_status status) {
    switch (status) {
        case PA_OK: return "ok";
        case PA_ERR_NULL: return "a required pointer is NULL";
        case PA_ERR_SHAPE: return "sizes or attributes violate the op contract";
        case PA_ERR_UNSUPPORTED: return "configuration not implemented by this build";
        case PA_ERR_WORKSPACE: return "workspace too small";
        case PA_ERR_HIP: return "HIP runtime error while enqueueing";
        default: return "unknown status";
    }
}

void pa_timing_enable(int32_t on) { g_timing.store(on ? 1 : 0); }

void pa_timing_reset(void) {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    for (auto &r : g_pending) {
        (void)hipEventSynchronize(r.stop);
        g_free.push_back(r.start);
        g_free.push_back(r.stop);
    }
    g_pending.clear();
    g_done.clear();
}

pa_status pa_timing_get(const char *kernel, double *total_ms, int64_t *launches) {
    if (!total_ms || !launches) return PA_ERR_NULL;
    std::lock_guard<std::mutex> lk(g_timing_mu);
    pa_status st = PA_OK;
    for (auto &r : g_pending) {
        float ms = 0.f;
        if (hipEventSynchronize(r.stop) != hipSuccess ||
            hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
            st = PA_ERR_HIP;
        auto &d = g_done[r.name];
        d.first += ms;
        d.second += 1;
        g_free.push_back(r.start);
        g_free.push_back(r.stop);
    }
    g_pending.clear();
    double t = 0.0;
    int64_t n = 0;
    for (auto &kv : g_done) {
        if (kernel && kv.first != kernel) continue;
        t += kv.second.first;
        n += kv.second.second;
    }
    *total_ms = t;
    *launches = n;
    return st;
}

// Checks and kernel arguments of one append (nothing is enqueued).
static pa_status make_append(const pa_paged_shape *shape, const void *query, const void *key,
                             const void *value, void *key_cache, void *value_cache,
                             const int32_t *cumulative_sequence_length,
                             const int32_t *past_seqlens, const int32_t *block_table,
                             const int32_t *slot_mapping, const void *cos_cache,
                             const void *sin_cache, int32_t rotary_dim, int32_t rotary_mode,
                             int32_t rotary_positions, void *q_out, AppendArgs &a) {
    pa_status st = check_shape(shape);
    if (st != PA_OK) return st;
    const pa_paged_shape &s = *shape;
    if (s.packed_qkv) {
        if (key || value) return PA_ERR_SHAPE;
        if (!query) return PA_ERR_NULL;
    } else {
        if ((key == nullptr) != (value == nullptr)) return PA_ERR_SHAPE;
        if (!key) return PA_ERR_NULL;
    }
    if (!key_cache || !value_cache || !cumulative_sequence_length || !past_seqlens)
        return PA_ERR_NULL;
    if (!slot_mapping && !block_table) return PA_ERR_NULL;
    if (rotary_mode != PA_ROTARY_NONE && rotary_mode != PA_ROTARY_NEOX &&
        rotary_mode != PA_ROTARY_INTERLEAVED)
        return PA_ERR_SHAPE;
    if (rotary_mode != PA_ROTARY_NONE) {
        if (rotary_dim <= 0 || rotary_dim % 2 != 0 || rotary_dim > s.head_size ||
            rotary_positions < 1)
            return PA_ERR_SHAPE;
        if (!cos_cache || !sin_cache) return PA_ERR_NULL;
    }
    const int H = s.num_heads, G = s.kv_num_heads, D = s.head_size;
    a.query = s.packed_qkv ? (const half_t *)query : nullptr;
    a.key = (const half_t *)key;
    a.value = (const half_t *)value;
    a.kc = (half_t *)key_cache;
    a.vc = (half_t *)value_cache;
    a.cu = cumulative_sequence_length;
    a.past = past_seqlens;
    a.bt = block_table;
    a.slot_mapping = slot_mapping;
    a.cos = (const half_t *)cos_cache;
    a.sin = (const half_t *)sin_cache;
    a.src_stride = s.packed_qkv ? (int64_t)(H + 2 * G) * D : (int64_t)G * D;
    a.k_off = s.packed_qkv ? (int64_t)H * D : 0;
    a.v_off = s.packed_qkv ? (int64_t)(H + G) * D : 0;
    a.T = s.num_tokens;
    a.B = s.batch;
    a.G = G;
    a.D = D;
    a.bs = s.block_size;
    a.MB = s.max_blocks;
    a.rotary_dim = rotary_mode == PA_ROTARY_NONE ? 0 : rotary_dim;
    a.rotary_mode = rotary_mode;
    a.q_out = (half_t *)q_out;
    a.q_src = (const half_t *)query;  // set for either layout (a.query is the packed rows only)
    a.q_stride = s.packed_qkv ? (int64_t)(H + 2 * G) * D : (int64_t)H * D;
    a.H = H;
    a.nkv = a.nkv_pad = a.nq = 0;  // set by the launcher
    return s.num_tokens == 0 ? PA_OK : check_kv_append(a);
}

static pa_status kv_append(const pa_paged_shape *shape, const void *query, const void *key,
                           const void *value, void *key_cache, void *value_cache,
                           const int32_t *cumulative_sequence_length,
                           const int32_t *past_seqlens, const int32_t *block_table,
                           const int32_t *slot_mapping, const void *cos_cache,
                           const void *sin_cache, int32_t rotary_dim, int32_t rotary_mode,
                           int32_t rotary_positions, void *q_out, void *stream) {
    AppendArgs a;
    pa_status st = make_append(shape, query, key, value, key_cache, value_cache,
                               cumulative_sequence_length, past_seqlens, block_table,
                               slot_mapping, cos_cache, sin_cache, rotary_dim, rotary_mode,
                               rotary_positions, q_out, a);
    if (st != PA_OK || shape->num_tokens == 0) return st;
    return launch_kv_append(a, (hipStream_t)stream);
}

pa_status pa_kv_append(const pa_paged_shape *shape, const void *query, const void *key,
                       const void *value, void *key_cache, void *value_cache,
                       const int32_t *cumulative_sequence_length, const int32_t *past_seqlens,
                       const int32_t *block_table, const int32_t *slot_mapping,
                       const void *cos_cache, const void *sin_cache, int32_t rotary_dim,
                       int32_t rotary_mode, int32_t rotary_positions, void *stream) {
    return kv_append(shape, query, key, value, key_cache, value_cache,
                     cumulative_sequence_length, past_seqlens, block_table, slot_mapping,
                     cos_cache, sin_cache, rotary_dim, rotary_mode, rotary_positions, nullptr,
                     stream);
}

pa_status pa_kv_append_rotate_query(const pa_paged_shape *shape, const void *query,
                                    const void *key, const void *value, void *key_cache,
                                    void *value_cache, const int32_t *cumulative_sequence_length,
                                    const int32_t *past_seqlens, const int32_t *block_table,
                                    const int32_t *slot_mapping, const void *cos_cache,
                                    const void *sin_cache, int32_t rotary_dim,
                                    int32_t rotary_mode, int32_t rotary_positions, void *q_out,
                                    void *stream) {
    if (!shape) return PA_ERR_NULL;
    if (!query || !q_out) return PA_ERR_NULL;
    if (q_out == query) return PA_ERR_SHAPE;  // rotated rows go to their own buffer
    return kv_append(shape, query, key, value, key_cache, value_cache,
                     cumulative_sequence_length, past_seqlens, block_table, slot_mapping,
                     cos_cache, sin_cache, rotary_dim, rotary_mode, rotary_positions, q_out,
                     stream);
}

size_t pa_paged_attention_workspace_size(const pa_paged_shape *shape, int32_t num_splits) {
    PagedPlan p;
    if (!make_plan(shape, num_splits, p)) return 0;
    return p.total;
}

}  // extern "C"

namespace {

// Everything one attention call launches, prepared and checked before anything is enqueued.
struct AttnCall {
    PlanArgs pl;
    AttnArgs a;
    CombineArgs c;
    int D, ncb_dec, blocks, pblocks, pstatic, cap_comb, comb_groups;
    bool combine, fused;
};

// q_stride: the query row stride in elements. With validate_only the call checks every
// argument except the workspace pointer (its size against workspace_bytes) and fills nothing.
pa_status make_attention(const pa_paged_shape *shape, const void *query, int64_t q_stride,
                         const void *key_cache, const void *value_cache,
                         const int32_t *cumulative_sequence_length, const int32_t *past_seqlens,
                         const int32_t *block_table, float scale, int32_t causal,
                         int32_t num_splits, void *workspace, size_t workspace_bytes,
                         void *output, AttnCall &call, bool validate_only = false) {
    pa_status st = check_shape(shape);
    if (st != PA_OK) return st;
    if (causal != 0 && causal != 1) return PA_ERR_SHAPE;
    if (num_splits < PA_SPLITS_PAGE_RULE) return PA_ERR_SHAPE;
    const pa_paged_shape &s = *shape;
    if (!query || !key_cache || !value_cache || !cumulative_sequence_length || !past_seqlens ||
        !block_table || !output)
        return PA_ERR_NULL;
    PagedPlan p;
    if (!make_plan(shape, num_splits, p)) return PA_ERR_SHAPE;
    const int Gc = s.kv_num_heads;  // cache heads (the layout); p.Gv groups of p.Q query heads
    if (s.num_tokens == 0) return PA_OK;
    if (validate_only) return workspace_bytes < p.total ? PA_ERR_WORKSPACE : PA_OK;
    if (!workspace) return PA_ERR_NULL;
    if (workspace_bytes < p.total || ((uintptr_t)workspace % kAlign) != 0)
        return PA_ERR_WORKSPACE;
    char *ws = (char *)workspace;
    const int H = s.num_heads, G = p.Gv, D = s.head_size;

    PlanArgs &pl = call.pl;
    pl.cu = cumulative_sequence_length;
    pl.past = past_seqlens;
    pl.B = s.batch;
    pl.G = G;
    pl.causal = causal;
    pl.tpi_dec = p.tpi_dec;
    pl.tpi_pre = p.tpi_pre;
    pl.mode = p.mode;
    pl.splits = p.splits;
    pl.slots = p.slots;
    pl.slot_ptr = (int32_t *)(ws + p.off_slot);
    pl.slot_first = (AttnItem *)(ws + p.off_first);
    pl.min_chunk = kSplitMinKeys;
    pl.unit_cap = p.unit_cap;
    pl.cap_dec = p.cap_dec;
    pl.cap_pre = p.cap_pre;
    pl.cap_comb = p.cap_comb;
    pl.hdr = (PlanHeader *)ws;
    pl.dec = (AttnItem *)(ws + p.off_dec);
    pl.pre = (AttnItem *)(ws + p.off_pre);
    pl.comb = (CombItem *)(ws + p.off_comb);

    const double sc = scale > 0.f ? (double)scale : 1.0 / sqrt((double)D);
    AttnArgs &a = call.a;
    a.query = (const half_t *)query;
    a.kc = (const half_t *)key_cache;
    a.vc = (const half_t *)value_cache;
    a.cu = cumulative_sequence_length;
    a.past = past_seqlens;
    a.bt = block_table;
    a.out = (half_t *)output;
    a.o_part = (float *)(ws + p.off_o);
    a.m_part = (float *)(ws + p.off_m);
    a.l_part = (float *)(ws + p.off_l);
    a.q_stride = q_stride;
    a.block_elems = (int64_t)s.block_size * Gc * D;
    a.key_elems = (uint32_t)(Gc * D);
    a.H = H;
    a.G = G;
    a.Q = p.Q;
    a.kv_div = p.kv_div;
    a.bs = s.block_size;
    a.MB = s.max_blocks;
    a.log2bs = log2_pow2_ge8(s.block_size);
    a.causal = causal;
    a.gw = p.gw;
    a.scale_log2 = (float)(sc * 1.4426950408889634);
    const int cus = device_cu_count();

    a.items = pl.dec;
    a.n_items = &pl.hdr->n_dec;
    a.counter = &pl.hdr->next_dec;
    a.tpi = p.tpi_dec;
    if (p.mode == 0) {
        a.slot_ptr = pl.slot_ptr;
        a.slot_first = pl.slot_first;
        call.blocks = p.slots;
    } else {
        a.slot_ptr = nullptr;
        const long long units = (long long)p.cap_dec * (G / p.gw);
        call.blocks = (int)std::min(
            units, p.fused ? (long long)cus
                           : (long long)cus * (D == 256 ? 4 : kWavesPerCu) / p.gw);
    }
    call.D = D;
    call.ncb_dec = p.ncb_dec;
    call.fused = p.fused;
    const long long pre_units = (long long)p.cap_pre * G;
    // persistent prefill workgroups: as many as fit at once (two waves per SIMD); beside the
    // decode, one per CU takes a first unit statically and one more per CU takes units only
    // from the counter (it runs when a decode workgroup leaves)
    call.pblocks = (int)std::min(pre_units, (long long)cus * (D == 256 ? 1 : 2));
    call.pstatic = p.fused ? (int)std::min(pre_units, (long long)cus) : call.pblocks;
    call.cap_comb = p.cap_comb;
    // combine entries are rows of decode-like sequences: at most B * tpi_dec
    call.comb_groups = (int)std::min<long long>(p.cap_comb, (long long)s.batch * p.tpi_dec);
    call.combine = p.unit_cap > 0;
    // The split decode rows are merged by extra workgroups of the prefill launch.
    CombineArgs &c = call.c;
    c.o = a.o_part;
    c.m = a.m_part;
    c.l = a.l_part;
    c.group_ptr = nullptr;
    c.items = pl.comb;
    c.n_items = &pl.hdr->n_comb;
    c.num_groups = 0;
    c.lanes = H;
    c.splits = 0;
    c.D = D;
    c.out_f32 = 0;
    c.out = output;
    return PA_OK;
}

// The decode launch, then the prefill launch (which also merges the split decode rows); the
// planner has run before them on the same stream.
// Fused: one launch runs the decode and the prefill items side by side, then the split decode
// rows are merged by a launch of their own.
pa_status run_attention(const AttnCall &call, int tpi_pre, hipStream_t strm) {
    AttnArgs a = call.a;
    AttnArgs pre = a;
    pre.items = call.pl.pre;
    pre.n_items = &call.pl.hdr->n_pre;
    pre.counter = &call.pl.hdr->next_pre;
    pre.slot_ptr = nullptr;
    pre.slot_first = nullptr;
    pre.tpi = tpi_pre;
    pre.gw = 1;
    if (call.fused) {
        pa_status st = launch_decode_prefill(a, pre, call.D, call.blocks, call.pstatic,
                                             call.pblocks, strm);
        if (st != PA_OK || !call.combine) return st;
        return launch_combine(call.c, call.comb_groups, strm);
    }
    pa_status st = launch_attention(a, call.D, call.ncb_dec, call.blocks, "attn_decode", strm);
    if (st != PA_OK) return st;
    return launch_prefill(pre, call.D, call.pblocks, call.combine ? &call.c : nullptr,
                          call.cap_comb, strm);
}

}  // namespace

extern "C" {

pa_status pa_paged_attention(const pa_paged_shape *shape, const void *query,
                             const void *key_cache, const void *value_cache,
                             const int32_t *cumulative_sequence_length,
                             const int32_t *past_seqlens, const int32_t *block_table, float scale,
                             int32_t causal, int32_t num_splits, void *workspace,
                             size_t workspace_bytes, void *output, void *stream) {
    if (!shape) return PA_ERR_NULL;
    const int64_t H = shape->num_heads, G = shape->kv_num_heads, D = shape->head_size;
    AttnCall call;
    pa_status st = make_attention(shape, query, shape->packed_qkv ? (H + 2 * G) * D : H * D,
                                  key_cache, value_cache, cumulative_sequence_length,
                                  past_seqlens, block_table, scale, causal, num_splits,
                                  workspace, workspace_bytes, output, call);
    if (st != PA_OK || shape->num_tokens == 0) return st;
    hipStream_t strm = (hipStream_t)stream;
    if ((st = launch_plan(call.pl, strm)) != PA_OK) return st;
    return run_attention(call, call.pl.tpi_pre, strm);
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// Scratch of pa_paged_attention_noalloc: one static array per device, never allocated by a
// call. Host code must not pass `scratch` itself to a kernel (in host code the name is only a
// stand-in for the device variable): each device's address comes from hipGetSymbolAddress,
// looked up once per device with that device current, and is kept in g_scratch_ptr.
// ---------------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The current device's scratch address, or nullptr when the lookup fails.
void *scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
    return p;
}
}  // namespace

extern "C" {

pa_status pa_paged_attention_noalloc(const pa_paged_shape *shape, const void *query,
                                     const void *key_cache, const void *value_cache,
                                     const int32_t *cumulative_sequence_length,
                                     const int32_t *past_seqlens, const int32_t *block_table,
                                     float scale, int32_t causal, int32_t num_splits,
                                     void *output, void *stream) {
    if (!shape) return PA_ERR_NULL;
    // every argument, and the shape's scratch size against the array's, is checked before the
    // address lookup (the one HIP call besides the launches)
    AttnCall call;
    const int64_t H = shape->num_heads, G = shape->kv_num_heads, D = shape->head_size;
    const pa_status st = make_attention(
        shape, query, shape->packed_qkv ? (H + 2 * G) * D : H * D, key_cache, value_cache,
        cumulative_sequence_length, past_seqlens, block_table, scale, causal, num_splits,
        nullptr, PA_NOALLOC_SCRATCH_BYTES, output, call, /*validate_only=*/true);
    if (st != PA_OK || shape->num_tokens == 0) return st;
    void *ws = scratch_address();
    if (!ws) return PA_ERR_HIP;
    return pa_paged_attention(shape, query, key_cache, value_cache, cumulative_sequence_length,
                              past_seqlens, block_table, scale, causal, num_splits, ws,
                              PA_NOALLOC_SCRATCH_BYTES, output, stream);
}

pa_status pa_append_attention(const pa_paged_shape *shape, const void *query, const void *key,
                              const void *value, void *key_cache, void *value_cache,
                              const int32_t *cumulative_sequence_length,
                              const int32_t *past_seqlens, const int32_t *block_table,
                              const int32_t *slot_mapping, const void *cos_cache,
                              const void *sin_cache, int32_t rotary_dim, int32_t rotary_mode,
                              int32_t rotary_positions, void *q_out, float scale,
                              int32_t causal, int32_t num_splits, void *workspace,
                              size_t workspace_bytes, void *output, void *stream) {
    if (!shape) return PA_ERR_NULL;
    if (!query) return PA_ERR_NULL;
    if (q_out && q_out == query) return PA_ERR_SHAPE;  // rotated rows go to their own buffer
    AppendArgs ap;
    pa_status st = make_append(shape, query, key, value, key_cache, value_cache,
                               cumulative_sequence_length, past_seqlens, block_table,
                               slot_mapping, cos_cache, sin_cache, rotary_dim, rotary_mode,
                               rotary_positions, q_out, ap);
    if (st != PA_OK) return st;
    const int64_t H = shape->num_heads, G = shape->kv_num_heads, D = shape->head_size;
    // attention reads the rotated rows [T, H*D] when q_out is given, else the query as passed
    const void *q_attn = q_out ? q_out : query;
    const int64_t q_stride = q_out ? H * D : (shape->packed_qkv ? (H + 2 * G) * D : H * D);
    AttnCall call;
    st = make_attention(shape, q_attn, q_stride, key_cache, value_cache,
                        cumulative_sequence_length, past_seqlens, block_table, scale, causal,
                        num_splits, workspace, workspace_bytes, output, call);
    if (st != PA_OK || shape->num_tokens == 0) return st;
    hipStream_t strm = (hipStream_t)stream;
    if ((st = launch_append_plan(ap, call.pl, strm)) != PA_OK) return st;
    return run_attention(call, call.pl.tpi_pre, strm);
}

pa_status pa_check_paged_indices(const pa_paged_shape *shape,
                                 const int32_t *cumulative_sequence_length,
                                 const int32_t *past_seqlens, const int32_t *block_table,
                                 const int32_t *slot_mapping, int32_t rotary_positions,
                                 int32_t *flags, void *stream) {
    if (!shape || !cumulative_sequence_length || !past_seqlens || !flags) return PA_ERR_NULL;
    const pa_status st = check_shape(shape);
    if (st != PA_OK) return st;
    if (rotary_positions < 0) return PA_ERR_SHAPE;
    return launch_check_paged(*shape, cumulative_sequence_length, past_seqlens, block_table,
                              slot_mapping, rotary_positions, flags, (hipStream_t)stream);
}

pa_status pa_split_combine(const float *o_partial, const float *m_partial,
                           const float *l_partial, const int32_t *group_ptr, int32_t num_groups,
                           int32_t lanes, int32_t num_splits, int32_t head_dim, int32_t out_dtype,
                           void *out, void *stream) {
    if (num_groups < 0 || lanes < 1 || head_dim <= 0 || head_dim % 4 != 0 ||
        (out_dtype != PA_F16 && out_dtype != PA_F32))
        return PA_ERR_SHAPE;
    if (!group_ptr && num_splits < 1) return PA_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return PA_ERR_UNSUPPORTED;
    if (num_groups == 0) return PA_OK;
    if (!o_partial || !m_partial || !l_partial || !out) return PA_ERR_NULL;
    CombineArgs c;
    c.o = o_partial;
    c.m = m_partial;
    c.l = l_partial;
    c.group_ptr = group_ptr;
    c.items = nullptr;
    c.n_items = nullptr;
    c.num_groups = num_groups;
    c.lanes = lanes;
    c.splits = num_splits;
    c.D = head_dim;
    c.out_f32 = out_dtype == PA_F32;
    c.out = out;
    return launch_combine(c, num_groups, (hipStream_t)stream);
}

static pa_status check_sparse(const pa_sparse_shape *s) {
    if (!s) return PA_ERR_NULL;
    if (s->num_edges < 0 || s->tq < 0 || s->hkv < 1 || s->qhead < 1 || s->head_dim <= 0 ||
        s->block_size < 1 || s->page_size < 1 || s->block_size % s->page_size != 0 ||
        s->num_pages < 0 || s->max_pages < 1 || s->batch < 1)
        return PA_ERR_SHAPE;
    if (s->head_dim != 64 && s->head_dim != 128 && s->head_dim != 256) return PA_ERR_UNSUPPORTED;
    // the key block's fp16 planes live in LDS: up to 128 keys, 64 at D = 256
    if (s->block_size > (s->head_dim == 256 ? 64 : 128)) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

static int sparse_units(const pa_sparse_shape *s) {
    const long long nblk = s->max_pages / (s->block_size / s->page_size) + 1;
    return (int)std::min((long long)s->batch * s->hkv * nblk, 1LL << 30);
}

size_t pa_sparse_forward_workspace_size(const pa_sparse_shape *shape) {
    if (check_sparse(shape) != PA_OK) return 0;
    return sparse_workspace_bytes(shape->num_edges, sparse_units(shape),
                                  (long long)shape->tq * shape->hkv * shape->qhead,
                                  shape->head_dim);
}

static pa_status sparse_forward(const pa_sparse_shape *shape, const float *q_buf,
                                const float *k_pages, const float *v_pages,
                                const int32_t *edge_meta, const int32_t *block_tables,
                                const int32_t *q_pos, float softmax_scale, void *workspace,
                                size_t workspace_bytes, float *o_partial, float *m_partial,
                                float *l_partial, void *stream) {
    pa_status st = check_sparse(shape);
    if (st != PA_OK) return st;
    const pa_sparse_shape &s = *shape;
    if (s.num_edges == 0) return PA_OK;
    if (!q_buf || !k_pages || !v_pages || !edge_meta || !block_tables || !o_partial ||
        !m_partial || !l_partial || !workspace)
        return PA_ERR_NULL;
    const int units = sparse_units(shape);
    if (workspace_bytes < sparse_workspace_bytes(s.num_edges, units,
                                                 (long long)s.tq * s.hkv * s.qhead, s.head_dim) ||
        ((uintptr_t)workspace % 256) != 0)
        return PA_ERR_WORKSPACE;
    SparseArgs a;
    a.q = q_buf;
    a.kp = k_pages;
    a.vp = v_pages;
    a.edge_meta = edge_meta;
    a.bt = block_tables;
    a.q_pos = q_pos;
    a.o = o_partial;
    a.m = m_partial;
    a.l = l_partial;
    a.ws = (int32_t *)workspace;
    a.E = s.num_edges;
    a.tq = s.tq;
    a.hkv = s.hkv;
    a.qhead = s.qhead;
    a.D = s.head_dim;
    a.block_size = s.block_size;
    a.page_size = s.page_size;
    a.ppb = s.block_size / s.page_size;
    a.max_pages = s.max_pages;
    a.batch = s.batch;
    a.num_pages = s.num_pages;
    a.units = units;
    a.nblk = units / (s.batch * s.hkv);
    a.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);
    return launch_sparse(a, (hipStream_t)stream);
}

pa_status pa_sparse_forward(const pa_sparse_shape *shape, const float *q_buf,
                            const float *k_pages, const float *v_pages,
                            const int32_t *edge_meta, const int32_t *block_tables,
                            float softmax_scale, int32_t causal, void *workspace,
                            size_t workspace_bytes, float *o_partial, float *m_partial,
                            float *l_partial, void *stream) {
    pa_status st = check_sparse(shape);
    if (st != PA_OK) return st;
    if (causal != 0) return PA_ERR_UNSUPPORTED;  // the mask needs positions: the causal entry
    return sparse_forward(shape, q_buf, k_pages, v_pages, edge_meta, block_tables, nullptr,
                          softmax_scale, workspace, workspace_bytes, o_partial, m_partial,
                          l_partial, stream);
}

pa_status pa_sparse_forward_causal(const pa_sparse_shape *shape, const float *q_buf,
                                   const float *k_pages, const float *v_pages,
                                   const int32_t *edge_meta, const int32_t *block_tables,
                                   const int32_t *q_pos, float softmax_scale, void *workspace,
                                   size_t workspace_bytes, float *o_partial, float *m_partial,
                                   float *l_partial, void *stream) {
    pa_status st = check_sparse(shape);
    if (st != PA_OK) return st;
    if (shape->num_edges > 0 && !q_pos) return PA_ERR_NULL;
    return sparse_forward(shape, q_buf, k_pages, v_pages, edge_meta, block_tables, q_pos,
                          softmax_scale, workspace, workspace_bytes, o_partial, m_partial,
                          l_partial, stream);
}

pa_status pa_kv_append_bnsh(const pa_bnsh_shape *shape, const void *query, const void *key,
                            const void *value, void *present_key, void *present_value,
                            const int32_t *total_sequence_length,
                            const int32_t *key_total_sequence_lengths, const void *cos_cache,
                            const void *sin_cache, int32_t rotary_dim, int32_t rotary_mode,
                            int32_t rotary_positions, void *stream) {
    if (!shape) return PA_ERR_NULL;
    const pa_bnsh_shape &s = *shape;
    if (s.batch < 1 || s.seq_len < 0 || s.num_heads <= 0 || s.kv_num_heads <= 0 ||
        s.num_heads % s.kv_num_heads != 0 || s.head_size <= 0 || s.max_cache_seq < 1 ||
        (s.packed_qkv != 0 && s.packed_qkv != 1))
        return PA_ERR_SHAPE;
    if (s.head_size != 64 && s.head_size != 128 && s.head_size != 256) return PA_ERR_UNSUPPORTED;
    if (s.packed_qkv) {
        if (key || value) return PA_ERR_SHAPE;
        if (!query) return PA_ERR_NULL;
    } else {
        if ((key == nullptr) != (value == nullptr)) return PA_ERR_SHAPE;
        if (!key) return PA_ERR_NULL;
    }
    if (rotary_mode != PA_ROTARY_NONE && rotary_mode != PA_ROTARY_NEOX &&
        rotary_mode != PA_ROTARY_INTERLEAVED)
        return PA_ERR_SHAPE;
    if (rotary_mode != PA_ROTARY_NONE) {
        if (rotary_dim <= 0 || rotary_dim % 2 != 0 || rotary_dim > s.head_size ||
            rotary_positions < 1)
            return PA_ERR_SHAPE;
        if (!cos_cache || !sin_cache) return PA_ERR_NULL;
    }
    if (s.seq_len == 0) return PA_OK;
    if (!present_key || !present_value || !total_sequence_length || !key_total_sequence_lengths)
        return PA_ERR_NULL;
    const int H = s.num_heads, G = s.kv_num_heads, D = s.head_size;
    BnshArgs a;
    a.query = s.packed_qkv ? (const half_t *)query : nullptr;
    a.key = (const half_t *)key;
    a.value = (const half_t *)value;
    a.pk = (half_t *)present_key;
    a.pv = (half_t *)present_value;
    a.total_seq = total_sequence_length;
    a.key_total = key_total_sequence_lengths;
    a.cos = (const half_t *)cos_cache;
    a.sin = (const half_t *)sin_cache;
    a.src_stride = s.packed_qkv ? (int64_t)(H + 2 * G) * D : (int64_t)G * D;
    a.k_off = s.packed_qkv ? (int64_t)H * D : 0;
    a.v_off = s.packed_qkv ? (int64_t)(H + G) * D : 0;
    a.B = s.batch;
    a.S = s.seq_len;
    a.H = H;
    a.KVH = G;
    a.D = D;
    a.max_seq = s.max_cache_seq;
    a.rotary_dim = rotary_mode == PA_ROTARY_NONE ? 0 : rotary_dim;
    a.rotary_mode = rotary_mode;
    a.rotary_positions = rotary_mode == PA_ROTARY_NONE ? 0 : rotary_positions;
    return launch_kv_append_bnsh(a, (hipStream_t)stream);
}

size_t pa_sparse_build_edges_workspace_size(int32_t tq, int32_t hkv) {
    if (tq < 0 || hkv < 1) return 0;
    return std::max<size_t>(256, edge_workspace_bytes((long long)tq * hkv));
}

pa_status pa_sparse_build_edges(int32_t tq, int32_t hkv, int32_t nblk, int32_t block_size,
                                int32_t batch, const uint8_t *block_mask,
                                const int32_t *q_batch, const int32_t *used_kv_lens,
                                int64_t edge_capacity, int32_t *edge_meta, int32_t *group_ptr,
                                void *workspace, size_t workspace_bytes, void *stream) {
    if (tq < 0 || hkv < 1 || nblk < 1 || block_size < 1 || batch < 1 || edge_capacity < 0)
        return PA_ERR_SHAPE;
    const long long rows = (long long)tq * hkv;
    if (rows * nblk >= (1LL << 31)) return PA_ERR_UNSUPPORTED;  // int32 edge offsets
    if (!group_ptr || !workspace) return PA_ERR_NULL;
    if (rows > 0 && (!block_mask || !q_batch || !used_kv_lens)) return PA_ERR_NULL;
    if (edge_capacity > 0 && !edge_meta) return PA_ERR_NULL;
    if (workspace_bytes < pa_sparse_build_edges_workspace_size(tq, hkv) ||
        ((uintptr_t)workspace % 256) != 0)
        return PA_ERR_WORKSPACE;
    EdgeArgs a;
    a.mask = block_mask;
    a.q_batch = q_batch;
    a.used = used_kv_lens;
    a.edge_meta = edge_meta;
    a.group_ptr = group_ptr;
    a.wg = (int32_t *)workspace;
    a.rows = rows;
    a.capacity = edge_capacity;
    a.hkv = hkv;
    a.nblk = nblk;
    a.block_size = block_size;
    a.batch = batch;
    return launch_build_edges(a, (hipStream_t)stream);
}

}  // extern "C"
