// Internal helpers shared by the HIP kernels and the host entry points of libpa.
// gfx950 (CDNA4) only: wave64, MFMA f32_16x16x32_f16 / f32_16x16x4_f32.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t int4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegLarge = -1.0e30f;  // the sentinel max of an empty partial

// ---------------------------------------------------------------------------------------------
// Host side: launch bookkeeping (timing hooks) and device properties.
// ---------------------------------------------------------------------------------------------
// Launch helper. When timing is enabled (pa_timing_enable), the first kernel launched through a
// scope carries the start event and the last one the stop event, recorded by the dispatch
// itself (hipExtLaunchKernelGGL), so the interval covers exactly the scope's kernels.
struct LaunchScope {
    LaunchScope(const char *name, hipStream_t stream, int launches = 1);
    ~LaunchScope();
    template <class F, class... Args>
    void launch(F kernel, dim3 grid, dim3 block, uint32_t shmem, Args... args) {
        hipEvent_t s = (idx_ == 0) ? start_ : nullptr;
        hipEvent_t e = (idx_ == n_ - 1) ? stop_ : nullptr;
        ++idx_;
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream_, s, e, 0, args...);
    }
    const char *name_;
    hipStream_t stream_;
    hipEvent_t start_, stop_;
    int n_, idx_;
};

int device_cu_count();  // compute units of the current device (cached per device)

// ---------------------------------------------------------------------------------------------
// Launchers (one per kernel family); each returns PA_OK or PA_ERR_HIP.
// ---------------------------------------------------------------------------------------------
struct AppendArgs {
    const half_t *query;  // packed rows, or NULL
    const half_t *key;
    const half_t *value;
    half_t *kc;
    half_t *vc;
    const int32_t *cu;
    const int32_t *past;
    const int32_t *bt;
    const int32_t *slot_mapping;
    const half_t *cos;
    const half_t *sin;
    int64_t src_stride;  // elements per source row (G*D or (H+2G)*D)
    int64_t k_off;       // element offset of K inside a source row
    int64_t v_off;       // element offset of V inside a source row
    int T, B, G, D, bs, MB;
    int rotary_dim, rotary_mode;
    half_t *q_out;       // rotated query rows [T, H*D], or NULL: no query rotation
    const half_t *q_src; // query rows to rotate (packed rows, or separate [T, H*D])
    int64_t q_stride;    // elements per query source row (H*D or (H+2G)*D)
    int H;
    int nkv, nkv_pad, nq;  // threads for key/value rows, padded to whole workgroups; query rows
};
pa_status launch_kv_append(const AppendArgs &a, hipStream_t stream);

// Append into a contiguous BNSH cache [B, KVH, max_seq, D] (the append page's own layout).
struct BnshArgs {
    const half_t *query;  // packed rows, or NULL
    const half_t *key;
    const half_t *value;
    half_t *pk;
    half_t *pv;
    const int32_t *total_seq;  // [1]: scalar total_sequence_length
    const int32_t *key_total;  // [B]: per-batch totals
    const half_t *cos;
    const half_t *sin;
    int64_t src_stride;  // elements per source row
    int64_t k_off, v_off;
    int B, S, H, KVH, D, max_seq;
    int rotary_dim, rotary_mode, rotary_positions;
};
pa_status launch_kv_append_bnsh(const BnshArgs &a, hipStream_t stream);

// Work item of the attention kernels, written by the device planner.
struct AttnItem {
    int32_t b;     // sequence
    int32_t t0;    // first new token of the item, within the sequence
    int32_t k0;    // key range [k0, k1) this item covers
    int32_t k1;
    int32_t base;  // first partial unit of the sequence, or -1: write the output directly
    int32_t nsplit;  // chunks the sequence's key range is cut into
    int32_t split;   // this item's chunk
    int32_t cu0;     // the sequence's first query row (cumulative_sequence_length[b])
    int32_t n;       // the sequence's new tokens
    int32_t past;    // the sequence's past length (past_seqlens[b])
};

// Combine work entry for one output row group (a query row with >= 2 partial units).
struct CombItem {
    int32_t row;    // output row group
    int32_t e0;     // first partial unit
    int32_t count;  // units
    int32_t pad;
};

// Header of the planner's output inside the workspace.
struct PlanHeader {
    int32_t n_dec;      // decode-like items
    int32_t n_pre;      // prefill items
    int32_t n_comb;     // combine entries
    int32_t chunk;      // chunk keys chosen for split decode (0 when no split)
    int32_t units;      // partial units used
    int32_t next_dec;   // dynamic scheduling counters, zeroed by the planner
    int32_t next_pre;
    int32_t pad[57];    // keeps the lists 256-byte aligned
};

struct PlanArgs {
    const int32_t *cu;
    const int32_t *past;
    int B, G, causal;
    int tpi_dec;        // max tokens of a decode-like item
    int tpi_pre;        // tokens per prefill item
    int mode;           // 0: stream-K shares over `slots`, 1: even split into `splits`
    int splits;         // S for mode 1
    int min_chunk;      // mode 0: smallest chunk
    int unit_cap;       // partial units that fit the workspace
    int cap_dec, cap_pre, cap_comb;
    int slots;          // mode 0: decode workgroups, one key-range share each
    int32_t *slot_ptr;  // mode 0: [slots + 1] first item of each share
    AttnItem *slot_first;  // mode 0: [slots] a copy of the first item of each share
    PlanHeader *hdr;
    AttnItem *dec;
    AttnItem *pre;
    CombItem *comb;
};
pa_status launch_plan(const PlanArgs &a, hipStream_t stream);
// The key/value append and the planner in one launch (workgroup 0 plans, the rest append).
pa_status launch_append_plan(const AppendArgs &a, const PlanArgs &p, hipStream_t stream);
// The checks of launch_kv_append that depend on the launch size, without launching.
pa_status check_kv_append(const AppendArgs &a);

struct AttnArgs {
    const half_t *query;
    const half_t *kc;
    const half_t *vc;
    const int32_t *cu;
    const int32_t *past;
    const int32_t *bt;
    const AttnItem *items;
    const int32_t *n_items;  // device count of items
    int32_t *counter;        // dynamic scheduling counter (zeroed by the planner)
    const int32_t *slot_ptr; // stream-K share table [gridDim.x + 1], or NULL for dynamic
    const AttnItem *slot_first;  // with slot_ptr: [gridDim.x] first item of each share
    half_t *out;
    float *o_part;
    float *m_part;
    float *l_part;
    int64_t q_stride;     // elements per query row
    int64_t block_elems;  // elements per cache block: bs * G * D
    uint32_t key_elems;   // elements between consecutive keys of a block: G * D
    int H, G, Q, bs, MB, log2bs;  // log2bs < 0: block size is not a power of two >= 8
    // G counts kv head groups of Q query heads; kv_div groups share one cache head (group g
    // reads cache head g / kv_div), so a kv head with more query heads than one wave serves is
    // split into kv_div groups of Q = H / (G_cache * kv_div) heads each
    int kv_div;
    int causal;
    int gw;            // waves per workgroup, a divisor of G
    int tpi;           // tokens per item
    float scale_log2;  // scale * log2(e)
};
// Decode items. ncb: 16-column blocks of (token, head) columns per item (1, 2 or 4); blocks:
// workgroups of a.gw waves.
pa_status launch_attention(const AttnArgs &a, int D, int ncb, int blocks, const char *name,
                           hipStream_t stream);
// Prefill items (a.tpi = kPrefillCols / Q tokens each) on workgroups of kPrefillCols / 32 waves, one per
// (item, kv head) taken from the planner's counter.
constexpr int kPrefillCols = 128;  // (token, head) columns per prefill item: 4 waves of 32
// cmb (may be NULL): planner-list combine of the split decode partials (max_groups list
// entries), run by extra workgroups of the same launch.
struct CombineArgs;
pa_status launch_prefill(const AttnArgs &a, int D, int blocks, const CombineArgs *cmb,
                         int max_groups, hipStream_t stream);
// Decode items (dec, workgroups of kPrefillCols / 32 waves: dec.gw must equal that) and prefill
// items (pre) in one launch: dec_blocks decode workgroups first, then pre_blocks prefill
// workgroups, the first pre_static of which take their first unit statically.
pa_status launch_decode_prefill(const AttnArgs &dec, const AttnArgs &pre, int D, int dec_blocks,
                                int pre_static, int pre_blocks, hipStream_t stream);

struct CombineArgs {
    const float *o;
    const float *m;
    const float *l;
    const int32_t *group_ptr;     // CSR mode
    const CombItem *items;        // list mode
    const int32_t *n_items;       // list mode: device count
    int num_groups;               // CSR / uniform modes
    int lanes, splits, D;
    int out_f32;
    void *out;
};
pa_status launch_combine(const CombineArgs &a, int max_groups, hipStream_t stream);

struct SparseArgs {
    const float *q;
    const float *kp;
    const float *vp;
    const int32_t *edge_meta;
    const int32_t *bt;
    float *o;
    float *m;
    float *l;
    const int32_t *q_pos;  // key position of each query row (causal limit), or NULL
    int32_t *ws;  // workspace (int32 words)
    int E, tq, hkv, qhead, D, block_size, page_size, ppb, max_pages, batch, num_pages;
    int units;    // batch * hkv * nblk
    int nblk;     // blocks per batch row (max_pages / ppb)
    float scale_log2;
};
pa_status launch_sparse(const SparseArgs &a, hipStream_t stream);

// Edge list of the block-sparse forward from a kept-block mask.
struct EdgeArgs {
    const uint8_t *mask;     // [tq, hkv, nblk], nonzero = keep
    const int32_t *q_batch;  // [tq]
    const int32_t *used;     // used_kv_lens [batch]
    int32_t *edge_meta;      // [capacity, 5]
    int32_t *group_ptr;      // [tq * hkv + 1]
    int32_t *wg;             // workspace: per-workgroup totals, then offsets
    long long rows;          // tq * hkv
    long long capacity;      // edges edge_meta can hold
    int hkv, nblk, block_size, batch;
};
pa_status launch_build_edges(const EdgeArgs &a, hipStream_t stream);
size_t edge_workspace_bytes(long long rows);
pa_status launch_check_paged(const pa_paged_shape &s, const int32_t *cu, const int32_t *past,
                             const int32_t *bt, const int32_t *slot, int32_t rotary_positions,
                             int32_t *flags, hipStream_t stream);
size_t sparse_workspace_bytes(int E, int units, long long qrows, int D);

// ---------------------------------------------------------------------------------------------
// Device helpers.
// ---------------------------------------------------------------------------------------------
// Load through a global (address space 1) pointer, so the access is a global_load rather than
// a flat load that must also check the LDS and scratch apertures.
template <class T>
__device__ __forceinline__ T gload(const void *p) {
    return *(const __attribute__((address_space(1))) T *)p;
}

// Streaming (non-temporal) global load, for data read once: K/V cache rows.
template <class T>
__device__ __forceinline__ T gload_nt(const void *p) {
    return __builtin_nontemporal_load((const __attribute__((address_space(1))) T *)p);
}

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
    return fmaxf(v, __shfl_xor(v, mask, 64));
}

__device__ __forceinline__ float4_t mfma16x16x32(half8_t a, half8_t b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float4_t mfma16x16x4f32(float a, float b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace pa
