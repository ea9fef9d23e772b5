// Fused KV append (rotary + scatter into paged cache slots) for gfx950.
//
// Operation: pass "scatter" (PagedAttention.ScatterKV) of the "com.microsoft.PagedAttention ...
// manifest.json" page, fused with the key rotation of the "com.microsoft.SparseAttention ...
// sparse-kv-append.wgsl.jinja" page (rotary macros and main): each new key row is rotated at its
// absolute position, then key and value rows are written to their cache slot; nothing else is
// written.
//
// One thread moves the 16-byte chunks d and d + D/2 of one (token, kv head) row of K and of V.
// With NeoX rotary over the whole row these two chunks are each other's rotation partners and
// share one cos/sin chunk, so nothing is loaded twice. The G rows of a token form one
// contiguous span of the cache.
//
// Token -> sequence: all loads that do not depend on the sequence go out first (source rows, and
// cumulative_sequence_length / past_seqlens held one entry per lane when the batch has at most
// 256 sequences). When a wave's lanes share one token, a ballot over the lanes' cu entries
// counts the sequences that start at or before it, and the sequence's cu and past entries come
// from lane shuffles: no LDS, no barrier, no dependent load. Other waves search the same entries
// lane by lane; batches above 256 sequences search cu staged in LDS (or in global memory).
// Then the slot (slot_mapping, or the block table) and the cos/sin row are loaded.
//
// Rotary arithmetic is the page's float32 expression with contraction disabled: two rounded
// products, one rounded add or subtract, then round-to-nearest-even to fp16.
//
// append_plan_kernel runs the same append beside the paged-attention planner (plan.h): the
// planner reads only the sequence lengths, which the append does not change, so the two share
// one launch when a caller asks for the append and the attention in one call.
#include "common.h"
#include "plan.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsCu = 2048;  // large batches: cumulative lengths staged in LDS up to this many
constexpr int kLaneCu = 4;    // small batches: up to 4 x 64 cu entries held in lanes

enum { kCopy = 0, kNeoxFull = 1, kNeox = 2, kInter = 3, kGeneric = 4 };

__device__ __forceinline__ int find_batch(const int32_t *cu, int B, int i) {
    // largest b with cu[b] <= i (sequences with no tokens are skipped over)
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return lo;
}

#pragma clang fp contract(off)
__device__ __forceinline__ float rot_f32(float own, float partner, float cs, float sn,
                                         bool first) {
    const float x = own * cs;
    const float y = partner * sn;
    return first ? x - y : x + y;
}

// Rotate one 16-byte chunk at dims d0 .. d0+7 (MODE kNeox / kNeoxFull / kInter / kGeneric).
template <int MODE, typename Args>
__device__ __forceinline__ half8_t rotate_chunk(const Args &a, const half_t *ks, half8_t kv,
                                                half8_t pk, half8_t cs, half8_t sn, int d0,
                                                int pos) {
    const int R = a.rotary_dim, half = R >> 1;
    half8_t out = kv;
    if (MODE == kNeox || MODE == kNeoxFull) {
        if (d0 < R) {
            const bool first = d0 < half;
            for (int e = 0; e < 8; ++e)
                out[e] = (half_t)rot_f32((float)kv[e], (float)pk[e], (float)cs[e], (float)sn[e],
                                         first);
        }
    } else if (MODE == kInter) {
        if (d0 < R)  // R % 8 == 0: the chunk holds 4 whole pairs; cs/sn lanes 0..3 are its columns
            for (int e = 0; e < 8; e += 2) {
                const float c = (float)cs[e >> 1], sv = (float)sn[e >> 1];
                out[e] = (half_t)rot_f32((float)kv[e], (float)kv[e + 1], c, sv, true);
                out[e + 1] = (half_t)rot_f32((float)kv[e + 1], (float)kv[e], c, sv, false);
            }
    } else if (MODE == kGeneric) {
        for (int e = 0; e < 8; ++e) {
            const int d = d0 + e;
            if (d >= R) break;
            int col, partner;
            bool fst;
            if (a.rotary_mode == PA_ROTARY_INTERLEAVED) {
                col = d >> 1; fst = (d & 1) == 0; partner = fst ? d + 1 : d - 1;
            } else {
                fst = d < half; col = fst ? d : d - half; partner = fst ? d + half : d - half;
            }
            const long long c0 = (long long)pos * half + col;
            out[e] = (half_t)rot_f32((float)kv[e], (float)ks[partner], (float)a.cos[c0],
                                     (float)a.sin[c0], fst);
        }
    }
    return out;
}

// cos/sin chunk for dims d0 .. d0+7 at pos (NeoX: 8 columns; interleaved: 4 columns). Chunks
// past the rotary dims load column 0 of the row instead (unused), so the loads are unconditional.
template <int MODE, typename Args>
__device__ __forceinline__ void load_cs(const Args &a, int d0, int pos, half8_t &cs,
                                        half8_t &sn) {
    const int R = a.rotary_dim, half = R >> 1;
    cs = half8_t{};
    sn = half8_t{};
    if (MODE == kNeox || MODE == kNeoxFull) {  // half % 8 == 0: aligned chunk of columns
        const int col = d0 >= R ? 0 : (d0 < half ? d0 : d0 - half);
        const long long c0 = (long long)pos * half + col;
        cs = gload<half8_t>(a.cos + c0);
        sn = gload<half8_t>(a.sin + c0);
    } else if (MODE == kInter) {
        const long long c0 = (long long)pos * half + (d0 >= R ? 0 : (d0 >> 1));
        const half4_t c4 = gload<half4_t>(a.cos + c0), s4 = gload<half4_t>(a.sin + c0);
        for (int e = 0; e < 4; ++e) { cs[e] = c4[e]; sn[e] = s4[e]; }
    }
}

// One row's two chunks: source data, then its destination.
struct RowIn {
    half8_t kA, kB, vA, vB, pA, pB;
};
struct RowAt {
    int pos;
    int32_t sv;  // slot_mapping entry, or the block id of pos (key/value rows)
    half8_t cA, sA, cB, sB;
};

template <int MODE, bool QROLE>
__device__ __forceinline__ RowIn load_row(const AppendArgs &a, const half_t *ks,
                                          const half_t *vs, int dA, int dB) {
    RowIn r;
    // source rows are read once: non-temporal (the 554 MB append reads and writes 23% faster)
    r.kA = gload_nt<half8_t>(ks + dA);
    r.kB = gload_nt<half8_t>(ks + dB);
    if (!QROLE) {
        r.vA = gload_nt<half8_t>(vs + dA);
        r.vB = gload_nt<half8_t>(vs + dB);
    }
    r.pA = r.kB;  // kNeoxFull: the chunks are each other's partners
    r.pB = r.kA;
    if (MODE == kNeox) {  // partners of chunks past the rotary dims: chunk 0 (unused)
        const int R = a.rotary_dim, half = R >> 1;
        r.pA = gload<half8_t>(ks + (dA >= R ? 0 : (dA < half ? dA + half : dA - half)));
        r.pB = gload<half8_t>(ks + (dB >= R ? 0 : (dB < half ? dB + half : dB - half)));
    }
    return r;
}

// Sequence b of token i, its first token cu[b] and past_seqlens[b], from the cu / past
// entries held by the wave's lanes (entry 64 c + lane in cuv[c], pav[c]).
__device__ __forceinline__ void lane_lookup(const AppendArgs &a, const int (&cuv)[kLaneCu],
                                            const int (&pav)[kLaneCu], int i, int &b, int &cb,
                                            int &pb) {
    const int i0 = __builtin_amdgcn_readfirstlane(i);
    int cnt = 0;
    if (__ballot(i != i0) == 0) {
        // one token per wave: b + 1 = number of entries cu[k] <= i (cu[B] = T > i)
        for (int c = 0; c < kLaneCu; ++c) cnt += __popcll(__ballot(cuv[c] <= i0));
    } else {
        // several tokens in the wave: count entry by entry
        for (int q = 0; q < kLaneCu; ++q)
            for (int l = 0; l < 64 && 64 * q + l <= a.B; ++l) cnt += __shfl(cuv[q], l, 64) <= i;
    }
    b = min(cnt, a.B) - 1;
    const int c = b >> 6, l = b & 63;
    cb = 0;
    pb = 0;
    for (int q = 0; q < kLaneCu; ++q) {
        const int x = __shfl(cuv[q], l, 64), y = __shfl(pav[q], l, 64);
        if (q == c) { cb = x; pb = y; }
    }
}

// Position of the token; for key/value rows one load of its slot_mapping entry or block id;
// the cos/sin chunks.
template <int MODE, bool QROLE>
__device__ __forceinline__ RowAt locate(const AppendArgs &a, int i, int b, int t, int past,
                                        int dA, int dB) {
    RowAt w;
    w.pos = past + t;
    w.sv = 0;
    if (!QROLE) {
        const int32_t *sp = a.slot_mapping ? a.slot_mapping + i
                                           : a.bt + (long long)b * a.MB + w.pos / a.bs;
        w.sv = *sp;
    }
    if (MODE != kCopy && MODE != kGeneric) {
        load_cs<MODE>(a, dA, w.pos, w.cA, w.sA);
        if (MODE == kNeoxFull) {  // dB = dA + R/2 uses the same columns
            w.cB = w.cA;
            w.sB = w.sA;
        } else {
            load_cs<MODE>(a, dB, w.pos, w.cB, w.sB);
        }
    }
    return w;
}

// Rotate K (or Q) and write: key/value rows to their cache slot, query rows to q_out.
template <int MODE, bool QROLE>
__device__ __forceinline__ void store_row(const AppendArgs &a, const half_t *ks, const RowIn &r,
                                          const RowAt &w, int i, int g, int dA, int dB) {
    half8_t oA = r.kA, oB = r.kB;
    if (MODE != kCopy) {
        oA = rotate_chunk<MODE>(a, ks, r.kA, r.pA, w.cA, w.sA, dA, w.pos);
        oB = rotate_chunk<MODE>(a, ks, r.kB, r.pB, w.cB, w.sB, dB, w.pos);
    }
    if (QROLE) {  // query rows: only launched with q_out and q_src set
        half_t *qd = a.q_out + ((long long)i * a.H + g) * a.D;
        *(half8_t *)(qd + dA) = oA;
        *(half8_t *)(qd + dB) = oB;
        return;
    }
    const long long slot =
        a.slot_mapping ? (long long)w.sv : (long long)w.sv * a.bs + (w.pos % a.bs);
    if (slot < 0) return;
    const long long dst = (slot * a.G + g) * a.D;
    *(half8_t *)(a.kc + dst + dA) = oA;
    *(half8_t *)(a.kc + dst + dB) = oB;
    *(half8_t *)(a.vc + dst + dA) = r.vA;
    *(half8_t *)(a.vc + dst + dB) = r.vB;
}

// Thread gid < n takes chunk pair j of head g (a kv head, or a query head when QROLE) for the
// two tokens 2p and 2p + 1. Token 2p + 1's rows are requested after token 2p's slot and
// cos/sin, so token 2p's stores do not wait for them. LANECU: at most kLaneCu * 64 cu entries,
// held in lanes; otherwise cu is searched in LDS (whole workgroups take one role, so the
// barrier is uniform) or in global memory.
template <int MODE, bool LANECU, bool QROLE>
__device__ __forceinline__ void append_pairs(const AppendArgs &a, int gid, int n,
                                             int32_t *s_cu, int32_t *s_past) {
    const int lhc = a.D == 256 ? 4 : (a.D == 128 ? 3 : 2);  // log2 of chunk pairs per row
    const int rows = QROLE ? a.H : a.G;  // head rows per token
    const int gidc = gid < n ? gid : n - 1;
    const int j = gidc & ((1 << lhc) - 1);
    const int rg = gidc >> lhc;
    const int p = (int)((unsigned)rg / (unsigned)rows);
    const int g = rg - p * rows;
    const int i0 = 2 * p, i1 = min(2 * p + 1, a.T - 1);
    const bool live0 = gid < n, live1 = live0 && 2 * p + 1 < a.T;
    const int dA = j << 3, dB = dA + (a.D >> 1);
    const int lane = threadIdx.x & 63;
    const half_t *src_k = QROLE ? a.q_src : (a.query ? a.query : a.key);
    const half_t *src_v = a.query ? a.query : a.value;
    const long long stride = QROLE ? a.q_stride : a.src_stride;
    const long long off_k = (QROLE ? 0 : a.k_off) + (long long)g * a.D;
    const long long off_v = a.v_off + (long long)g * a.D;
    const half_t *ks0 = src_k + (long long)i0 * stride + off_k;
    const half_t *ks1 = src_k + (long long)i1 * stride + off_k;
    const half_t *vs0 = QROLE ? nullptr : src_v + (long long)i0 * stride + off_v;
    const half_t *vs1 = QROLE ? nullptr : src_v + (long long)i1 * stride + off_v;

    // cu / past entries first (clamped, unconditional), then token 2p's rows: waiting for the
    // entries leaves the rows in flight
    int cuv[kLaneCu], pav[kLaneCu];
    if (LANECU)
        for (int c = 0; c < kLaneCu; ++c) {
            const int k = 64 * c + lane;
            cuv[c] = a.cu[min(k, a.B)];
            pav[c] = a.past[min(k, a.B - 1)];
        }
    const RowIn r0 = load_row<MODE, QROLE>(a, ks0, vs0, dA, dB);
    int b0, b1, cb0, cb1, pb0, pb1;
    if (LANECU) {
        for (int c = 0; c < kLaneCu; ++c)
            if (64 * c + lane > a.B) cuv[c] = 0x7fffffff;  // entries past cu[B] never count
        lane_lookup(a, cuv, pav, i0, b0, cb0, pb0);
        lane_lookup(a, cuv, pav, i1, b1, cb1, pb1);
    } else {
        const bool lds = a.B + 1 <= kLdsCu;  // uniform over the grid
        if (lds) {
            for (int k = threadIdx.x; k <= a.B; k += kThreads) {
                s_cu[k] = a.cu[k];
                if (k < a.B) s_past[k] = a.past[k];
            }
            __syncthreads();
        }
        const int32_t *cu = lds ? s_cu : a.cu;
        const int32_t *pa = lds ? s_past : a.past;
        b0 = find_batch(cu, a.B, i0);
        b1 = find_batch(cu, a.B, i1);
        cb0 = cu[b0]; pb0 = pa[b0];
        cb1 = cu[b1]; pb1 = pa[b1];
    }
    const RowAt w0 = locate<MODE, QROLE>(a, i0, b0, i0 - cb0, pb0, dA, dB);
    const RowIn r1 = load_row<MODE, QROLE>(a, ks1, vs1, dA, dB);
    const RowAt w1 = locate<MODE, QROLE>(a, i1, b1, i1 - cb1, pb1, dA, dB);
    if (live0) store_row<MODE, QROLE>(a, ks0, r0, w0, i0, g, dA, dB);
    if (live1) store_row<MODE, QROLE>(a, ks1, r1, w1, i1, g, dA, dB);
}

// Workgroups [0, nkv_pad / kThreads) append key/value rows; the rest (when q_out is given)
// rotate query rows.
template <int MODE, bool LANECU>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
    __shared__ int32_t s_cu[LANECU ? 1 : kLdsCu];
    __shared__ int32_t s_past[LANECU ? 1 : kLdsCu];
    const int gid = blockIdx.x * kThreads + threadIdx.x;
    if (gid < a.nkv_pad)
        append_pairs<MODE, LANECU, false>(a, gid, a.nkv, s_cu, s_past);
    else
        append_pairs<MODE, LANECU, true>(a, gid - a.nkv_pad, a.nq, s_cu, s_past);
}

// Workgroup 0 runs the planner (on its first PTH threads; the other waves exit at once); the
// rest run append_kernel's roles with workgroup indexes shifted by one.
template <int MODE, bool LANECU, int PTH>
__global__ __launch_bounds__(kThreads) void append_plan_kernel(AppendArgs a, PlanArgs p) {
    __shared__ int32_t s_cu[LANECU ? 1 : kLdsCu];
    __shared__ int32_t s_past[LANECU ? 1 : kLdsCu];
    if (blockIdx.x == 0) {
        if ((int)threadIdx.x >= PTH) return;  // whole waves: PTH is a multiple of 64
        plan_body<PTH>(p);
        return;
    }
    const int gid = (blockIdx.x - 1) * kThreads + threadIdx.x;
    if (gid < a.nkv_pad)
        append_pairs<MODE, LANECU, false>(a, gid, a.nkv, s_cu, s_past);
    else
        append_pairs<MODE, LANECU, true>(a, gid - a.nkv_pad, a.nq, s_cu, s_past);
}

// The append page's own pass over a contiguous BNSH cache [B, KVH, max_seq, D]: thread gid takes
// chunk pair j of new token t of (batch b, kv head h), with j fastest, then t, so a wave's
// stores run along consecutive cache rows of one head. past(b) is the padded-batch rule.
template <int MODE>
__global__ __launch_bounds__(kThreads) void bnsh_kernel(BnshArgs a) {
    const int lhc = a.D == 256 ? 4 : (a.D == 128 ? 3 : 2);  // log2(D / 16)
    const long long n = (long long)a.B * a.KVH * a.S << lhc;
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= n) return;
    const int j = (int)(gid & ((1 << lhc) - 1));
    long long rest = gid >> lhc;
    const int t = (int)(rest % a.S);
    rest /= a.S;
    const int h = (int)(rest % a.KVH);
    const int b = (int)(rest / a.KVH);
    // past length: zero when the scalar total equals seq_len (a prompt), else own total - S
    const uint32_t total = (uint32_t)a.total_seq[0], own = (uint32_t)a.key_total[b];
    const uint32_t S = (uint32_t)a.S;
    const long long past = total == S ? 0 : (own >= S ? (long long)(own - S) : 0);
    const long long pos = past + t;
    if (pos >= a.max_seq) return;  // outside the cache: not written
    if (MODE != kCopy && pos >= a.rotary_positions) return;
    const int dA = j << 3, dB = dA + (a.D >> 1);
    const long long row = (long long)b * a.S + t;
    const half_t *ks = (a.query ? a.query : a.key) + row * a.src_stride + a.k_off +
                       (long long)h * a.D;
    const half_t *vs = (a.query ? a.query : a.value) + row * a.src_stride + a.v_off +
                       (long long)h * a.D;
    // source rows are read once: non-temporal
    const half8_t kA = gload_nt<half8_t>(ks + dA), kB = gload_nt<half8_t>(ks + dB);
    const half8_t vA = gload_nt<half8_t>(vs + dA), vB = gload_nt<half8_t>(vs + dB);
    half8_t oA = kA, oB = kB;
    if (MODE != kCopy) {
        half8_t pA = kB, pB = kA;  // kNeoxFull: each other's partners
        if (MODE == kNeox) {
            const int R = a.rotary_dim, half = R >> 1;
            pA = gload<half8_t>(ks + (dA >= R ? 0 : (dA < half ? dA + half : dA - half)));
            pB = gload<half8_t>(ks + (dB >= R ? 0 : (dB < half ? dB + half : dB - half)));
        }
        half8_t cA, sA, cB, sB;
        load_cs<MODE>(a, dA, (int)pos, cA, sA);
        if (MODE == kNeoxFull) {
            cB = cA;
            sB = sA;
        } else {
            load_cs<MODE>(a, dB, (int)pos, cB, sB);
        }
        oA = rotate_chunk<MODE>(a, ks, kA, pA, cA, sA, dA, (int)pos);
        oB = rotate_chunk<MODE>(a, ks, kB, pB, cB, sB, dB, (int)pos);
    }
    const long long dst = (((long long)b * a.KVH + h) * a.max_seq + pos) * a.D;
    *(half8_t *)(a.pk + dst + dA) = oA;
    *(half8_t *)(a.pk + dst + dB) = oB;
    *(half8_t *)(a.pv + dst + dA) = vA;
    *(half8_t *)(a.pv + dst + dB) = vB;
}

}  // namespace

pa_status launch_kv_append_bnsh(const BnshArgs &a, hipStream_t stream) {
    LaunchScope scope("kv_append_bnsh", stream);
    const long long n = ((long long)a.B * a.KVH * a.S) * (a.D >> 4);
    if (n == 0) return PA_OK;
    const unsigned grid = (unsigned)((n + kThreads - 1) / kThreads);
    const int R = a.rotary_dim;
    int mode = kCopy;
    if (a.rotary_mode == PA_ROTARY_NEOX)
        mode = R == a.D ? kNeoxFull : (R % 16 == 0 ? kNeox : kGeneric);
    else if (a.rotary_mode == PA_ROTARY_INTERLEAVED)
        mode = (R % 8 == 0) ? kInter : kGeneric;
    switch (mode) {
        case kCopy: scope.launch(bnsh_kernel<kCopy>, dim3(grid), dim3(kThreads), 0, a); break;
        case kNeoxFull:
            scope.launch(bnsh_kernel<kNeoxFull>, dim3(grid), dim3(kThreads), 0, a);
            break;
        case kNeox: scope.launch(bnsh_kernel<kNeox>, dim3(grid), dim3(kThreads), 0, a); break;
        case kInter: scope.launch(bnsh_kernel<kInter>, dim3(grid), dim3(kThreads), 0, a); break;
        default: scope.launch(bnsh_kernel<kGeneric>, dim3(grid), dim3(kThreads), 0, a); break;
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

namespace {

// Thread counts and the rotary variant of one append launch; false when the launch would need
// more than 32-bit thread indexes.
bool size_append(AppendArgs &a, unsigned &grid, int &mode) {
    const long long pairs = (long long)((a.T + 1) / 2) * (a.D >> 4);  // per head row
    const long long nkv = pairs * a.G;
    const long long nkv_pad = (nkv + kThreads - 1) / kThreads * kThreads;
    const long long nq = a.q_out ? pairs * a.H : 0;
    const long long total = nkv_pad + nq;
    if (total + 2 * kThreads >= (1LL << 31)) return false;  // 32-bit thread indexing
    a.nkv = (int)nkv;
    a.nkv_pad = (int)nkv_pad;
    a.nq = (int)nq;
    grid = (unsigned)((total + kThreads - 1) / kThreads);
    const int R = a.rotary_dim;
    mode = kCopy;
    if (a.rotary_mode == PA_ROTARY_NEOX)
        mode = R == a.D ? kNeoxFull : (R % 16 == 0 ? kNeox : kGeneric);
    else if (a.rotary_mode == PA_ROTARY_INTERLEAVED)
        mode = (R % 8 == 0) ? kInter : kGeneric;
    return true;
}

}  // namespace

pa_status launch_kv_append(const AppendArgs &a_in, hipStream_t stream) {
    LaunchScope scope("kv_append", stream);
    AppendArgs a = a_in;
    if (a.T == 0) return PA_OK;
    if (a.q_out && !a.q_src) return PA_ERR_NULL;
    unsigned grid;
    int mode;
    if (!size_append(a, grid, mode)) return PA_ERR_UNSUPPORTED;
    const bool lanecu = a.B + 1 <= kLaneCu * 64;
#define PA_APPEND(M)                                                                    \
    if (lanecu)                                                                         \
        scope.launch(append_kernel<M, true>, dim3(grid), dim3(kThreads), 0, a);         \
    else                                                                                \
        scope.launch(append_kernel<M, false>, dim3(grid), dim3(kThreads), 0, a);
    switch (mode) {
        case kCopy: PA_APPEND(kCopy); break;
        case kNeoxFull: PA_APPEND(kNeoxFull); break;
        case kNeox: PA_APPEND(kNeox); break;
        case kInter: PA_APPEND(kInter); break;
        default: PA_APPEND(kGeneric); break;
    }
#undef PA_APPEND
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status check_kv_append(const AppendArgs &a_in) {
    AppendArgs a = a_in;
    unsigned grid;
    int mode;
    if (a.q_out && !a.q_src) return PA_ERR_NULL;
    return size_append(a, grid, mode) ? PA_OK : PA_ERR_UNSUPPORTED;
}

pa_status launch_append_plan(const AppendArgs &a_in, const PlanArgs &p, hipStream_t stream) {
    LaunchScope scope("append_plan", stream);
    AppendArgs a = a_in;
    if (a.q_out && !a.q_src) return PA_ERR_NULL;
    unsigned grid;
    int mode;
    if (!size_append(a, grid, mode)) return PA_ERR_UNSUPPORTED;
    grid += 1;  // workgroup 0: the planner
    const bool lanecu = a.B + 1 <= kLaneCu * 64;
    const bool wave = p.B <= 64;  // the one-wave planner when the batch fits in a wave
#define PA_AP(M, LC)                                                                         \
    if (wave)                                                                                \
        scope.launch(append_plan_kernel<M, LC, 64>, dim3(grid), dim3(kThreads), 0, a, p);    \
    else                                                                                     \
        scope.launch(append_plan_kernel<M, LC, kPlanThreads>, dim3(grid), dim3(kThreads), 0, \
                     a, p);
#define PA_APM(M)    \
    if (lanecu) {    \
        PA_AP(M, true)  \
    } else {         \
        PA_AP(M, false) \
    }
    switch (mode) {
        case kCopy: PA_APM(kCopy); break;
        case kNeoxFull: PA_APM(kNeoxFull); break;
        case kNeox: PA_APM(kNeox); break;
        case kInter: PA_APM(kInter); break;
        default: PA_APM(kGeneric); break;
    }
#undef PA_APM
#undef PA_AP
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
