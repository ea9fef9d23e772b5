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
#include "common.h"

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
template <int MODE>
__device__ __forceinline__ half8_t rotate_chunk(const AppendArgs &a, const half_t *ks, half8_t kv,
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

// cos/sin chunk for dims d0 .. d0+7 at pos (NeoX: 8 columns; interleaved: 4 columns).
template <int MODE>
__device__ __forceinline__ void load_cs(const AppendArgs &a, int d0, int pos, half8_t &cs,
                                        half8_t &sn) {
    const int R = a.rotary_dim, half = R >> 1;
    cs = half8_t{};
    sn = half8_t{};
    if (d0 >= R) return;
    if (MODE == kNeox || MODE == kNeoxFull) {  // half % 8 == 0: aligned chunk of columns
        const long long c0 = (long long)pos * half + (d0 < half ? d0 : d0 - half);
        cs = gload<half8_t>(a.cos + c0);
        sn = gload<half8_t>(a.sin + c0);
    } else if (MODE == kInter) {
        const long long c0 = (long long)pos * half + (d0 >> 1);
        const half4_t c4 = gload<half4_t>(a.cos + c0), s4 = gload<half4_t>(a.sin + c0);
        for (int e = 0; e < 4; ++e) { cs[e] = c4[e]; sn[e] = s4[e]; }
    }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
    __shared__ int32_t s_cu[kLdsCu];
    __shared__ int32_t s_past[kLdsCu];
    const int hc = a.D >> 4;  // chunk pairs per row
    const long long n = (long long)a.T * a.G * hc;
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    const bool live = gid < n;
    const long long gidc = live ? gid : n - 1;
    const int j = (int)(gidc % hc);
    const long long rg = gidc / hc;
    const int g = (int)(rg % a.G);
    const int i = (int)(rg / a.G);
    const int dA = j << 3, dB = dA + (a.D >> 1);
    const int lane = threadIdx.x & 63;

    // Loads that do not depend on the sequence: both chunks of K and V, NeoX partners that are
    // not the other chunk, the slot, and (small batches) this lane's cu / past entries.
    const half_t *ks = (a.query ? a.query : a.key) + (long long)i * a.src_stride + a.k_off +
                       (long long)g * a.D;
    const half_t *vs = (a.query ? a.query : a.value) + (long long)i * a.src_stride + a.v_off +
                       (long long)g * a.D;
    const half8_t kA = gload<half8_t>(ks + dA), kB = gload<half8_t>(ks + dB);
    const half8_t vA = gload<half8_t>(vs + dA), vB = gload<half8_t>(vs + dB);
    half8_t pA = kB, pB = kA;  // kNeoxFull: the chunks are each other's partners
    if (MODE == kNeox) {
        const int half = a.rotary_dim >> 1;
        if (dA < a.rotary_dim) pA = gload<half8_t>(ks + (dA < half ? dA + half : dA - half));
        if (dB < a.rotary_dim) pB = gload<half8_t>(ks + (dB < half ? dB + half : dB - half));
    }
    long long slot = a.slot_mapping ? a.slot_mapping[i] : 0;

    int b, t, past;
    if (a.B + 1 <= kLaneCu * 64) {
        int cuv[kLaneCu], pav[kLaneCu];
        for (int c = 0; c < kLaneCu; ++c) {
            const int k = 64 * c + lane;
            cuv[c] = k <= a.B ? a.cu[k] : 0x7fffffff;
            pav[c] = k < a.B ? a.past[k] : 0;
        }
        const int i0 = __builtin_amdgcn_readfirstlane(i);
        if (__ballot(i != i0) == 0) {
            // one token per wave: b + 1 = number of entries cu[k] <= i (cu[B] = T > i)
            int cnt = 0;
            for (int c = 0; c < kLaneCu; ++c) cnt += __popcll(__ballot(cuv[c] <= i0));
            b = min(cnt, a.B) - 1;
            const int c = b >> 6, l = b & 63;
            int cb = 0, pb = 0;
            for (int q = 0; q < kLaneCu; ++q)
                if (q == c) { cb = __shfl(cuv[q], l, 64); pb = __shfl(pav[q], l, 64); }
            t = i0 - cb;
            past = pb;
        } else {
            // several tokens in the wave: count entry by entry
            int cnt = 0;
            for (int q = 0; q < kLaneCu; ++q)
                for (int l = 0; l < 64 && 64 * q + l <= a.B; ++l) cnt += __shfl(cuv[q], l, 64) <= i;
            b = min(cnt, a.B) - 1;
            const int c = b >> 6, l = b & 63;
            int cb = 0, pb = 0;
            for (int q = 0; q < kLaneCu; ++q) {
                const int x = __shfl(cuv[q], l, 64), y = __shfl(pav[q], l, 64);
                if (q == c) { cb = x; pb = y; }
            }
            t = i - cb;
            past = pb;
        }
    } else {
        const bool lds = a.B + 1 <= kLdsCu;  // uniform over the grid
        if (lds) {
            for (int k = threadIdx.x; k <= a.B; k += kThreads) {
                s_cu[k] = a.cu[k];
                if (k < a.B) s_past[k] = a.past[k];
            }
            __syncthreads();
        }
        b = lds ? find_batch(s_cu, a.B, i) : find_batch(a.cu, a.B, i);
        t = i - (lds ? s_cu[b] : a.cu[b]);
        past = lds ? s_past[b] : a.past[b];
    }
    if (!live) return;
    const int pos = past + t;
    if (!a.slot_mapping) {
        const int blk = pos / a.bs;
        slot = (long long)a.bt[(long long)b * a.MB + blk] * a.bs + (pos - blk * a.bs);
    }

    half8_t oA = kA, oB = kB;
    if (MODE != kCopy) {
        half8_t cA, sA, cB, sB;
        load_cs<MODE>(a, dA, pos, cA, sA);
        if (MODE == kNeoxFull) {  // dB = dA + R/2 uses the same columns
            cB = cA;
            sB = sA;
        } else {
            load_cs<MODE>(a, dB, pos, cB, sB);
        }
        oA = rotate_chunk<MODE>(a, ks, kA, pA, cA, sA, dA, pos);
        oB = rotate_chunk<MODE>(a, ks, kB, pB, cB, sB, dB, pos);
    }
    if (slot < 0) return;
    const long long dst = (slot * a.G + g) * a.D;
    *(half8_t *)(a.kc + dst + dA) = oA;
    *(half8_t *)(a.kc + dst + dB) = oB;
    *(half8_t *)(a.vc + dst + dA) = vA;
    *(half8_t *)(a.vc + dst + dB) = vB;
}

}  // namespace

pa_status launch_kv_append(const AppendArgs &a, hipStream_t stream) {
    LaunchScope scope("kv_append", stream);
    const long long n = (long long)a.T * a.G * (a.D >> 4);
    if (n == 0) return PA_OK;
    const unsigned grid = (unsigned)((n + kThreads - 1) / kThreads);
    const int R = a.rotary_dim;
    int mode = kCopy;
    if (a.rotary_mode == PA_ROTARY_NEOX)
        mode = R == a.D ? kNeoxFull : (R % 16 == 0 ? kNeox : kGeneric);
    else if (a.rotary_mode == PA_ROTARY_INTERLEAVED)
        mode = (R % 8 == 0) ? kInter : kGeneric;
    switch (mode) {
        case kCopy: scope.launch(append_kernel<kCopy>, dim3(grid), dim3(kThreads), 0, a); break;
        case kNeoxFull:
            scope.launch(append_kernel<kNeoxFull>, dim3(grid), dim3(kThreads), 0, a);
            break;
        case kNeox: scope.launch(append_kernel<kNeox>, dim3(grid), dim3(kThreads), 0, a); break;
        case kInter: scope.launch(append_kernel<kInter>, dim3(grid), dim3(kThreads), 0, a); break;
        default: scope.launch(append_kernel<kGeneric>, dim3(grid), dim3(kThreads), 0, a); break;
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
