// Fused KV append (rotary + scatter into paged cache slots) for gfx950.
//
// Operation: pass "scatter" (PagedAttention.ScatterKV) of the "com.microsoft.PagedAttention ...
// manifest.json" page, fused with the key rotation of the "com.microsoft.SparseAttention ...
// sparse-kv-append.wgsl.jinja" page (rotary macros and main): each new key row is rotated at its
// absolute position, then key and value rows are written to their cache slot; nothing else is
// written.
//
// One thread moves 8 components (16 bytes) of one (token, kv head) row of K and of V, so a wave
// writes 4 (D = 128) or 8 (D = 64) whole 256/128-byte rows and the G rows of a token form one
// contiguous span of the cache. The source rows are requested first; meanwhile the token's
// sequence comes from a binary search of cumulative_sequence_length (staged in LDS with
// past_seqlens when the batch is short), then the slot and the cos/sin row.
//
// Rotary arithmetic is the page's float32 expression with contraction disabled: two rounded
// products, one rounded add or subtract, then round-to-nearest-even to fp16.
#include "common.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsCu = 2048;  // cumulative lengths staged in LDS up to this many entries

enum { kCopy = 0, kNeox = 1, kInter = 2, kGeneric = 3 };

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

template <int MODE>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a) {
    __shared__ int32_t s_cu[kLdsCu];
    __shared__ int32_t s_past[kLdsCu];
    const int chunks = a.D >> 3;
    const long long n = (long long)a.T * a.G * chunks;
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    const bool live = gid < n;
    const long long gidc = live ? gid : n - 1;
    const int j = (int)(gidc % chunks);
    const long long rg = gidc / chunks;
    const int g = (int)(rg % a.G);
    const int i = (int)(rg / a.G);
    const int d0 = j << 3;
    const int R = a.rotary_dim;
    const int half = R >> 1;

    // Loads that do not depend on the row's sequence go first, so their latency overlaps the
    // sequence lookup below: the key and value chunks, the NeoX partner chunk, the slot.
    const half_t *ks = (a.query ? a.query : a.key) + (long long)i * a.src_stride + a.k_off +
                       (long long)g * a.D;
    const half_t *vs = (a.query ? a.query : a.value) + (long long)i * a.src_stride + a.v_off +
                       (long long)g * a.D;
    const half8_t kv = gload<half8_t>(ks + d0);
    const half8_t vv = gload<half8_t>(vs + d0);
    const bool rot = MODE != kCopy && d0 < R;
    const bool first = MODE == kNeox ? d0 < half : true;
    half8_t pk = kv;
    if (MODE == kNeox && rot) pk = gload<half8_t>(ks + (first ? d0 + half : d0 - half));
    long long slot = a.slot_mapping ? a.slot_mapping[i] : 0;

    const bool lds = a.B + 1 <= kLdsCu;
    if (lds) {
        for (int k = threadIdx.x; k <= a.B; k += kThreads) {
            s_cu[k] = a.cu[k];
            if (k < a.B) s_past[k] = a.past[k];
        }
        __syncthreads();
    }
    if (!live) return;
    const int b = lds ? find_batch(s_cu, a.B, i) : find_batch(a.cu, a.B, i);
    const int t = i - (lds ? s_cu[b] : a.cu[b]);
    const int pos = (lds ? s_past[b] : a.past[b]) + t;
    if (!a.slot_mapping) {
        const int blk = pos / a.bs;
        slot = (long long)a.bt[(long long)b * a.MB + blk] * a.bs + (pos - blk * a.bs);
    }

    half8_t kout = kv;
    if (MODE == kNeox) {
        if (rot) {  // half % 8 == 0: the chunk and its partner chunk are aligned
            const long long c0 = (long long)pos * half + (first ? d0 : d0 - half);
            const half8_t cs = gload<half8_t>(a.cos + c0);
            const half8_t sn = gload<half8_t>(a.sin + c0);
            for (int e = 0; e < 8; ++e)
                kout[e] = (half_t)rot_f32((float)kv[e], (float)pk[e], (float)cs[e], (float)sn[e],
                                          first);
        }
    } else if (MODE == kInter) {
        if (rot) {  // R % 8 == 0: the chunk holds 4 whole pairs, columns d0/2 .. d0/2 + 3
            const long long c0 = (long long)pos * half + (d0 >> 1);
            const half4_t cs = gload<half4_t>(a.cos + c0);
            const half4_t sn = gload<half4_t>(a.sin + c0);
            for (int e = 0; e < 8; e += 2) {
                const float c = (float)cs[e >> 1], sv = (float)sn[e >> 1];
                kout[e] = (half_t)rot_f32((float)kv[e], (float)kv[e + 1], c, sv, true);
                kout[e + 1] = (half_t)rot_f32((float)kv[e + 1], (float)kv[e], c, sv, false);
            }
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
            kout[e] = (half_t)rot_f32((float)kv[e], (float)ks[partner], (float)a.cos[c0],
                                      (float)a.sin[c0], fst);
        }
    }
    if (slot < 0) return;
    const long long dst = (slot * a.G + g) * a.D + d0;
    *(half8_t *)(a.kc + dst) = kout;
    *(half8_t *)(a.vc + dst) = vv;
}

}  // namespace

pa_status launch_kv_append(const AppendArgs &a, hipStream_t stream) {
    LaunchScope scope("kv_append", stream);
    const long long n = (long long)a.T * a.G * (a.D >> 3);
    if (n == 0) return PA_OK;
    const unsigned grid = (unsigned)((n + kThreads - 1) / kThreads);
    int mode = kCopy;
    if (a.rotary_mode == PA_ROTARY_NEOX)
        mode = (a.rotary_dim % 16 == 0) ? kNeox : kGeneric;
    else if (a.rotary_mode == PA_ROTARY_INTERLEAVED)
        mode = (a.rotary_dim % 8 == 0) ? kInter : kGeneric;
    switch (mode) {
        case kCopy: scope.launch(append_kernel<kCopy>, dim3(grid), dim3(kThreads), 0, a); break;
        case kNeox: scope.launch(append_kernel<kNeox>, dim3(grid), dim3(kThreads), 0, a); break;
        case kInter: scope.launch(append_kernel<kInter>, dim3(grid), dim3(kThreads), 0, a); break;
        default: scope.launch(append_kernel<kGeneric>, dim3(grid), dim3(kThreads), 0, a); break;
    }
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
