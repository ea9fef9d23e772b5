// Log-sum-exp merge of (o, m, l) partials: the per-wave loop shared by the combine kernel and the
// combine role of the post-decode launch.
//
// Operation: the merge pass of the "com.microsoft.PagedAttention ... manifest.json" page
// (PagedAttention.AttendSplitKMerge over the partialOut / partialStats intermediates), and the
// merge of the per-edge partials of the "alice-llm ... sparse_attention_forward.wgsl" page.
// Output row r = k*lanes + lane of group k:
//   M = max m over units with l > 0, w = exp(m - M), out = sum w o / sum w l (0 if no l > 0).
//
// D/4 lanes own one output row (a float4 each), so a wave covers 64*4/D rows; the rows of one
// unit are adjacent in memory, so a wave's loads for one unit are one contiguous span. Units are
// merged online, eight per memory round trip (running max, rescaled sums), so a row costs
// ceil(units / 8) dependent loads. wave / nwaves: this wave's index among the waves that share
// the work (grid-stride over row blocks). mode: 0 uniform splits, 1 CSR offsets, 2 planner list.
#pragma once
#include "common.h"

namespace pa {

template <int D>
__device__ __forceinline__ void combine_rows(const CombineArgs &a, int mode, int wave, int nwaves) {
    constexpr int LPR = D / 4;      // lanes per row
    constexpr int RPW = 64 / LPR;   // rows per wave
    constexpr int NB = 8;           // units loaded per round trip
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR;     // float4 index inside the row
    const int rw = lane / LPR;      // row inside the wave's row block
    const int n_groups = (mode == 2) ? a.n_items[0] : a.num_groups;
    const int blocks_per_group = (a.lanes + RPW - 1) / RPW;
    const long long n_work = (long long)n_groups * blocks_per_group;

    for (long long w = wave; w < n_work; w += nwaves) {
        const int k = (int)(w / blocks_per_group);
        const int lane_row = (int)(w - (long long)k * blocks_per_group) * RPW + rw;
        long long e0, e1, row_group;
        if (mode == 0) {          // uniform splits
            e0 = (long long)k * a.splits; e1 = e0 + a.splits; row_group = k;
        } else if (mode == 1) {   // CSR offsets
            e0 = a.group_ptr[k]; e1 = a.group_ptr[k + 1]; row_group = k;
        } else {                  // planner list
            const CombItem it = a.items[k];
            e0 = it.e0; e1 = e0 + it.count; row_group = it.row;
        }
        const bool active = lane_row < a.lanes;
        const int lr = active ? lane_row : 0;

        // Online merge, NB units per round trip: every lane of the row loads the units' m and l
        // (one broadcast line) and its own float4 of o, all before any of them is used.
        float M = -INFINITY, Ls = 0.f;
        float4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (long long e = e0; e < e1; e += NB) {
            float mv[NB], lv[NB];
            float4_t ov[NB];
            for (int u = 0; u < NB; ++u) {
                const long long eu = e + u < e1 ? e + u : e1 - 1;
                const long long p = eu * a.lanes + lr;
                mv[u] = a.m[p];
                lv[u] = e + u < e1 ? a.l[p] : 0.f;
                ov[u] = gload_nt<float4_t>(a.o + p * D + 4 * sub);
            }
            float bm = -INFINITY;
            for (int u = 0; u < NB; ++u)
                if (lv[u] > 0.f) bm = fmaxf(bm, mv[u]);
            if (bm == -INFINITY) continue;             // no unit of this batch counts
            const float Mn = fmaxf(M, bm);
            const float sc = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((M - Mn) * kLog2e);
            acc *= sc;
            Ls *= sc;
            for (int u = 0; u < NB; ++u) {
                const float wu = lv[u] > 0.f ? __builtin_amdgcn_exp2f((mv[u] - Mn) * kLog2e) : 0.f;
                acc += wu * ov[u];
                Ls += wu * lv[u];
            }
            M = Mn;
        }
        if (!active) continue;
        const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
        acc *= inv;
        const long long r = row_group * a.lanes + lane_row;
        if (a.out_f32) {
            *(float4_t *)((float *)a.out + r * D + 4 * sub) = acc;
        } else {
            half4_t h;
            for (int i = 0; i < 4; ++i) h[i] = (half_t)acc[i];
            *(half4_t *)((half_t *)a.out + r * D + 4 * sub) = h;
        }
    }
}


// Waves to launch for up to max_groups groups of `lanes` rows of head dim D.
inline long long combine_waves(int max_groups, int lanes, int D) {
    const int rpw = 64 / (D / 4);
    const long long work = (long long)max_groups * ((lanes + rpw - 1) / rpw);
    const long long cap = (long long)device_cu_count() * 32;  // waves: 8 per SIMD
    return work < cap ? work : cap;
}

}  // namespace pa
