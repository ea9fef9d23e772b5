// Log-sum-exp merge of (o, m, l) partials: the per-wave loop shared by the combine kernel and the
// combine role of the post-decode launch.
//
// Operation: the merge pass of the "com.microsoft.PagedAttention ... manifest.json" page
// (PagedAttention.AttendSplitKMerge over the partialOut / partialStats intermediates), and the
// merge of the per-edge partials of the "alice-llm ... sparse_attention_forward.wgsl" page.
// Output row r = k*lanes + lane of group k:
//   M = max m over units with l > 0, w = exp(m - M), out = sum w o / sum w l (0 if no l > 0).
//
// D/4 lanes own one output row (a float4 each), so a row block of 64*4/D rows fills a wave; a
// wave takes R row blocks of a group at once. The rows of one unit are adjacent in memory, so a
// wave's loads for one unit are one contiguous span (with R = 2 and four rows per unit at
// D = 128, the unit's whole 2 KB). Units are merged online, 8 / R per memory round trip
// (running max, rescaled sums), the next round's loads in flight while one is merged.
// wave / nwaves: this wave's index among the waves that share the
// work (grid-stride over groups' row-block pairs). mode: 0 uniform splits, 1 CSR offsets,
// 2 planner list. combine_dispatch picks R from the row count.
#pragma once
#include "common.h"

namespace pa {

template <int D, int R>
__device__ __forceinline__ void combine_rows(const CombineArgs &a, int mode, int wave, int nwaves) {
    constexpr int LPR = D / 4;      // lanes per row
    constexpr int RPW = 64 / LPR;   // rows per wave per row block
    constexpr int NB = 8 / R;       // units loaded per round trip
    const int lane = threadIdx.x & 63;
    const int sub = lane % LPR;     // float4 index inside the row
    const int rw = lane / LPR;      // row inside the wave's row block
    const int n_groups = (mode == 2) ? a.n_items[0] : a.num_groups;
    const int blocks_per_group = (a.lanes + R * RPW - 1) / (R * RPW);
    const long long n_work = (long long)n_groups * blocks_per_group;

    for (long long w = wave; w < n_work; w += nwaves) {
        const int k = (int)(w / blocks_per_group);
        const int row0 = (int)(w - (long long)k * blocks_per_group) * R * RPW + rw;
        long long e0, e1, row_group;
        if (mode == 0) {
            e0 = (long long)k * a.splits; e1 = e0 + a.splits; row_group = k;
        } else if (mode == 1) {
            e0 = a.group_ptr[k]; e1 = a.group_ptr[k + 1]; row_group = k;
        } else {
            const CombItem it = a.items[k];
            e0 = it.e0; e1 = e0 + it.count; row_group = it.row;
        }
        int lr[R];
        bool active[R];
        for (int j = 0; j < R; ++j) {
            const int r = row0 + j * RPW;
            active[j] = r < a.lanes;
            lr[j] = active[j] ? r : 0;
        }
        float M[R], Ls[R];
        float4_t acc[R];
        for (int j = 0; j < R; ++j) {
            M[j] = -INFINITY; Ls[j] = 0.f; acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
        }
        // Software-pipelined: the loads of round e + NB are issued before round e is merged,
        // so a wave always has a round of partials in flight.
        float mv[NB][R], lv[NB][R];
        float4_t ov[NB][R];
        auto load_round = [&](long long e) {
            for (int u = 0; u < NB; ++u) {
                const long long eu = e + u < e1 ? e + u : e1 - 1;
                for (int j = 0; j < R; ++j) {
                    const long long p = eu * a.lanes + lr[j];
                    mv[u][j] = a.m[p];
                    lv[u][j] = e + u < e1 ? a.l[p] : 0.f;
                    ov[u][j] = gload_nt<float4_t>(a.o + p * D + 4 * sub);
                }
            }
        };
        if (e0 < e1) load_round(e0);
        for (long long e = e0; e < e1; e += NB) {
            float cm[NB][R], cl[NB][R];
            float4_t co[NB][R];
            for (int u = 0; u < NB; ++u)
                for (int j = 0; j < R; ++j) {
                    cm[u][j] = mv[u][j]; cl[u][j] = lv[u][j]; co[u][j] = ov[u][j];
                }
            if (e + NB < e1) load_round(e + NB);
            for (int j = 0; j < R; ++j) {
                float bm = -INFINITY;
                for (int u = 0; u < NB; ++u)
                    if (cl[u][j] > 0.f) bm = fmaxf(bm, cm[u][j]);
                if (bm == -INFINITY) continue;
                const float Mn = fmaxf(M[j], bm);
                const float sc =
                    (M[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((M[j] - Mn) * kLog2e);
                acc[j] *= sc;
                Ls[j] *= sc;
                for (int u = 0; u < NB; ++u) {
                    const float wu =
                        cl[u][j] > 0.f ? __builtin_amdgcn_exp2f((cm[u][j] - Mn) * kLog2e) : 0.f;
                    acc[j] += wu * co[u][j];
                    Ls[j] += wu * cl[u][j];
                }
                M[j] = Mn;
            }
        }
        for (int j = 0; j < R; ++j) {
            if (!active[j]) continue;
            const float inv = Ls[j] > 0.f ? 1.f / Ls[j] : 0.f;
            float4_t o = acc[j] * inv;
            const long long r = row_group * a.lanes + row0 + j * RPW;
            if (a.out_f32) {
                *(float4_t *)((float *)a.out + r * D + 4 * sub) = o;
            } else {
                half4_t h;
                for (int i = 0; i < 4; ++i) h[i] = (half_t)o[i];
                *(half4_t *)((half_t *)a.out + r * D + 4 * sub) = h;
            }
        }
    }
}


// Two row blocks per wave when a group has that many rows (fewer, longer contiguous loads);
// one otherwise, so that no load is spent on rows past the group.
__host__ __device__ constexpr int combine_r(int lanes, int D) { return lanes >= 2 * (256 / D) ? 2 : 1; }

template <int D>
__device__ __forceinline__ void combine_dispatch(const CombineArgs &a, int mode, int wave,
                                                 int nwaves) {
    if (combine_r(a.lanes, D) == 2) combine_rows<D, 2>(a, mode, wave, nwaves);
    else combine_rows<D, 1>(a, mode, wave, nwaves);
}

// Waves to launch for up to max_groups groups of `lanes` rows of head dim D. Capped at 8 (two
// row blocks per wave) or 12 waves per CU: on the 2 GB block-sparse merge more waves in flight
// read HBM more slowly (8192 waves: 5.2 TB/s; 2048 waves of two row blocks: 5.6 TB/s).
inline long long combine_waves(int max_groups, int lanes, int D) {
    const int R = combine_r(lanes, D);
    const int rows = R * (64 / (D / 4));
    const long long work = (long long)max_groups * ((lanes + rows - 1) / rows);
    const long long cap = (long long)device_cu_count() * (R == 2 ? 8 : 12);
    return work < cap ? work : cap;
}

}  // namespace pa
