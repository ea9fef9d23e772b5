// The device planner of paged attention: one workgroup turns the sequence lengths into the
// decode, prefill and combine work lists in the workspace. Included by the translation units
// that launch it: on its own (plan_kernel) or beside the key/value append in one launch.
//
// Operation: the split policy of the "com.microsoft.PagedAttention ... manifest.json" page
// (its numSplits derivation and the split_attention / merge passes), decided on the device from
// the device-resident sequence lengths so that the host never waits on data.
#pragma once

#include "common.h"

namespace pa {

// ============================================================================================
// Device planner
// ============================================================================================
namespace {

constexpr int kPlanThreads = 256;
constexpr int kTileKeys = 32;

template <int TH>
__device__ __forceinline__ long long block_sum_ll(long long v, long long *sh) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if (lane == 0) sh[wid] = v;
    __syncthreads();
    long long t = 0;
    for (int i = 0; i < TH / 64; ++i) t += sh[i];
    return t;
}

// Exclusive scan of NV counters across the workgroup; returns totals in tot[].
template <int TH, int NV, int M>
__device__ __forceinline__ void block_scan(const int (&v)[NV], int (&excl)[NV], int (&tot)[NV],
                                           int (&sh)[M]) {
    static_assert(M >= TH / 64 * NV, "scan scratch: one entry per wave and counter");
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int inc[NV];
    for (int k = 0; k < NV; ++k) {
        int x = v[k];
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        inc[k] = x;
    }
    __syncthreads();
    if (lane == 63)
        for (int k = 0; k < NV; ++k) sh[wid * NV + k] = inc[k];
    __syncthreads();
    for (int k = 0; k < NV; ++k) {
        int before = 0, all = 0;
        for (int i = 0; i < TH / 64; ++i) {
            const int x = sh[i * NV + k];
            if (i < wid) before += x;
            all += x;
        }
        excl[k] = before + inc[k] - v[k];
        tot[k] = all;
    }
}

__device__ __forceinline__ int ceil_div_i(long long a, long long b) { return (int)((a + b - 1) / b); }

// Prefill items are listed longest first (by 64-key tiles, counting-sorted in LDS over four bins
// per planner thread; items of bins - 1 or more tiles share the top bin), so that the persistent
// prefill workgroups take the long items early and the short ones fill the tail.
template <int TH>
constexpr int pre_bins() { return 4 * TH; }
constexpr int kPreBinKeys = 64;
template <int TH>
__device__ __forceinline__ int pre_bin(int k1) {
    return min(pre_bins<TH>() - 1, (k1 + kPreBinKeys - 1) / kPreBinKeys);
}
__device__ __forceinline__ int round_tile(long long x) {
    return (int)((x + kTileKeys - 1) / kTileKeys * kTileKeys);
}

}  // namespace

// One workgroup turns the sequence lengths into work lists.
//  * Decode-like sequences (1 <= n_b <= tpi_dec) are cut into pieces of their key range [0, L_b).
//    Auto mode balances them stream-K style: the 32-key tiles of all decode-like sequences are
//    laid end to end and cut into `slots` equal shares of q tiles; the decode kernel's
//    workgroup j processes share j, i.e. the pieces of the sequences that overlap
//    [j*q, (j+1)*q). Even mode cuts sequence b into ceil(L_b / C_b) pieces with
//    C_b = ceil(L_b / splits) rounded up to the tile, listed whole pieces first and taken from a
//    dynamic counter.
//  * Every query row of a sequence cut into >= 2 pieces gets nsplit partial units and one entry
//    of the combine list; a sequence left whole writes its output directly.
//  * Longer sequences get tiles of tpi_pre rows; the prefill list holds them longest key range
//    first across all sequences.
// Runs on the first TH threads of a workgroup (TH = 64: one wave, or kPlanThreads); when the
// workgroup is larger, its other waves must have exited (a barrier then waits for the
// surviving waves only).
template <int TH>
__device__ __forceinline__ void plan_body(const PlanArgs &a) {
    constexpr int kPreBins = pre_bins<TH>();
    __shared__ long long sh_ll[TH / 64];
    __shared__ int sh_i[TH / 64 * 5];  // block_scan<NV> needs (waves x NV)
    __shared__ int sh_bin[kPreBins];  // prefill items per length bin, then list offsets
    const int tid = threadIdx.x;
    for (int i = tid; i < kPreBins; i += TH) sh_bin[i] = 0;
    const bool streamk = a.mode == 0;

    auto decode_like = [&](int n) { return n >= 1 && n <= a.tpi_dec; };
    auto piece_keys = [&](int L) { return round_tile(ceil_div_i(L, a.splits)); };
    // key range end of prefill item `tile` of a sequence with n new tokens after `past`
    auto pre_k1 = [&](int tile, int n, int past) {
        return a.causal ? past + min(n, (tile + 1) * a.tpi_pre) : past + n;
    };

    // Sequence b's first token, new tokens and past length. The first TH sequences are
    // read once, here, and kept in registers for all passes (one memory round trip instead of
    // three); later chunks are read where they are needed.
    int r_cu0 = 0, r_n = 0, r_past = 0;
    if (tid < a.B) {
        r_cu0 = a.cu[tid];
        r_n = a.cu[tid + 1] - r_cu0;
        r_past = a.past[tid];
    }
    auto seq = [&](int b, int &cu0, int &n, int &past) {
        if (b < TH) {  // b == tid
            cu0 = r_cu0; n = r_n; past = r_past;
        } else {
            cu0 = a.cu[b]; n = a.cu[b + 1] - cu0; past = a.past[b];
        }
    };

    // Pass 1: tiles of decode-like sequences; in even mode, the count of whole pieces.
    long long ntiles = 0, nfull = 0;
    for (int b = tid; b < a.B; b += TH) {
        int cu0, n, past;
        seq(b, cu0, n, past);
        if (!decode_like(n)) continue;
        const int L = past + n;
        ntiles += ceil_div_i(L, kTileKeys);
        if (!streamk) {
            const int Cb = piece_keys(L);
            const int c = ceil_div_i(L, Cb);
            nfull += (L % Cb == 0) ? c : c - 1;
        }
    }
    ntiles = block_sum_ll<TH>(ntiles, sh_ll);
    const int full_total = (int)block_sum_ll<TH>(nfull, sh_ll);
    long long q = 1;
    int used = 0;
    if (streamk && ntiles > 0) {
        const long long min_tiles = max(1, (a.min_chunk + kTileKeys - 1) / kTileKeys);
        q = max(min_tiles, (ntiles + a.slots - 1) / a.slots);
        used = (int)((ntiles + q - 1) / q);
    }

    // Pass 2: per-sequence counts, scans, lists.
    // carry: decode items, partial units, combine rows, prefill tiles, tiles before the chunk
    int carry[4] = {0, 0, 0, 0};
    long long carry_tiles = 0;
    int carry_tail = 0;
    for (int base = 0; base < a.B; base += TH) {
        const int b = base + tid;
        int n = 0, L = 0, past = 0, cu0 = 0, T = 0;
        if (b < a.B) {
            seq(b, cu0, n, past);
            L = past + n;
            if (decode_like(n)) T = ceil_div_i(L, kTileKeys);
        }
        int tv[1] = {T}, tex[1], ttot[1];
        block_scan<TH, 1>(tv, tex, ttot, sh_i);
        const long long TB = carry_tiles + tex[0];   // first global tile of sequence b
        int c = 0, Cb = 1, tail = 0;
        int cnt[5] = {0, 0, 0, 0, 0};  // items, partial units, combine rows, prefill, tail
        if (b < a.B) {
            if (decode_like(n)) {
                if (streamk) {
                    c = (int)((TB + T - 1) / q - TB / q + 1);
                } else {
                    Cb = piece_keys(L);
                    c = ceil_div_i(L, Cb);
                    tail = (L % Cb == 0) ? 0 : 1;
                }
                cnt[0] = c;
                if (c >= 2) {
                    cnt[1] = n * c;
                    cnt[2] = n;
                }
            } else if (n > a.tpi_dec) {
                cnt[3] = ceil_div_i(n, a.tpi_pre);
            }
        }
        cnt[4] = tail;
        int ex[5], tot[5];
        block_scan<TH, 5>(cnt, ex, tot, sh_i);
        const int tlex = ex[4];
        if (b < a.B) {
            const int ubase = carry[1] + ex[1];
            const int cbase = carry[2] + ex[2];
            for (int sp = 0; sp < c; ++sp) {
                AttnItem it;
                it.b = b; it.t0 = 0;
                it.base = c >= 2 ? ubase : -1; it.nsplit = c; it.split = sp;
                it.cu0 = cu0; it.n = n; it.past = past;
                int idx;
                if (streamk) {
                    idx = carry[0] + ex[0] + sp;
                    const long long j = TB / q + sp;
                    const long long t0 = max(TB, j * q), t1 = min(TB + T, (j + 1) * q);
                    it.k0 = (int)(t0 - TB) * kTileKeys;
                    it.k1 = min(L, (int)(t1 - TB) * kTileKeys);
                    if (t0 == j * q && j < a.slots) {
                        a.slot_ptr[j] = idx;
                        a.slot_first[j] = it;
                    }
                } else {
                    const bool is_tail = sp >= c - tail;
                    idx = is_tail ? full_total + carry_tail + tlex : carry[0] - carry_tail +
                                                                         (ex[0] - tlex) + sp;
                    it.k0 = sp * Cb;
                    it.k1 = min(L, (sp + 1) * Cb);
                }
                if (idx < a.cap_dec) a.dec[idx] = it;
            }
            for (int t = 0; t < cnt[2]; ++t) {
                const int idx = cbase + t;
                if (idx < a.cap_comb) {
                    CombItem ci;
                    ci.row = cu0 + t; ci.e0 = ubase + t * c; ci.count = c; ci.pad = 0;
                    a.comb[idx] = ci;
                }
            }
            for (int tile = 0; tile < cnt[3]; ++tile)
                atomicAdd(&sh_bin[pre_bin<TH>(pre_k1(tile, n, past))], 1);
        }
        for (int k = 0; k < 4; ++k) carry[k] += tot[k];
        carry_tiles += ttot[0];
        carry_tail += tot[4];
    }
    // Pass 3: prefill items, longest first. Bin offsets in descending bin order, then each item
    // takes the next place of its bin (the order inside a bin is arbitrary; every item writes
    // its own output rows, so the results do not depend on it).
    if (carry[3] > 0) {  // block-uniform
        __syncthreads();
        int c4[4], s4 = 0;
        for (int i = 0; i < 4; ++i) {
            c4[i] = sh_bin[kPreBins - 1 - (4 * tid + i)];
            s4 += c4[i];
        }
        int sv[1] = {s4}, sex[1], stot[1];
        block_scan<TH, 1>(sv, sex, stot, sh_i);
        int run = sex[0];
        for (int i = 0; i < 4; ++i) {
            sh_bin[kPreBins - 1 - (4 * tid + i)] = run;
            run += c4[i];
        }
        __syncthreads();
    }
    for (int b = tid; b < a.B && carry[3] > 0; b += TH) {
        int cu0, n, past;
        seq(b, cu0, n, past);
        if (n <= a.tpi_dec) continue;
        const int ntile = ceil_div_i(n, a.tpi_pre);
        for (int tile = 0; tile < ntile; ++tile) {
            AttnItem it;
            it.b = b; it.t0 = tile * a.tpi_pre; it.k0 = 0;
            it.k1 = pre_k1(tile, n, past);
            it.base = -1; it.nsplit = 1; it.split = 0;
            it.cu0 = cu0; it.n = n; it.past = past;
            const int idx = atomicAdd(&sh_bin[pre_bin<TH>(it.k1)], 1);
            if (idx < a.cap_pre) a.pre[idx] = it;
        }
    }
    const int ndec_items = min(carry[0], a.cap_dec);
    if (streamk)
        for (int j = used + tid; j <= a.slots; j += TH) a.slot_ptr[j] = ndec_items;
    if (tid == 0) {
        a.hdr->n_dec = ndec_items;
        a.hdr->units = carry[1];
        a.hdr->n_comb = min(carry[2], a.cap_comb);
        a.hdr->n_pre = min(carry[3], a.cap_pre);
        a.hdr->chunk = (int)(q * kTileKeys);
        a.hdr->next_dec = 0;
        a.hdr->next_pre = 0;
    }
}

}  // namespace pa
