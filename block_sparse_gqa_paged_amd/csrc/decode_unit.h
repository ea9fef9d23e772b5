// Decode attention over a paged fp16 cache for gfx950: the per-(work item, kv head) wave body
// and the persistent loop over the planner's decode items. Included by the translation units
// that launch it: the decode kernel on its own (attention.hip), and the decode role of the launch
// that runs the prefill beside it (prefill.hip).
//
// Operation: the PagedAttention op of the "com.microsoft.PagedAttention ... manifest.json" page
// (passes "main" and "split_attention") for the query rows of decode-like sequences: every
// (token, head) column attends to keys [k0, k1) of its item through the block table, with
// softmax over the scaled scores; whole key ranges write the output, pieces write (o, m, l).
#pragma once

#include "common.h"
#include "plan.h"

#include <math.h>

namespace pa {
namespace {

// Key-row order inside a 32-key tile. MFMA row m of 16-key half u holds key kappa(u, m); the
// choice puts, in the S^T accumulator of lane (g16, n16), keys 8*g16 + 4u + i (i = 0..3), i.e.
// the 8 consecutive keys 8*g16 .. 8*g16 + 7 that the P operand of lane (g16, n16) needs.
__device__ __forceinline__ int kappa(int u, int m) { return 8 * (m >> 2) + 4 * u + (m & 3); }

template <int D>
struct Tile {
    static constexpr int KB = D / 32;  // 32-dim k-blocks of QK^T
    static constexpr int W = D / 16;   // dims per lane of the V layout (D = 16 * W)
    // K operands held in registers for the whole tile at D <= 128; at D = 256 each k-block's
    // operands are read from LDS right before its products (the registers go to V and O)
    static constexpr bool kKRegs = D <= 128;
    half8_t k[2][kKRegs ? KB : 1];     // A operand rows (from LDS): keys kappa(u, n16), dims 32kb+8g16..+7
    uint32_t v[8][W / 2];              // keys 8*g16 + s, dims W*n16 .. W*n16 + W - 1
};

// Physical block of a lane's V row group at the tile at kt (power-of-two block sizes >= 8):
// keys kt + 8*g16 .. + 7, one aligned group, so one block. Lane 16j thereby holds the block of
// group j, which the K copies of rows 8j .. 8j + 7 take by lane read. Groups past the last valid
// key are clamped to it, so no table entry beyond the range is read.
struct TileIds {
    int bv;
};

__device__ __forceinline__ TileIds tile_ids(const AttnArgs &a, const int32_t *bt, int kt, int k1,
                                            int g16) {
    const int lastg = (k1 - 1) & ~7;
    return TileIds{bt[min(kt + 8 * g16, lastg) >> a.log2bs]};
}

// XOR mask, in 16-byte chunks, of row r of a wave's LDS key tile: LDS chunk position p of row r
// holds cache chunk p ^ krow_mask(r). The A-operand read takes the 16 rows kappa(u, 0..15) at
// one chunk; the mask gives those rows distinct positions, so at D = 128 the 16 lanes of a
// 256-byte read pass hit all 64 banks once.
template <int KC>
__device__ __forceinline__ int krow_mask(int r) {
    return ((r & 3) | ((r >> 1) & 12)) & (KC - 1);
}

// One 16-byte global -> LDS copy per lane, non-temporal (the cache is read once): lane l writes
// LDS bytes [16 l, 16 l + 16) of the wave-uniform destination dst.
__device__ __forceinline__ void dma16_nt(const half_t *src, half_t *dst) {
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1))) *)src,
        (void __attribute__((address_space(3))) *)dst, 16, 0, 2 /* nt */);
}

// Issue the copies of the K rows of the tile at kt into this wave's LDS tile kl [32 rows][D]
// (row r = key kt + r). A copy instruction moves 64 * 16 / (2D) whole rows; keys past k1 - 1
// copy key k1 - 1 instead (their scores are masked), so nothing outside the sequence is read.
// A row of key j inside block B sits at B*block_elems + (j mod bs)*key_elems of kcg (kv head g
// of cache row 0).
template <int D, bool POW2>
__device__ __forceinline__ void copy_k(const AttnArgs &a, const int32_t *bt, TileIds ids,
                                       const half_t *kcg, int kt, int k1, int lane, half_t *kl) {
    constexpr int KC = D / 8;      // 16-byte chunks per row
    constexpr int RPI = 64 / KC;   // rows per copy instruction (4 or 8: inside one 8-key group)
    const int klast = k1 - 1;
    const uint32_t ke = a.key_elems;
    const int rr = lane / KC, p = lane % KC;
    for (int i = 0; i < kTileKeys / RPI; ++i) {
        const int r = RPI * i + rr;
        const int key = min(kt + r, klast);
        const half_t *src;
        if (POW2) {
            // rows of group j = RPI*i/8 lie in the block lane 16j looked up for its V rows; the
            // in-block offset uses a 24-bit multiply (key_elems < 2^24 is checked on the host)
            const int blk = __builtin_amdgcn_readlane(ids.bv, 16 * ((RPI * i) >> 3));
            src = kcg + (size_t)blk * a.block_elems + __umul24(key & (a.bs - 1), ke);
        } else {
            const int j = key / a.bs;
            src = kcg + (size_t)bt[j] * a.block_elems + (uint32_t)(key - j * a.bs) * ke;
        }
        dma16_nt(src + 8 * (p ^ krow_mask<KC>(r)), kl + RPI * i * D);
    }
}

// The A operands of the tile from the wave's LDS tile: row kappa(u, n16), dims 32kb+8g16 .. +7.
template <int D>
__device__ __forceinline__ void read_k(Tile<D> &t, const half_t *kl, int g16, int n16) {
    if constexpr (!Tile<D>::kKRegs) return;  // read per k-block inside tile_scores
    constexpr int KC = D / 8, KB = Tile<D>::KB;
    for (int u = 0; u < 2; ++u) {
        const int r = kappa(u, n16);
        for (int kb = 0; kb < KB; ++kb)
            t.k[u][kb] = *(const half8_t *)(kl + r * D + 8 * ((4 * kb + g16) ^ krow_mask<KC>(r)));
    }
}

// Issue the 8 V loads of the tile at kt into registers: lane (g16, n16) takes dims W*n16 ..
// of keys kt + 8*g16 + s (4 whole rows per instruction). vcg points at kv head g of cache row
// 0. Keys past k1 - 1 load key k1 - 1 instead.
template <int D, bool POW2, bool NT>
__device__ __forceinline__ void load_v(Tile<D> &t, const AttnArgs &a, const int32_t *bt,
                                       TileIds ids, const half_t *vcg, int kt, int k1, int g16,
                                       int n16) {
    constexpr int W = Tile<D>::W;
    const int kl = k1 - 1;
    const uint32_t ke = a.key_elems;
    const half_t *pv[8];
    if (POW2) {
        // bs is a power of two >= 8, so each aligned 8-key group lies inside one block.
        const int gv = min(kt + 8 * g16, kl & ~7);
        const half_t *bV = vcg + (size_t)ids.bv * a.block_elems + __umul24(gv & (a.bs - 1), ke);
        if (kt + kTileKeys <= k1) {
            for (int s = 0; s < 8; ++s) pv[s] = bV + (uint32_t)s * ke;
        } else {
            for (int s = 0; s < 8; ++s) pv[s] = bV + __umul24(min(kt + 8 * g16 + s, kl) - gv, ke);
        }
    } else {
        for (int s = 0; s < 8; ++s) {
            const int key = min(kt + 8 * g16 + s, kl);
            const int j = key / a.bs;
            pv[s] = vcg + (size_t)bt[j] * a.block_elems + (uint32_t)(key - j * a.bs) * ke;
        }
    }
    for (int s = 0; s < 8; ++s) {
        const half_t *p = pv[s] + W * n16;
        if constexpr (W == 16) {  // 32 bytes of the row: two 16-byte loads
            const u32x4_t x = NT ? gload_nt<u32x4_t>(p) : gload<u32x4_t>(p);
            const u32x4_t y = NT ? gload_nt<u32x4_t>(p + 8) : gload<u32x4_t>(p + 8);
            for (int c = 0; c < 4; ++c) { t.v[s][c] = x[c]; t.v[s][4 + c] = y[c]; }
        } else if constexpr (W == 8) {
            const u32x4_t x = NT ? gload_nt<u32x4_t>(p) : gload<u32x4_t>(p);
            t.v[s][0] = x[0]; t.v[s][1] = x[1]; t.v[s][2] = x[2]; t.v[s][3] = x[3];
        } else {
            const u32x2_t x = NT ? gload_nt<u32x2_t>(p) : gload<u32x2_t>(p);
            t.v[s][0] = x[0]; t.v[s][1] = x[1];
        }
    }
}

template <int D, int NCB>
struct State {
    static constexpr int KB = D / 32, W = D / 16;
    half8_t q[NCB][KB];     // B operand of S^T: column n16, dims 32kb + 8g16 .. +7
    int kend[NCB];          // per column: keys < kend are visible (0 for an unused column)
    float m[NCB];           // running max of the column (log2 units), replicated over g16
    float l[NCB];           // running sum of the lane's own keys
    float4_t o[NCB][W];     // O accumulator: rows 4g16 + j, dim W*n16 + i for MFMA i
};

// Phase 1 of a tile: S^T = K . Q^T for every column block. s[cb][u] holds, for lane
// (g16, n16), the scores of keys 8*g16 + 4u + i (i = 0..3) against column n16.
template <int D, int NCB>
__device__ __forceinline__ void tile_scores(const State<D, NCB> &st, const Tile<D> &t,
                                            float4_t (&s)[NCB][2], const half_t *kl, int g16,
                                            int n16) {
    constexpr int KB = Tile<D>::KB, KC = D / 8;
    for (int cb = 0; cb < NCB; ++cb) {
        float4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        for (int kb = 0; kb < KB; ++kb) {
            if constexpr (Tile<D>::kKRegs) {
                s0 = mfma16x16x32(t.k[0][kb], st.q[cb][kb], s0);
                s1 = mfma16x16x32(t.k[1][kb], st.q[cb][kb], s1);
            } else {
                const int r0 = kappa(0, n16), r1 = kappa(1, n16);
                const half8_t k0 =
                    *(const half8_t *)(kl + r0 * D + 8 * ((4 * kb + g16) ^ krow_mask<KC>(r0)));
                const half8_t k1 =
                    *(const half8_t *)(kl + r1 * D + 8 * ((4 * kb + g16) ^ krow_mask<KC>(r1)));
                s0 = mfma16x16x32(k0, st.q[cb][kb], s0);
                s1 = mfma16x16x32(k1, st.q[cb][kb], s1);
            }
        }
        s[cb][0] = s0;
        s[cb][1] = s1;
    }
}

// Phase 2 of a tile: V^T operands. vb[i] holds keys 8*g16 + s (s = 0..7) of dimension
// W*n16 + i, built from the lane's own 16-byte row chunks by 16-bit interleaves.
template <int D>
__device__ __forceinline__ void tile_vt(const Tile<D> &t, half8_t (&vb)[Tile<D>::W]) {
    constexpr int W = Tile<D>::W;
    for (int a2 = 0; a2 < W / 2; ++a2) {
        u32x4_t lo, hi;
        for (int k = 0; k < 4; ++k) {
            const uint32_t x = t.v[2 * k][a2], y = t.v[2 * k + 1][a2];
            lo[k] = (x & 0xffffu) | (y << 16);
            hi[k] = (x >> 16) | (y & 0xffff0000u);
        }
        vb[2 * a2] = __builtin_bit_cast(half8_t, lo);
        vb[2 * a2 + 1] = __builtin_bit_cast(half8_t, hi);
    }
}

// Phase 3 of a tile: masked online softmax of the scores and O += P . V.
template <int D, int NCB>
__device__ __forceinline__ void tile_softmax_pv(State<D, NCB> &st, const float4_t (&s)[NCB][2],
                                                const half8_t (&vb)[Tile<D>::W], int kt,
                                                float scale_log2, int g16) {
    constexpr int W = Tile<D>::W;
    for (int cb = 0; cb < NCB; ++cb) {
        const int kend = st.kend[cb];
        const int key0 = kt + 8 * g16;
        float sc[8];
        float mx = -INFINITY;
        for (int i = 0; i < 4; ++i) {
            sc[i] = (key0 + i < kend) ? s[cb][0][i] * scale_log2 : -INFINITY;
            sc[4 + i] = (key0 + 4 + i < kend) ? s[cb][1][i] * scale_log2 : -INFINITY;
            mx = fmaxf(mx, fmaxf(sc[i], sc[4 + i]));
        }
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);
        const float m_old = st.m[cb];
        const float m_new = fmaxf(m_old, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = (m_new == m_old) ? 1.f : __builtin_amdgcn_exp2f(m_old - m_use);
        half8_t pf;
        float ps = 0.f;
        for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(sc[e] - m_use);
            ps += p;
            pf[e] = (half_t)p;
        }
        st.l[cb] = st.l[cb] * alpha + ps;
        st.m[cb] = m_new;
        if (__ballot(alpha != 1.f)) {
            for (int j = 0; j < 4; ++j) {
                const float aj = __shfl(alpha, 4 * g16 + j, 64);
                for (int i = 0; i < W; ++i) st.o[cb][i][j] *= aj;
            }
        }
        for (int i = 0; i < W; ++i) st.o[cb][i] = mfma16x16x32(pf, vb[i], st.o[cb][i]);
    }
}

// Work of one (item, kv head) unit: one wave.
template <int D, int NCB, bool POW2, bool NT>
__device__ __forceinline__ void process_unit(const AttnArgs &a, const AttnItem &it, int g,
                                             int lane, half_t *kl) {
    constexpr int KB = D / 32, W = D / 16;
    const int g16 = lane >> 4, n16 = lane & 15;
    const int cu_b = it.cu0, n_b = it.n, past_b = it.past;
    const int ntok = min(a.tpi, n_b - it.t0);
    const int ncols = ntok * a.Q;

    State<D, NCB> st;
    for (int cb = 0; cb < NCB; ++cb) {
        const int col = cb * 16 + n16;
        st.m[cb] = -INFINITY;
        st.l[cb] = 0.f;
        for (int i = 0; i < W; ++i) st.o[cb][i] = float4_t{0.f, 0.f, 0.f, 0.f};
        if (col < ncols) {
            const int t = col / a.Q, qh = col - t * a.Q;
            const half_t *qp = a.query + (long long)(cu_b + it.t0 + t) * a.q_stride +
                               (long long)(g * a.Q + qh) * D + 8 * g16;
            for (int kb = 0; kb < KB; ++kb) st.q[cb][kb] = *(const half8_t *)(qp + 32 * kb);
            const int lim = a.causal ? past_b + it.t0 + t + 1 : past_b + n_b;
            st.kend[cb] = min(lim, it.k1);
        } else {
            for (int kb = 0; kb < KB; ++kb) st.q[cb][kb] = half8_t{};
            st.kend[cb] = 0;
        }
    }

    // One tile buffer: K rows in the wave's LDS tile kl, V rows in registers. In each step the
    // tile's K operands are read from LDS, its scores and V^T operands are formed, then the next
    // tile's copies and loads are issued while softmax and PV run. The last tile is peeled off
    // so the in-loop copies are unconditional. The block ids of tile t+2 are requested before
    // the copies of tile t+1, so they have arrived when those copies issue.
    const int32_t *bt = a.bt + (long long)it.b * a.MB;
    const half_t *kcg = a.kc + (size_t)(g / a.kv_div) * D;  // physical kv head
    const half_t *vcg = a.vc + (size_t)(g / a.kv_div) * D;
    if (it.k0 < it.k1) {
        Tile<D> tl;
        int kt = it.k0;
        TileIds ids2 = {0};
        if (POW2) ids2 = tile_ids(a, bt, kt, it.k1, g16);
        copy_k<D, POW2>(a, bt, ids2, kcg, kt, it.k1, lane, kl);
        load_v<D, POW2, NT>(tl, a, bt, ids2, vcg, kt, it.k1, g16, n16);
        if (POW2 && kt + kTileKeys < it.k1) ids2 = tile_ids(a, bt, kt + kTileKeys, it.k1, g16);
        for (; kt + kTileKeys < it.k1; kt += kTileKeys) {
            // the LDS copies are tracked by the vector-memory counter only: wait for all
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
            read_k<D>(tl, kl, g16, n16);
            float4_t s[NCB][2];
            tile_scores<D, NCB>(st, tl, s, kl, g16, n16);
            half8_t vb[W];
            tile_vt<D>(tl, vb);
            const int kn = kt + kTileKeys;
            TileIds ids3 = ids2;
            if (POW2 && kn + kTileKeys < it.k1) ids3 = tile_ids(a, bt, kn + kTileKeys, it.k1, g16);
            // the K operand reads are back before the next copies overwrite the tile
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
            copy_k<D, POW2>(a, bt, ids2, kcg, kn, it.k1, lane, kl);
            load_v<D, POW2, NT>(tl, a, bt, ids2, vcg, kn, it.k1, g16, n16);
            tile_softmax_pv<D, NCB>(st, s, vb, kt, a.scale_log2, g16);
            ids2 = ids3;
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        read_k<D>(tl, kl, g16, n16);
        float4_t s[NCB][2];
        tile_scores<D, NCB>(st, tl, s, kl, g16, n16);
        half8_t vb[W];
        tile_vt<D>(tl, vb);
        tile_softmax_pv<D, NCB>(st, s, vb, kt, a.scale_log2, g16);
        // the tile's LDS reads are back before another unit's copies reuse it
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    }

    // Column totals, then each lane writes rows 4*g16 + j of every column block.
    for (int cb = 0; cb < NCB; ++cb) {
        float lt = st.l[cb] + __shfl_xor(st.l[cb], 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        float lr[4], mr[4];
        for (int j = 0; j < 4; ++j) {
            lr[j] = __shfl(lt, 4 * g16 + j, 64);
            mr[j] = __shfl(st.m[cb], 4 * g16 + j, 64);
        }
        for (int j = 0; j < 4; ++j) {
            const int col = cb * 16 + 4 * g16 + j;
            if (col >= ncols) continue;
            const int t = col / a.Q, qh = col - t * a.Q;
            const int h = g * a.Q + qh;
            const long long row = cu_b + it.t0 + t;
            if (it.base < 0) {
                const float inv = 1.f / lr[j];
                half_t *op = a.out + row * (long long)a.H * D + (long long)h * D + W * n16;
                if constexpr (W == 16) {
                    half8_t r0, r1;
                    for (int i = 0; i < 8; ++i) {
                        r0[i] = (half_t)(st.o[cb][i][j] * inv);
                        r1[i] = (half_t)(st.o[cb][8 + i][j] * inv);
                    }
                    *(half8_t *)op = r0;
                    *(half8_t *)(op + 8) = r1;
                } else if constexpr (W == 8) {
                    half8_t r;
                    for (int i = 0; i < W; ++i) r[i] = (half_t)(st.o[cb][i][j] * inv);
                    *(half8_t *)op = r;
                } else {
                    half4_t r;
                    for (int i = 0; i < W; ++i) r[i] = (half_t)(st.o[cb][i][j] * inv);
                    *(half4_t *)op = r;
                }
            } else {
                const long long p =
                    (long long)(it.base + t * it.nsplit + it.split) * a.H + h;
                float *op = a.o_part + p * D + W * n16;
                for (int i = 0; i < W; i += 4)
                    *(float4_t *)(op + i) = float4_t{st.o[cb][i][j], st.o[cb][i + 1][j],
                                                     st.o[cb][i + 2][j], st.o[cb][i + 3][j]};
                if (n16 == 0) {
                    a.m_part[p] = (lr[j] > 0.f) ? mr[j] * kLn2 : kNegLarge;
                    a.l_part[p] = lr[j];
                }
            }
        }
    }
}

// The persistent loop of one decode workgroup of a.gw waves (gw divides G; gw = 1 unless
// NCB == 1), so the kv heads of one work item run side by side on one CU and read neighbouring
// rows of the same cache blocks. With a slot table (stream-K balanced decode) workgroup `block`
// processes the items of share `block`; otherwise workgroups take (item, head group) units from
// the planner's counter, longest items first (s_unit: a workgroup-shared word). kl: this wave's
// 32-key K tile in LDS ([32][D] halves).
template <int D, int NCB, bool POW2, bool NT>
__device__ __forceinline__ void decode_loop(const AttnArgs &a, int block, half_t *kl, int *s_unit) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int gblocks = a.G / a.gw;
    if (a.slot_ptr) {
        const int u0 = a.slot_ptr[block] * gblocks, u1 = a.slot_ptr[block + 1] * gblocks;
        // the share's first item comes from its own copy (requested beside the share bounds),
        // and each later unit's item is requested while the unit before it runs
        AttnItem next = a.slot_first[block];
        for (int unit = u0; unit < u1; ++unit) {
            const AttnItem it = next;
            if (unit + 1 < u1) next = a.items[(unit + 1) / gblocks];
            const int g = (unit - (unit / gblocks) * gblocks) * a.gw + wave;
            process_unit<D, NCB, POW2, NT>(a, it, g, lane, kl);
        }
        return;
    }
    const int n_work = a.n_items[0] * gblocks;
    if (n_work == 0) return;  // nothing listed: leave before touching the counter
    for (;;) {
        if (threadIdx.x == 0) *s_unit = atomicAdd(a.counter, 1);
        __syncthreads();
        const int unit = *s_unit;
        __syncthreads();
        if (unit >= n_work) break;
        const AttnItem it = a.items[unit / gblocks];
        const int g = (unit - (unit / gblocks) * gblocks) * a.gw + wave;
        process_unit<D, NCB, POW2, NT>(a, it, g, lane, kl);
    }
}

}  // namespace
}  // namespace pa
