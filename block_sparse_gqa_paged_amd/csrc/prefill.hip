// Chunked-prefill attention for gfx950: the query rows of sequences with more new tokens than a
// decode item holds. The same launch also merges the split decode partials (see prefill_kernel).
//
// Operation: the PagedAttention op of the "com.microsoft.PagedAttention ... manifest.json" page
// (pass "main") for those rows: each (token, head) column attends, through the block table, to
// keys [0, past_b + t + 1) of its sequence (causal) or to all L_b keys, with softmax over the
// scaled scores; the output row is written directly (prefill items are never split).
//
// MI355X design: the work unit is (planner item, kv head). An item is up to 128 / Q new tokens
// of one sequence, so its (token, head) columns fill four waves of 32 columns each, and the
// workgroup's four waves share every key tile:
//  * 64-key tiles of K and V are copied straight from the cache into LDS (global_load_lds,
//    16 bytes per lane: no registers, no LDS store instructions), into two stages: the next
//    tile's copies are issued right after the one barrier per tile and land while the current
//    tile is computed. The XOR swizzles of the LDS rows are applied on the source side: lane p
//    of a row copies the cache chunk that belongs at LDS chunk p.
//  * S^T = K . Q^T on v_mfma_f32_16x16x32_f16 with keys as rows (K read from LDS in the row order
//    pkappa, so each lane's accumulator holds 8 consecutive keys of one column: the k-slots of
//    the P^T operand) and O^T = V^T . P^T, whose V^T operand comes from the row-major V tile
//    through the gfx950 transposing LDS read (ds_read_b64_tr_b16: within 16 lanes, lane i gets
//    element i % 4 of the rows addressed by lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4). O^T gives
//    each lane its own column, so the softmax rescale needs no shuffles and stores are 8 bytes.
//  * Online base-2 softmax per column with a lazily raised maximum (O is rescaled only when the
//    maximum grows by more than 2^8); the column reductions use row-swap permutes, not LDS.
//    The two column blocks of a wave share each K and V read.
#include "combine_rows.h"
#include "decode_unit.h"

namespace pa {
namespace {

constexpr int kKT = 64;  // keys per tile

// Workgroup geometry by head size: each wave takes CB blocks of 16 (token, head) columns of the
// item's kPrefillCols (two at D <= 128; one at D = 256, where a second block's query and output
// registers do not fit), so a workgroup has kPrefillCols / (16 CB) waves; each wave copies KPW
// keys of every tile. Workgroups per CU follow from the LDS stages (64 KB, or 128 KB at 256).
template <int D>
struct PfShape {
    static constexpr int CB = D == 256 ? 1 : 2;
    static constexpr int COLS = 16 * CB;
    static constexpr int WAVES = kPrefillCols / COLS;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int KPW = kKT / WAVES;
    static constexpr int PER_CU = D == 256 ? 1 : 2;
};

// Key-row order inside a 32-key group: MFMA row m of 16-key half u holds key pkappa(u, m), so
// that the S^T accumulator of lane (g16, n16) holds keys 8*g16 + 4u + i: 8*g16 .. 8*g16 + 7.
__device__ __forceinline__ int pkappa(int u, int m) { return 8 * (m >> 2) + 4 * u + (m & 3); }

// XOR swizzles of the 16-byte chunks of a tile row (row = key within the tile), as masks:
// LDS chunk position p of row r holds cache chunk p ^ mask(r).
//  * K rows are read 16 at a time in the order pkappa (rows 8*(m>>2) + (m&3) + 4u): kmask gives
//    those 16 rows distinct chunk positions.
//  * V rows are read by the transposing read: per half wave, keys {b..b+3, b+8..b+11} at two
//    adjacent chunks each (32 bytes); vmask spreads those 16 chunks over all LDS banks.
template <int KC>
__device__ __forceinline__ int kmask(int r) {
    return ((r & 3) | ((r >> 1) & 12)) & (KC - 1);
}
template <int KC>
__device__ __forceinline__ int vmask(int r) {
    if (KC >= 16) return 2 * ((r & 3) | ((r >> 1) & 4));          // rows of 256 bytes or more
    return 2 * (((r >> 1) & 1) | ((r >> 2) & 2));                 // 128-byte rows: two per bank line
}

// One 16-byte global -> LDS copy per lane: lane l writes LDS bytes [16 l, 16 l + 16) of the
// wave-uniform destination dst.
__device__ __forceinline__ void dma16(const half_t *src, half_t *dst) {
    __builtin_amdgcn_global_load_lds(
        (const void __attribute__((address_space(1))) *)src,
        (void __attribute__((address_space(3))) *)dst, 16, 0, 0);
}

// Cache block of this wave's keys kt + KPW*wave .. + KPW - 1 when they all lie before k1
// in one block (block size a multiple of KPW), else -1. Wave-uniform; read one tile ahead of
// the copies that use it, so that they do not wait on the table lookup.
template <int KPW>
__device__ __forceinline__ int pf_wave_block(const AttnArgs &a, const int32_t *bt, int kt, int k1,
                                             int wave) {
    const int kw = kt + KPW * wave;
    if (a.bs % KPW != 0 || kw + KPW - 1 >= k1) return -1;
    return bt[a.log2bs >= 0 ? (kw >> a.log2bs) : kw / a.bs];
}

// Issue this wave's share of the copies of the tile at kt into the stage (Kd, Vd): keys
// kt + KPW*wave .. + KPW - 1 of K and of V; pb is pf_wave_block(kt). A copy instruction
// moves RPI whole rows (lane l: row l / KC, chunk position l % KC). Keys past k1 - 1 copy key
// k1 - 1 (masked later), so no table entry or row outside the sequence's range is read.
template <int D>
__device__ __forceinline__ void pf_copy(const AttnArgs &a, const int32_t *bt, const half_t *kcg,
                                        const half_t *vcg, int kt, int k1, int pb, half_t *Kd,
                                        half_t *Vd, int wave, int lane) {
    constexpr int KC = D / 8;          // 16-byte chunks per row
    constexpr int RPI = 64 / KC;       // rows per copy instruction
    constexpr int KPW = PfShape<D>::KPW;
    constexpr int IPW = KPW / RPI;     // copy instructions per wave and matrix
    const int pos = lane % KC, rsub = lane / KC;
    const uint32_t ke = a.key_elems;  // < 2^24 (checked on the host): 24-bit multiplies
    const int kw = kt + KPW * wave;
    const int jw = a.log2bs >= 0 ? (kw >> a.log2bs) : kw / a.bs;
    for (int t = 0; t < IPW; ++t) {
        const int r = KPW * wave + t * RPI + rsub;  // row within the tile
        size_t row;
        if (pb >= 0) {
            row = (size_t)pb * a.block_elems + __umul24(kt + r - jw * a.bs, ke);
        } else {
            const int key = min(kt + r, k1 - 1);
            const int j = a.log2bs >= 0 ? (key >> a.log2bs) : key / a.bs;
            row = (size_t)bt[j] * a.block_elems + __umul24(key - j * a.bs, ke);
        }
        const int r0 = KPW * wave + t * RPI;    // first row of this instruction
        dma16(kcg + row + 8 * (pos ^ kmask<KC>(r)), Kd + r0 * D);
        dma16(vcg + row + 8 * (pos ^ vmask<KC>(r)), Vd + r0 * D);
    }
}

// Transposing LDS read of 4 halves (ds_read_b64_tr_b16).
__device__ __forceinline__ half4_t lds_read_tr(const half_t *p) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s4 __attribute__((address_space(3))) *)p);
    return __builtin_bit_cast(half4_t, v);
}

// Reductions over the four lanes n16, n16 + 16, n16 + 32, n16 + 48 (one column of the S^T
// accumulator) with the gfx950 row-swap permutes: each swap exchanges rows between two copies of
// the value, so combining the two results gives the reduction without a trip through LDS.
__device__ __forceinline__ float col_max(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    const uint32_t v = __float_as_uint(x);
    const auto t = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float col_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const uint32_t v = __float_as_uint(x);
    const auto t = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// The running maximum of a column is raised only when a tile's maximum exceeds it by more than
// this many powers of two, so the O rescale runs rarely; P entries then stay below 2^kSlack
// (exact in fp16 range) and the final O / l does not depend on which reference maximum was used.
constexpr float kSlack = 8.f;

// One launch, two roles by workgroup index:
//  * workgroups [0, gridDim.x - pre_blocks) either merge the split decode partials (combine
//    role, at most one per CU; the decode kernel ran in the launch before), or, with
//    dec_blocks > 0, run the decode (decode role: decode_loop over dec with 4-wave
//    workgroups, each wave's 32-key K tile in the first LDS stage) beside the prefill;
//  * the other pre_blocks run the persistent prefill loop; the first static_first of them take
//    their first unit without the counter.
// The roles are independent (prefill rows are written directly, and decode and prefill items
// never share a row), so one launch serves both. The front roles come first in launch order:
// placed last, the combine would wait for the persistent prefill workgroups to leave, and the
// decode's static shares must all be resident from the start. With the decode role the grid
// holds one decode and one prefill workgroup per CU (two 4-wave workgroups fit a CU by LDS and
// registers), then prefill workgroups that only take units from the counter, which run once
// decode workgroups leave.
template <int D>
__global__ __launch_bounds__(PfShape<D>::THREADS, PfShape<D>::PER_CU) void prefill_kernel(
    AttnArgs a, CombineArgs cmb,
                                                                 int pre_blocks, AttnArgs dec,
                                                                 int dec_blocks,
                                                                 int static_first) {
    constexpr int KB = D / 32;           // 32-dim k-blocks of QK^T
    constexpr int NDT = D / 16;          // 16-dim output tiles
    constexpr int KC = D / 8;
    constexpr int CB = PfShape<D>::CB, COLS = PfShape<D>::COLS, WAVES = PfShape<D>::WAVES;
    constexpr int KPW = PfShape<D>::KPW;
    static_assert(KPW * WAVES == kKT && KPW % 8 == 0, "each wave copies whole rows");
    // Two stages of row-major K and V tiles (64 KB at D = 128: two workgroups per CU).
    __shared__ __attribute__((aligned(16))) half_t Ks[2][kKT * D];
    __shared__ __attribute__((aligned(16))) half_t Vs[2][kKT * D];
    __shared__ int s_unit;

    if ((int)blockIdx.x < (int)gridDim.x - pre_blocks) {
        if (dec_blocks > 0) {
            // decode role: dec.gw == WAVES waves, K tiles of 32 keys in the first stage (only
            // at D <= 128: the host never asks for it at 256)
            if constexpr (WAVES * kTileKeys <= 2 * kKT) {
                half_t *kl = &Ks[0][0] + (threadIdx.x >> 6) * (kTileKeys * D);
                if (dec.log2bs >= 0)
                    decode_loop<D, 1, true, true>(dec, blockIdx.x, kl, &s_unit);
                else
                    decode_loop<D, 1, false, true>(dec, blockIdx.x, kl, &s_unit);
            }
            return;
        }
        constexpr int kWg = WAVES;
        combine_dispatch<D>(cmb, 2, blockIdx.x * kWg + (threadIdx.x >> 6),
                        (gridDim.x - pre_blocks) * kWg);
        return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g16 = lane >> 4, n16 = lane & 15;
    const int n_work = a.n_items[0] * a.G;
    if (n_work == 0) return;

    // Prefill workgroup pb < static_first takes unit pb first (the planner lists the longest
    // units first): no atomic round trip and no barrier before the first unit. Every other unit
    // is static_first + k for the counter's ticket k; it starts after a barrier, so no wave
    // still reads the previous unit's LDS stage when the new unit's first copies land in it.
    const int pb = (int)blockIdx.x - ((int)gridDim.x - pre_blocks);
    for (int iter = 0;; ++iter) {
        int unit = pb;
        if (iter > 0 || pb >= static_first) {
            if (threadIdx.x == 0) s_unit = static_first + atomicAdd(a.counter, 1);
            __syncthreads();
            unit = s_unit;
            __syncthreads();
        }
        if (unit >= n_work) break;
        const AttnItem it = a.items[unit / a.G];
        const int g = unit - (unit / a.G) * a.G;
        const int cu_b = it.cu0, n_b = it.n, past_b = it.past;
        const int ntok = min(a.tpi, n_b - it.t0);
        const int ncols = ntok * a.Q;

        // Query operands and key limits of this lane's two columns 32*wave + 16*cb + n16.
        half8_t q[CB][KB];
        int kend[CB];
        float m[CB], l[CB];
        float4_t o[CB][NDT];
        int wave_end = 0, wave_min = 0x7fffffff;  // over the wave's live columns
        for (int cb = 0; cb < CB; ++cb) {
            const int col = COLS * wave + 16 * cb + n16;
            m[cb] = -INFINITY;
            l[cb] = 0.f;
            for (int dt = 0; dt < NDT; ++dt) o[cb][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
            if (col < ncols) {
                const int t = col / a.Q, qh = col - t * a.Q;
                const half_t *qp = a.query + (long long)(cu_b + it.t0 + t) * a.q_stride +
                                   (long long)(g * a.Q + qh) * D + 8 * g16;
                for (int kb = 0; kb < KB; ++kb) q[cb][kb] = gload<half8_t>(qp + 32 * kb);
                const int lim = a.causal ? past_b + it.t0 + t + 1 : past_b + n_b;
                kend[cb] = min(lim, it.k1);
                wave_end = max(wave_end, kend[cb]);
                wave_min = min(wave_min, kend[cb]);
            } else {  // no column: zero query, any limit; its result is never stored
                for (int kb = 0; kb < KB; ++kb) q[cb][kb] = half8_t{};
                kend[cb] = it.k1;
            }
        }
        for (int o2 = 32; o2 > 0; o2 >>= 1) {
            wave_end = max(wave_end, __shfl_xor(wave_end, o2, 64));
            wave_min = min(wave_min, __shfl_xor(wave_min, o2, 64));
        }

        const int32_t *bt = a.bt + (long long)it.b * a.MB;
        const half_t *kcg = a.kc + (size_t)(g / a.kv_div) * D;  // physical kv head
        const half_t *vcg = a.vc + (size_t)(g / a.kv_div) * D;
        const int k1 = it.k1;
        // Tile ti sits in stage ti & 1. At the top of each tile: wait for this wave's copies
        // (and, on the first tile, the query loads), one barrier (every wave's copies of tile ti
        // have landed, and every wave has finished tile ti - 1, whose stage the next copies
        // overwrite), then issue the copies of tile ti + 1 and compute tile ti. The barrier is a
        // bare s_barrier: a workgroup fence would also wait for the copies just issued.
        const int ntl = (k1 + kKT - 1) / kKT;
        int pbn = -1;  // pf_wave_block of the tile after the one whose copies are in flight
        if (ntl > 0) {
            pf_copy<D>(a, bt, kcg, vcg, 0, k1, pf_wave_block<KPW>(a, bt, 0, k1, wave), Ks[0], Vs[0],
                       wave, lane);
            if (ntl > 1) pbn = pf_wave_block<KPW>(a, bt, kKT, k1, wave);
        }
        for (int ti = 0; ti < ntl; ++ti) {
            const int kt = ti * kKT;
            const half_t *Kb = Ks[ti & 1], *Vb = Vs[ti & 1];
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
            asm volatile("s_barrier" ::: "memory");
            if (ti + 1 < ntl) {
                pf_copy<D>(a, bt, kcg, vcg, kt + kKT, k1, pbn, Ks[(ti + 1) & 1], Vs[(ti + 1) & 1],
                           wave, lane);
                pbn = ti + 2 < ntl ? pf_wave_block<KPW>(a, bt, kt + 2 * kKT, k1, wave) : -1;
            }
            if (kt >= wave_end) continue;  // every column of this wave ends before the tile

            // S^T: keys 32s + 8*g16 + 4u + i of columns n16 (every column block per K read).
            float sc[CB][2][2][4];
            // The score products run at raised wave priority: of the two waves sharing a SIMD,
            // the one in this phase keeps the matrix unit fed while the other runs its softmax.
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(1);
            for (int s = 0; s < 2; ++s)
                for (int u = 0; u < 2; ++u) {
                    float4_t acc[CB];
                    for (int cb = 0; cb < CB; ++cb) acc[cb] = float4_t{0.f, 0.f, 0.f, 0.f};
                    const int row = 32 * s + pkappa(u, n16);
                    for (int kb = 0; kb < KB; ++kb) {
                        const half8_t kr = *(const half8_t *)(
                            Kb + row * D + 8 * ((4 * kb + g16) ^ kmask<KC>(row)));
                        for (int cb = 0; cb < CB; ++cb)
                            acc[cb] = mfma16x16x32(kr, q[cb][kb], acc[cb]);
                    }
                    for (int cb = 0; cb < CB; ++cb)
                        for (int i = 0; i < 4; ++i) sc[cb][s][u][i] = acc[cb][i];
                }
            // Online softmax per column, P in fp16 as the B operand of O^T = V^T . P^T. Keys at or
            // past a column's limit are masked only on tiles that reach some limit; the scale
            // (> 0) is applied after the max, inside the exponent's fma.
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
            if (kt + kKT > wave_min)
                for (int cb = 0; cb < CB; ++cb)
                    for (int s = 0; s < 2; ++s)
                        for (int u = 0; u < 2; ++u)
                            for (int i = 0; i < 4; ++i)
                                if (kt + 32 * s + 8 * g16 + 4 * u + i >= kend[cb])
                                    sc[cb][s][u][i] = -INFINITY;
            half8_t pf[CB][2];
            for (int cb = 0; cb < CB; ++cb) {
                float mx = -INFINITY;
                for (int s = 0; s < 2; ++s)
                    for (int u = 0; u < 2; ++u)
                        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[cb][s][u][i]);
                const float mt = col_max(mx) * a.scale_log2;
                const bool raise = mt > m[cb] + kSlack;  // false while the whole tile is masked
                const float m_new = raise ? mt : m[cb];
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = raise ? __builtin_amdgcn_exp2f(m[cb] - m_use) : 1.f;
                float ps = 0.f;
                for (int s = 0; s < 2; ++s)
                    for (int u = 0; u < 2; ++u)
                        for (int i = 0; i < 4; ++i) {
                            const float p = __builtin_amdgcn_exp2f(
                                __builtin_fmaf(sc[cb][s][u][i], a.scale_log2, -m_use));
                            ps += p;
                            pf[cb][s][4 * u + i] = (half_t)p;
                        }
                l[cb] = l[cb] * alpha + ps;
                m[cb] = m_new;
                // O^T columns are this lane's own column: rescale in place
                if (__ballot(raise))
                    for (int dt = 0; dt < NDT; ++dt) o[cb][dt] *= alpha;
            }
            // O^T += V^T . P^T: A operand = keys 32s + 8*g16 + 0..7 of dim 16*dt + n16, two
            // transposing reads of 4 keys (lane r of a 16-lane group addresses key kb + r/4,
            // dims 16*dt + 4*(r%4) .. +3); the accumulator holds dims 16*dt + 4*g16 + i of column n16.
            // Each operand is read two output tiles ahead of its products.
            const int csub = (n16 & 3) >> 1, hoff = 4 * (n16 & 1);
            auto vop = [&](int s, int dt) {
                const int k0 = 32 * s + 8 * g16 + (n16 >> 2), k4 = k0 + 4;
                const int c = 2 * dt + csub;
                const half4_t lo = lds_read_tr(Vb + k0 * D + 8 * (c ^ vmask<KC>(k0)) + hoff);
                const half4_t hi = lds_read_tr(Vb + k4 * D + 8 * (c ^ vmask<KC>(k4)) + hoff);
                return half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            };
            half8_t va = vop(0, 0), vbn = vop(0, 1);
            for (int x = 0; x < 2 * NDT; ++x) {
                const int s = x / NDT, dt = x % NDT;
                const half8_t vb = va;
                va = vbn;
                if (x + 2 < 2 * NDT) vbn = vop((x + 2) / NDT, (x + 2) % NDT);
                for (int cb = 0; cb < CB; ++cb)
                    o[cb][dt] = mfma16x16x32(vb, pf[cb][s], o[cb][dt]);
            }
        }

        // Output. Lane (g16, n16) holds dims 16*dt + 4*g16 .. +3 of its columns; stored
        // directly, each instruction would write 8 bytes into 16 columns. The wave's COLS
        // columns go instead through its own part of the LDS stage the last tile did not use
        // (every wave finished the tile before it at the last barrier; the next unit's first
        // copies land only after the next unit's barriers; the waves' parts run through that
        // stage's K then V tile), XOR-swizzled by column, and leave as whole columns:
        // 64*16/(2D) columns per store instruction, a token's Q heads contiguous.
        constexpr int CPL = D / 8;  // 16-byte chunks per column
        static_assert(WAVES * COLS * D <= 2 * kKT * D, "the output columns fit one stage");
        const int ooff = wave * COLS * D;
        half_t *ost = ooff < kKT * D ? Ks[ntl & 1] + ooff : Vs[ntl & 1] + (ooff - kKT * D);
        for (int cb = 0; cb < CB; ++cb) {
            const float lt = col_sum(l[cb]);
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            const int lc = 16 * cb + n16;
            for (int dt = 0; dt < NDT; ++dt) {
                half4_t r;
                for (int i = 0; i < 4; ++i) r[i] = (half_t)(o[cb][dt][i] * inv);
                const int ch = 2 * dt + (g16 >> 1);
                *(half4_t *)(ost + lc * D + 8 * (ch ^ (lc & (CPL - 1))) + 4 * (g16 & 1)) = r;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll 4
        for (int j = 0; j < COLS * CPL / 64; ++j) {
            const int lc = (64 / CPL) * j + lane / CPL, ch = lane % CPL;
            const half8_t v = *(const half8_t *)(ost + lc * D + 8 * (ch ^ (lc & (CPL - 1))));
            const int col = COLS * wave + lc;
            if (col < ncols) {
                const int t = col / a.Q, qh = col - t * a.Q;
                half_t *dst = a.out + (long long)(cu_b + it.t0 + t) * a.H * D +
                              (long long)(g * a.Q + qh) * D + 8 * ch;
                __builtin_nontemporal_store(v, (half8_t *)dst);  // written once
            }
        }
    }
}

}  // namespace

pa_status launch_prefill(const AttnArgs &a, int D, int blocks, const CombineArgs *cmb,
                         int max_groups, hipStream_t stream) {
    LaunchScope scope("prefill_combine", stream);
    int comb_blocks = 0;
    CombineArgs c{};
    if (cmb && max_groups > 0) {
        c = *cmb;
        // At most one combine workgroup per CU: max_groups is a bound (every row split); the
        // waves loop when more rows are split than they cover in one pass.
        const int waves = D == 256 ? PfShape<256>::WAVES : PfShape<128>::WAVES;
        comb_blocks = (int)std::min<long long>(
            (combine_waves(max_groups, c.lanes, D) + waves - 1) / waves, device_cu_count());
    }
    const int grid = blocks + comb_blocks;
    if (grid <= 0) return PA_OK;
    const AttnArgs none{};
    if (D == 256)
        scope.launch(prefill_kernel<256>, dim3(grid), dim3(PfShape<256>::THREADS), 0, a, c,
                     blocks, none, 0, blocks);
    else if (D == 128)
        scope.launch(prefill_kernel<128>, dim3(grid), dim3(PfShape<128>::THREADS), 0, a, c,
                     blocks, none, 0, blocks);
    else if (D == 64)
        scope.launch(prefill_kernel<64>, dim3(grid), dim3(PfShape<64>::THREADS), 0, a, c, blocks,
                     none, 0, blocks);
    else
        return PA_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status launch_decode_prefill(const AttnArgs &dec, const AttnArgs &pre, int D, int dec_blocks,
                                int pre_static, int pre_blocks, hipStream_t stream) {
    LaunchScope scope("decode_prefill", stream);
    if ((D != 64 && D != 128) || dec.gw != PfShape<128>::WAVES || pre_static > pre_blocks ||
        dec_blocks < 0)
        return PA_ERR_UNSUPPORTED;
    const int grid = dec_blocks + pre_blocks;
    if (grid <= 0) return PA_OK;
    const CombineArgs c{};
    if (D == 128)
        scope.launch(prefill_kernel<128>, dim3(grid), dim3(PfShape<128>::THREADS), 0, pre, c,
                     pre_blocks, dec, dec_blocks, pre_static);
    else if (D == 64)
        scope.launch(prefill_kernel<64>, dim3(grid), dim3(PfShape<64>::THREADS), 0, pre, c,
                     pre_blocks, dec, dec_blocks, pre_static);
    else
        return PA_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
