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
//  * 64-key tiles of K (row-major) and V (transposed) are staged in LDS as fp16, once per
//    workgroup; the next tile's global loads are issued before the current tile is computed,
//    and the block-table entries they need are read one tile earlier still.
//  * S^T = K . Q^T on v_mfma_f32_16x16x32_f16 with keys as rows (K read from LDS in the row order
//    pkappa, so each lane's accumulator holds 8 consecutive keys of one column: the k-slots of
//    the P^T operand) and O^T = V^T . P^T with V^T rows read as 16-byte operands. O^T gives each
//    lane its own column, so the softmax rescale needs no shuffles and stores are 8 bytes wide.
//  * Online base-2 softmax per column with a lazily raised maximum (O is rescaled only when the
//    maximum grows by more than 2^8); the column reductions use row-swap permutes, not LDS.
//    The two column blocks of a wave share each K and V read.
#include "combine_rows.h"

namespace pa {
namespace {

constexpr int kPfThreads = 256;  // four waves
constexpr int kKT = 64;          // keys per tile

// Key-row order inside a 32-key group: MFMA row m of 16-key half u holds key pkappa(u, m), so
// that the S^T accumulator of lane (g16, n16) holds keys 8*g16 + 4u + i: 8*g16 .. 8*g16 + 7.
__device__ __forceinline__ int pkappa(int u, int m) { return 8 * (m >> 2) + 4 * u + (m & 3); }

// XOR swizzles of 16-byte chunks. K rows are read 16 at a time in the order pkappa (rows
// 8*(m>>2) + (m&3) + 4u): kswz gives those 16 rows distinct chunk offsets. V^T rows are read as
// 16 consecutive rows (two per 256-byte bank line) and written as 16 rows 8 apart: vswz spreads
// both patterns.
template <int KC>
__device__ __forceinline__ int kswz(int row, int c) {
    return c ^ (((row & 3) | ((row >> 1) & 12)) & (KC - 1));
}
__device__ __forceinline__ int vswz(int d, int c) { return c ^ (((d >> 1) ^ (d >> 4)) & 7); }

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

template <int D>
struct PfTile {            // one thread's share of a tile: 4 consecutive keys x 8 dims, K and V
    half8_t k[4], v[4];
};

// Physical block of keys k4 .. k4 + 3 when the four share one block and all lie before k1, else
// -1 (the per-key path below). Loaded one tile ahead, so that the next tile's key and value loads
// do not wait on the table lookup.
__device__ __forceinline__ int pf_block(const AttnArgs &a, const int32_t *bt, int k4, int k1) {
    if ((a.bs & 3) == 0 && k4 + 3 < k1) {
        const int j = a.log2bs >= 0 ? (k4 >> a.log2bs) : k4 / a.bs;
        return bt[j];
    }
    return -1;
}

// Global loads of this thread's part of the tile holding keys k4 .. k4 + 3 (k4 = kt + 4*kq),
// dims 8*c .. +7; pb is pf_block(k4). Keys past k1 - 1 load key k1 - 1 (masked later), so no
// table entry or row outside the sequence's range is read.
template <int D>
__device__ __forceinline__ void pf_load(PfTile<D> &t, const AttnArgs &a, const int32_t *bt,
                                        const half_t *kcg, const half_t *vcg, int pb, int k4,
                                        int k1, int c) {
    const uint32_t ke = a.key_elems;  // < 2^24 (checked on the host): 24-bit multiplies
    if (pb >= 0) {
        const int j = a.log2bs >= 0 ? (k4 >> a.log2bs) : k4 / a.bs;
        const size_t off = (size_t)pb * a.block_elems + __umul24(k4 - j * a.bs, ke) + 8 * c;
        for (int r = 0; r < 4; ++r) {
            t.k[r] = gload<half8_t>(kcg + off + __umul24(r, ke));
            t.v[r] = gload<half8_t>(vcg + off + __umul24(r, ke));
        }
        return;
    }
    for (int r = 0; r < 4; ++r) {
        const int key = min(k4 + r, k1 - 1);
        const int j = a.log2bs >= 0 ? (key >> a.log2bs) : key / a.bs;
        const size_t off = (size_t)bt[j] * a.block_elems + __umul24(key - j * a.bs, ke) + 8 * c;
        t.k[r] = gload<half8_t>(kcg + off);
        t.v[r] = gload<half8_t>(vcg + off);
    }
}

// Store the thread's part into LDS: K rows [kKT][D] and V^T rows [D][kKT], both with 16-byte
// chunks XOR-swizzled by row.
template <int D>
__device__ __forceinline__ void pf_store(const PfTile<D> &t, half_t *Ks, half_t *Vt, int kq,
                                         int c) {
    constexpr int KC = D / 8;     // 16-byte chunks per K row
    static_assert(kKT / 8 == 8, "vswz assumes 8 chunks per V^T row");
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * kq + r;
        *(half8_t *)(Ks + row * D + 8 * kswz<KC>(row, c)) = t.k[r];
    }
    for (int x = 0; x < 8; ++x) {
        const int d = 8 * c + x;
        const half4_t q4 = {t.v[0][x], t.v[1][x], t.v[2][x], t.v[3][x]};
        *(half4_t *)(Vt + d * kKT + 8 * vswz(d, kq >> 1) + 4 * (kq & 1)) = q4;
    }
}

// The launch after the decode kernel: the first gridDim.x - pre_blocks workgroups merge the
// split decode partials (combine role, at most one per CU), the other pre_blocks run the
// persistent prefill loop. The two roles are independent (prefill rows are written directly),
// so one launch serves both and the step has one launch fewer. The combine workgroups come
// first: placed last they would wait for the persistent prefill workgroups to leave.
template <int D>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_kernel(AttnArgs a, CombineArgs cmb,
                                                                 int pre_blocks) {
    constexpr int KB = D / 32;           // 32-dim k-blocks of QK^T
    constexpr int NDT = D / 16;          // 16-dim output tiles
    constexpr int KC = D / 8;
    constexpr int TASKS = kKT / 4 * KC;  // (key quad, 8-dim chunk) pairs per tile
    static_assert(TASKS <= kPfThreads, "one load task per thread");
    __shared__ __attribute__((aligned(16))) half_t Ks[kKT * D];
    __shared__ __attribute__((aligned(16))) half_t Vt[D * kKT];
    __shared__ int s_unit;

    if ((int)blockIdx.x < (int)gridDim.x - pre_blocks) {
        constexpr int kWg = kPfThreads / 64;
        combine_rows<D>(cmb, 2, blockIdx.x * kWg + (threadIdx.x >> 6),
                        (gridDim.x - pre_blocks) * kWg);
        return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g16 = lane >> 4, n16 = lane & 15;
    const bool loader = TASKS == kPfThreads || threadIdx.x < TASKS;
    const int kq = threadIdx.x / KC, c = threadIdx.x % KC;
    const int n_work = a.n_items[0] * a.G;
    if (n_work == 0) return;

    for (;;) {
        if (threadIdx.x == 0) s_unit = atomicAdd(a.counter, 1);
        __syncthreads();
        const int unit = s_unit;
        __syncthreads();
        if (unit >= n_work) break;
        const AttnItem it = a.items[unit / a.G];
        const int g = unit - (unit / a.G) * a.G;
        const int cu_b = a.cu[it.b];
        const int n_b = a.cu[it.b + 1] - cu_b;
        const int past_b = a.past[it.b];
        const int ntok = min(a.tpi, n_b - it.t0);
        const int ncols = ntok * a.Q;

        // Query operands and key limits of this lane's two columns 32*wave + 16*cb + n16.
        half8_t q[2][KB];
        int kend[2];
        float m[2], l[2];
        float4_t o[2][NDT];
        int wave_end = 0, wave_min = 0x7fffffff;  // over the wave's live columns
        for (int cb = 0; cb < 2; ++cb) {
            const int col = 32 * wave + 16 * cb + n16;
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
        const half_t *kcg = a.kc + (size_t)g * D;
        const half_t *vcg = a.vc + (size_t)g * D;
        const int k1 = it.k1;
        PfTile<D> tl;
        int pbn = -1;  // pf_block of this thread's keys in the tile after the one in flight
        if (loader && k1 > 0) {
            pf_load<D>(tl, a, bt, kcg, vcg, pf_block(a, bt, 4 * kq, k1), 4 * kq, k1, c);
            if (kKT < k1) pbn = pf_block(a, bt, kKT + 4 * kq, k1);
        }
        // Drain the query and first-tile loads here. Without this wait the compiler treats the
        // query registers as possibly in flight inside the tile loop, and since the vector-memory
        // counter retires in order, its wait before the first score product would also cover the
        // next tile's prefetch.
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        for (int kt = 0; kt < k1; kt += kKT) {
            __syncthreads();  // every wave is done with the previous tile
            if (loader) pf_store<D>(tl, Ks, Vt, kq, c);
            __syncthreads();
            if (loader && kt + kKT < k1) {
                pf_load<D>(tl, a, bt, kcg, vcg, pbn, kt + kKT + 4 * kq, k1, c);
                pbn = kt + 2 * kKT < k1 ? pf_block(a, bt, kt + 2 * kKT + 4 * kq, k1) : -1;
            }
            if (kt >= wave_end) continue;  // every column of this wave ends before the tile

            // S^T: keys 32s + 8*g16 + 4u + i of columns n16 (both column blocks per K read).
            float sc[2][2][2][4];
            for (int s = 0; s < 2; ++s)
                for (int u = 0; u < 2; ++u) {
                    float4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
                    const int row = 32 * s + pkappa(u, n16);
                    for (int kb = 0; kb < KB; ++kb) {
                        const half8_t kr =
                            *(const half8_t *)(Ks + row * D + 8 * kswz<KC>(row, 4 * kb + g16));
                        acc[0] = mfma16x16x32(kr, q[0][kb], acc[0]);
                        acc[1] = mfma16x16x32(kr, q[1][kb], acc[1]);
                    }
                    for (int cb = 0; cb < 2; ++cb)
                        for (int i = 0; i < 4; ++i) sc[cb][s][u][i] = acc[cb][i];
                }
            // Online softmax per column, P in fp16 as the B operand of O^T = V^T . P^T. Keys at or
            // past a column's limit are masked only on tiles that reach some limit; the scale
            // (> 0) is applied after the max, inside the exponent's fma.
            if (kt + kKT > wave_min)
                for (int cb = 0; cb < 2; ++cb)
                    for (int s = 0; s < 2; ++s)
                        for (int u = 0; u < 2; ++u)
                            for (int i = 0; i < 4; ++i)
                                if (kt + 32 * s + 8 * g16 + 4 * u + i >= kend[cb])
                                    sc[cb][s][u][i] = -INFINITY;
            half8_t pf[2][2];
            for (int cb = 0; cb < 2; ++cb) {
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
            // O^T += V^T . P^T: A operand = 8 keys of dim 16*dt + n16 from a V^T row; the
            // accumulator holds dims 16*dt + 4*g16 + i of column n16.
            for (int s = 0; s < 2; ++s)
                for (int dt = 0; dt < NDT; ++dt) {
                    const int d = 16 * dt + n16;
                    const half8_t vb =
                        *(const half8_t *)(Vt + d * kKT + 8 * vswz(d, 4 * s + g16));
                    o[0][dt] = mfma16x16x32(vb, pf[0][s], o[0][dt]);
                    o[1][dt] = mfma16x16x32(vb, pf[1][s], o[1][dt]);
                }
        }

        // Column totals; lane (g16, n16) writes dims 16*dt + 4*g16 .. +3 of column n16.
        for (int cb = 0; cb < 2; ++cb) {
            const float lt = col_sum(l[cb]);
            const int col = 32 * wave + 16 * cb + n16;
            if (col >= ncols) continue;
            const int t = col / a.Q, qh = col - t * a.Q;
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            half_t *op = a.out + (long long)(cu_b + it.t0 + t) * a.H * D +
                         (long long)(g * a.Q + qh) * D + 4 * g16;
            for (int dt = 0; dt < NDT; ++dt) {
                half4_t r;
                for (int i = 0; i < 4; ++i) r[i] = (half_t)(o[cb][dt][i] * inv);
                *(half4_t *)(op + 16 * dt) = r;
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
        comb_blocks = (int)std::min<long long>((combine_waves(max_groups, c.lanes, D) + 3) / 4,
                                               device_cu_count());
    }
    const int grid = blocks + comb_blocks;
    if (grid <= 0) return PA_OK;
    if (D == 128)
        scope.launch(prefill_kernel<128>, dim3(grid), dim3(kPfThreads), 0, a, c, blocks);
    else if (D == 64)
        scope.launch(prefill_kernel<64>, dim3(grid), dim3(kPfThreads), 0, a, c, blocks);
    else
        return PA_ERR_UNSUPPORTED;
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
