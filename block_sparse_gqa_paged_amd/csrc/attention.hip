// Paged GQA attention for gfx950: the device planner and the MFMA attention kernel.
//
// Operation: the PagedAttention op of the "com.microsoft.PagedAttention ... manifest.json" page
// (passes "main", "split_attention" and "merge"): every query row attends, per kv head, to the
// keys of its sequence that a block table maps into an fp16 cache [NB, bs, G, D]; the key range
// may be cut into chunks whose (o, m, l) partials a log-sum-exp merge combines.
//
// MI355X design (not the page's WebGPU one):
//  * One wave64 per (work item, kv head). A work item is a sequence's query rows (all of them for
//    a decode-like sequence, a 64-column tile for a prefill sequence) and a key chunk. The wave
//    serves every query head of the kv group, so each K/V byte of the chunk is read from HBM
//    once per work item.
//  * QK^T and PV run on MFMA v_mfma_f32_16x16x32_f16. The score tile is S^T = K . Q^T with
//    16 keys as rows and 16 (token, head) columns: K rows load straight from the cache as the A
//    operand (16 contiguous bytes per lane), so no LDS is needed. The tile's C layout already
//    gives each lane 8 keys of one column, exactly the k-slots of the P operand of O = P . V.
//    The V operand wants 8 keys of one dimension per lane; V is loaded as 16-byte row chunks
//    (fully coalesced, 4 rows per load) and transposed in registers with byte permutes.
//  * Online softmax in base 2 (scores pre-multiplied by scale*log2 e); the stored partial max is
//    converted back to natural-log units. Column max/sum reductions are two cross-row shuffles.
//  * A persistent grid walks the planner's item list; the planner (one workgroup) reads the
//    sequence lengths on the device and picks the chunk size, so the host never waits on data.
#include "common.h"

#include <math.h>

namespace pa {

// ============================================================================================
// Device planner
// ============================================================================================
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kTileKeys = 32;

__device__ __forceinline__ long long block_sum_ll(long long v, long long *sh) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if (lane == 0) sh[wid] = v;
    __syncthreads();
    long long t = 0;
    for (int i = 0; i < kPlanThreads / 64; ++i) t += sh[i];
    return t;
}

__device__ __forceinline__ int block_max_i(int v, long long *sh) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    __syncthreads();
    if (lane == 0) sh[wid] = v;
    __syncthreads();
    int t = 0;
    for (int i = 0; i < kPlanThreads / 64; ++i) t = max(t, (int)sh[i]);
    return t;
}

// Exclusive scan of four counters across the workgroup; returns totals in tot[].
__device__ __forceinline__ void block_scan4(int v[4], int excl[4], int tot[4], int *sh) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int inc[4];
    for (int k = 0; k < 4; ++k) {
        int x = v[k];
        for (int o = 1; o < 64; o <<= 1) {
            int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        inc[k] = x;
    }
    __syncthreads();
    if (lane == 63)
        for (int k = 0; k < 4; ++k) sh[wid * 4 + k] = inc[k];
    __syncthreads();
    for (int k = 0; k < 4; ++k) {
        int before = 0, all = 0;
        for (int i = 0; i < kPlanThreads / 64; ++i) {
            const int s = sh[i * 4 + k];
            if (i < wid) before += s;
            all += s;
        }
        excl[k] = before + inc[k] - v[k];
        tot[k] = all;
    }
}

__device__ __forceinline__ int ceil_div_i(long long a, long long b) { return (int)((a + b - 1) / b); }

__device__ __forceinline__ int chunk_of(int mode, int C, int S, int L) {
    if (mode == 0) return C;
    const int per = ceil_div_i(L, S);
    return ((per + kTileKeys - 1) / kTileKeys) * kTileKeys;
}

}  // namespace

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
    __shared__ long long sh_ll[kPlanThreads / 64];
    __shared__ int sh_i[kPlanThreads / 64 * 4];
    const int tid = threadIdx.x;

    // Pass 1: decode-like sequences (1 <= n_b <= tpi_dec): count and longest key range.
    int ndec = 0, maxL = 0;
    for (int b = tid; b < a.B; b += kPlanThreads) {
        const int n = a.cu[b + 1] - a.cu[b];
        if (n >= 1 && n <= a.tpi_dec) {
            ++ndec;
            maxL = max(maxL, a.past[b] + n);
        }
    }
    ndec = (int)block_sum_ll(ndec, sh_ll);
    maxL = block_max_i(maxL, sh_ll);

    // Auto mode: smallest chunk (multiple of 32, >= min_chunk) whose item count fits the target.
    int C = max(kTileKeys, ((maxL + kTileKeys - 1) / kTileKeys) * kTileKeys);
    if (a.mode == 0 && ndec > 0) {
        const long long want = max((long long)ndec, (long long)max(1, a.target_units / a.G));
        int lo = max(1, (a.min_chunk + kTileKeys - 1) / kTileKeys), hi = C / kTileKeys;
        if (lo > hi) lo = hi;
        while (lo < hi) {  // smallest k in [lo, hi] with items(32k) <= want
            const int mid = (lo + hi) / 2;
            const int Cm = mid * kTileKeys;
            long long items = 0;
            for (int b = tid; b < a.B; b += kPlanThreads) {
                const int n = a.cu[b + 1] - a.cu[b];
                if (n >= 1 && n <= a.tpi_dec) items += ceil_div_i(a.past[b] + n, Cm);
            }
            items = block_sum_ll(items, sh_ll);
            if (items <= want) hi = mid; else lo = mid + 1;
        }
        C = lo * kTileKeys;
    }

    // Pass 2: per-sequence counts, exclusive scans, item lists.
    int carry[4] = {0, 0, 0, 0};  // dec items, partial units, combine rows, prefill items
    for (int base = 0; base < a.B; base += kPlanThreads) {
        const int b = base + tid;
        int cnt[4] = {0, 0, 0, 0};
        int n = 0, L = 0, Cb = 0, c = 0, past = 0, cu0 = 0;
        if (b < a.B) {
            cu0 = a.cu[b];
            n = a.cu[b + 1] - cu0;
            past = a.past[b];
            L = past + n;
            if (n >= 1 && n <= a.tpi_dec) {
                Cb = chunk_of(a.mode, C, a.splits, L);
                c = ceil_div_i(L, Cb);
                cnt[0] = c;
                if (c >= 2) {
                    cnt[1] = n * c;
                    cnt[2] = n;
                }
            } else if (n > a.tpi_dec) {
                cnt[3] = ceil_div_i(n, a.tpi_pre);
            }
        }
        int ex[4], tot[4];
        block_scan4(cnt, ex, tot, sh_i);
        if (b < a.B) {
            const int ubase = carry[1] + ex[1];
            for (int s = 0; s < cnt[0]; ++s) {
                const int idx = carry[0] + ex[0] + s;
                if (idx < a.cap_dec) {
                    AttnItem it;
                    it.b = b; it.t0 = 0; it.k0 = s * Cb; it.k1 = min(L, (s + 1) * Cb);
                    it.base = c >= 2 ? ubase : -1; it.nsplit = c; it.split = s; it.pad = 0;
                    a.dec[idx] = it;
                }
            }
            for (int t = 0; t < cnt[2]; ++t) {
                const int idx = carry[2] + ex[2] + t;
                if (idx < a.cap_comb) {
                    CombItem ci;
                    ci.row = cu0 + t; ci.e0 = ubase + t * c; ci.count = c; ci.pad = 0;
                    a.comb[idx] = ci;
                }
            }
            for (int j = 0; j < cnt[3]; ++j) {
                const int idx = carry[3] + ex[3] + j;
                if (idx < a.cap_pre) {
                    const int tlast = min(n, (j + 1) * a.tpi_pre) - 1;
                    AttnItem it;
                    it.b = b; it.t0 = j * a.tpi_pre; it.k0 = 0;
                    it.k1 = a.causal ? past + tlast + 1 : L;
                    it.base = -1; it.nsplit = 1; it.split = 0; it.pad = 0;
                    a.pre[idx] = it;
                }
            }
        }
        for (int k = 0; k < 4; ++k) carry[k] += tot[k];
    }
    if (tid == 0) {
        a.hdr->n_dec = min(carry[0], a.cap_dec);
        a.hdr->units = carry[1];
        a.hdr->n_comb = min(carry[2], a.cap_comb);
        a.hdr->n_pre = min(carry[3], a.cap_pre);
        a.hdr->chunk = C;
    }
}

pa_status launch_plan(const PlanArgs &a, hipStream_t stream) {
    LaunchScope scope("plan", stream);
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// ============================================================================================
// Attention kernel
// ============================================================================================
namespace {

// Key-row order inside a 32-key tile. MFMA row m of 16-key half u holds key kappa(u, m); the
// choice puts, in the S^T accumulator of lane (g16, n16), keys 8*g16 + 4u + i (i = 0..3), i.e.
// the 8 consecutive keys 8*g16 .. 8*g16 + 7 that the P operand of lane (g16, n16) needs.
__device__ __forceinline__ int kappa(int u, int m) { return 8 * (m >> 2) + 4 * u + (m & 3); }

template <int D>
struct Tile {
    static constexpr int KB = D / 32;  // 32-dim k-blocks of QK^T
    static constexpr int W = D / 16;   // dims per lane of the V layout (D = 16 * W)
    half8_t k[2][KB];                  // A operand rows: keys kappa(u, n16), dims 32kb+8g16..+7
    uint32_t v[8][W / 2];              // keys 8*g16 + s, dims W*n16 .. W*n16 + W - 1
};

template <int D, bool POW2>
__device__ __forceinline__ void load_tile(Tile<D> &t, const AttnArgs &a, int b, int g, int kt,
                                          int k1, int g16, int n16) {
    constexpr int KB = Tile<D>::KB, W = Tile<D>::W;
    const int32_t *bt = a.bt + (long long)b * a.MB;
    const int kl = k1 - 1;
    size_t rowK[2], rowV[8];
    if (POW2) {
        // bs is a power of two >= 8, so each aligned 8-key group lies inside one block.
        const int lastg = kl & ~7;
        const int gk = min(kt + 8 * (n16 >> 2), lastg);
        const int gv = min(kt + 8 * g16, lastg);
        const int bk = bt[gk >> a.log2bs];
        const int bv = bt[gv >> a.log2bs];
        const int mask = a.bs - 1;
        for (int u = 0; u < 2; ++u) {
            const int key = min(kt + kappa(u, n16), kl);
            rowK[u] = ((size_t)bk * a.bs + (gk & mask) + (key - gk)) * a.G + g;
        }
        for (int s = 0; s < 8; ++s) {
            const int key = min(kt + 8 * g16 + s, kl);
            rowV[s] = ((size_t)bv * a.bs + (gv & mask) + (key - gv)) * a.G + g;
        }
    } else {
        for (int u = 0; u < 2; ++u) {
            const int key = min(kt + kappa(u, n16), kl);
            const int j = key / a.bs;
            rowK[u] = ((size_t)bt[j] * a.bs + (key - j * a.bs)) * a.G + g;
        }
        for (int s = 0; s < 8; ++s) {
            const int key = min(kt + 8 * g16 + s, kl);
            const int j = key / a.bs;
            rowV[s] = ((size_t)bt[j] * a.bs + (key - j * a.bs)) * a.G + g;
        }
    }
    for (int u = 0; u < 2; ++u) {
        const half_t *p = a.kc + rowK[u] * D + 8 * g16;
        for (int kb = 0; kb < KB; ++kb) t.k[u][kb] = *(const half8_t *)(p + 32 * kb);
    }
    for (int s = 0; s < 8; ++s) {
        const half_t *p = a.vc + rowV[s] * D + W * n16;
        if constexpr (W == 8) {
            const u32x4_t x = *(const u32x4_t *)p;
            t.v[s][0] = x[0]; t.v[s][1] = x[1]; t.v[s][2] = x[2]; t.v[s][3] = x[3];
        } else {
            const u32x2_t x = *(const u32x2_t *)p;
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
                                            float4_t (&s)[NCB][2]) {
    constexpr int KB = Tile<D>::KB;
    for (int cb = 0; cb < NCB; ++cb) {
        float4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
        for (int kb = 0; kb < KB; ++kb) {
            s0 = mfma16x16x32(t.k[0][kb], st.q[cb][kb], s0);
            s1 = mfma16x16x32(t.k[1][kb], st.q[cb][kb], s1);
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

template <int D, int NCB, bool POW2>
__global__ __launch_bounds__(64) void attn_kernel(AttnArgs a) {
    constexpr int KB = D / 32, W = D / 16;
    const int lane = threadIdx.x;
    const int g16 = lane >> 4, n16 = lane & 15;
    const int n_work = a.n_items[0] * a.G;
    for (int w = blockIdx.x; w < n_work; w += gridDim.x) {
        const AttnItem it = a.items[w / a.G];
        const int g = w - (w / a.G) * a.G;
        const int cu_b = a.cu[it.b];
        const int n_b = a.cu[it.b + 1] - cu_b;
        const int past_b = a.past[it.b];
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

        // One tile buffer: the tile's scores and V^T operands are formed first, then the next
        // tile's loads reuse its registers while the softmax and PV of this tile run.
        Tile<D> tl;
        int kt = it.k0;
        if (kt < it.k1) load_tile<D, POW2>(tl, a, it.b, g, kt, it.k1, g16, n16);
        while (kt < it.k1) {
            float4_t s[NCB][2];
            tile_scores<D, NCB>(st, tl, s);
            half8_t vb[W];
            tile_vt<D>(tl, vb);
            const int kn = kt + kTileKeys;
            if (kn < it.k1) load_tile<D, POW2>(tl, a, it.b, g, kn, it.k1, g16, n16);
            tile_softmax_pv<D, NCB>(st, s, vb, kt, a.scale_log2, g16);
            kt = kn;
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
                    if constexpr (W == 8) {
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
}

template <int D, int NCB>
pa_status launch_d_ncb(const AttnArgs &a, int grid, hipStream_t stream) {
    if (a.log2bs >= 0)
        hipLaunchKernelGGL((attn_kernel<D, NCB, true>), dim3(grid), dim3(64), 0, stream, a);
    else
        hipLaunchKernelGGL((attn_kernel<D, NCB, false>), dim3(grid), dim3(64), 0, stream, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

template <int D>
pa_status launch_d(const AttnArgs &a, int ncb, int grid, hipStream_t stream) {
    switch (ncb) {
        case 1: return launch_d_ncb<D, 1>(a, grid, stream);
        case 2: return launch_d_ncb<D, 2>(a, grid, stream);
        case 4: return launch_d_ncb<D, 4>(a, grid, stream);
        default: return PA_ERR_UNSUPPORTED;
    }
}

}  // namespace

pa_status launch_attention(const AttnArgs &a, int D, int ncb, int grid, const char *name,
                           hipStream_t stream) {
    LaunchScope scope(name, stream);
    if (grid <= 0) return PA_OK;
    switch (D) {
        case 64: return launch_d<64>(a, ncb, grid, stream);
        case 128: return launch_d<128>(a, ncb, grid, stream);
        default: return PA_ERR_UNSUPPORTED;
    }
}

}  // namespace pa
