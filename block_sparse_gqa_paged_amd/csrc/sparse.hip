// Block-sparse "edge" forward in fp32 for gfx950, KV-outer.
//
// Operation: sparse_forward of the "alice-llm ... sparse_attention_forward.wgsl" page. Edge
// e = (q_idx, h, blk, batch, block_len); for each q-head lane qh it scores the query row
// (q_idx, h*qhead + qh) against keys t < block_len of block blk (pages through the batch's
// table row; unmapped pages contribute nothing), and writes the block-local, unnormalised
// (o, m, l) at p = e*qhead + qh. block_len <= 0, or no mapped key, gives o = 0, m = -1e30, l = 0.
//
// MI355X design: edges are grouped by their (batch, h, blk) key block with a counting sort on
// the device (histogram, scan, scatter into a workspace permutation), so one workgroup stages a
// key block (K row-major, V transposed, both fp32) in LDS once and reuses it for up to kChunk
// edges. Four waves each take 16 query rows (16 / qhead edges) at a time; S^T = K . Q^T and
// O = P . V run on v_mfma_f32_16x16x4_f32. The S^T accumulator gives each lane 4 keys of one
// query row, which are exactly its A-operand k-slots for the PV product, so P never leaves
// registers. Results per edge do not depend on the grouping or the order.
//
// Edges whose batch, head, block or query index lie outside the shapes write the sentinel.
#include "common.h"

namespace pa {
namespace {

constexpr int kChunk = 64;     // edges per work item
constexpr int kThreads = 256;  // 4 waves

struct SparseWs {
    int32_t *counts, *cursor, *offs, *ioffs, *nitems, *item_unit, *perm;
    int max_items;
};

size_t al(size_t x) { return (x + 63) / 64 * 64; }  // in int32 words (256 bytes)

SparseWs carve(int32_t *ws, int E, int units) {
    SparseWs w;
    w.max_items = (E + kChunk - 1) / kChunk + units;
    size_t off = 0;
    w.counts = ws + off; off = al(off + units);
    w.cursor = ws + off; off = al(off + units);
    w.offs = ws + off; off = al(off + units + 1);
    w.ioffs = ws + off; off = al(off + units + 1);
    w.nitems = ws + off; off = al(off + 1);
    w.item_unit = ws + off; off = al(off + w.max_items);
    w.perm = ws + off; off = al(off + E);
    return w;
}

__device__ __forceinline__ bool decode_edge(const SparseArgs &a, int e, int &q, int &h, int &blk,
                                            int &b, int &len, int &unit) {
    const int32_t *m = a.edge_meta + 5LL * e;
    q = m[0]; h = m[1]; blk = m[2]; b = m[3]; len = m[4];
    if (q < 0 || q >= a.tq || h < 0 || h >= a.hkv || blk < 0 || blk >= a.nblk || b < 0 ||
        b >= a.batch || len <= 0)
        return false;
    len = min(len, a.block_size);
    unit = (b * a.hkv + h) * a.nblk + blk;
    return true;
}

__global__ void sp_zero(int32_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// Histogram of valid edges per key block; invalid and empty edges get their sentinel here.
__global__ void sp_hist(SparseArgs a, SparseWs w) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= a.E) return;
    int q, h, blk, b, len, unit;
    if (decode_edge(a, e, q, h, blk, b, len, unit)) {
        atomicAdd(&w.counts[unit], 1);
        return;
    }
    for (int qh = 0; qh < a.qhead; ++qh) {
        const long long p = (long long)e * a.qhead + qh;
        for (int d = 0; d < a.D; d += 4)
            *(float4_t *)(a.o + p * a.D + d) = float4_t{0.f, 0.f, 0.f, 0.f};
        a.m[p] = kNegLarge;
        a.l[p] = 0.f;
    }
}

// One workgroup: exclusive scans of edge counts and of work-item counts, and the item map.
__global__ __launch_bounds__(1024) void sp_scan(SparseArgs a, SparseWs w) {
    __shared__ int sh[2][16];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    int carry_e = 0, carry_i = 0;
    for (int base = 0; base < a.units; base += 1024) {
        const int u = base + tid;
        const int c = u < a.units ? w.counts[u] : 0;
        const int ni = (c + kChunk - 1) / kChunk;
        int xe = c, xi = ni;
        for (int o = 1; o < 64; o <<= 1) {
            const int ye = __shfl_up(xe, o, 64), yi = __shfl_up(xi, o, 64);
            if (lane >= o) { xe += ye; xi += yi; }
        }
        __syncthreads();
        if (lane == 63) { sh[0][wid] = xe; sh[1][wid] = xi; }
        __syncthreads();
        int be = 0, bi = 0, te = 0, ti = 0;
        for (int i = 0; i < 16; ++i) {
            if (i < wid) { be += sh[0][i]; bi += sh[1][i]; }
            te += sh[0][i]; ti += sh[1][i];
        }
        if (u < a.units) {
            const int oe = carry_e + be + xe - c;
            const int oi = carry_i + bi + xi - ni;
            w.offs[u] = oe;
            w.ioffs[u] = oi;
            for (int k = 0; k < ni; ++k) w.item_unit[oi + k] = u;
        }
        carry_e += te;
        carry_i += ti;
    }
    if (tid == 0) {
        w.offs[a.units] = carry_e;
        w.ioffs[a.units] = carry_i;
        w.nitems[0] = carry_i;
    }
}

__global__ void sp_scatter(SparseArgs a, SparseWs w) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= a.E) return;
    int q, h, blk, b, len, unit;
    if (!decode_edge(a, e, q, h, blk, b, len, unit)) return;
    const int pos = w.offs[unit] + atomicAdd(&w.cursor[unit], 1);
    w.perm[pos] = e;
}

// LDS float4 chunk swizzle: chunk q of row r lives at q ^ (r & (nq - 1)) (nq = chunks per row,
// a power of two), so the 16 rows a 16-lane group reads at one column hit distinct banks.
__device__ __forceinline__ int swz(int row, int q, int nq) { return q ^ (row & (min(nq, 16) - 1)); }

template <int D, int NT>
__global__ __launch_bounds__(kThreads) void sp_main(SparseArgs a, SparseWs w) {
    constexpr int BSP = 16 * NT;     // padded keys per block
    constexpr int KD = D / 4;        // dims per lane group in the QK^T contraction
    constexpr int NDT = D / 16;      // 16-dim output tiles
    constexpr int KQ = D / 4;        // float4 chunks per K row
    constexpr int VQ = BSP / 4;      // float4 chunks per V^T row
    extern __shared__ float lds[];
    float *Ks = lds;                 // [BSP][D], swizzled chunks
    float *Vt = lds + BSP * D;       // [D][BSP], swizzled chunks

    const int item = blockIdx.x;
    if (item >= w.nitems[0]) return;
    const int u = w.item_unit[item];
    const int c = item - w.ioffs[u];
    const int ebeg = w.offs[u] + c * kChunk;
    const int nE = min(kChunk, w.offs[u + 1] - ebeg);
    const int blk = u % a.nblk;
    const int bh = u / a.nblk;
    const int h = bh % a.hkv;
    const int b = bh / a.hkv;
    const int32_t *btrow = a.bt + (long long)b * a.max_pages;

    // Stage the key block: K row-major, V transposed; zeros for unmapped or missing keys.
    for (int idx = threadIdx.x; idx < BSP * KQ; idx += kThreads) {
        const int t = idx / KQ, q = idx - t * KQ;
        const int slot = blk * a.ppb + t / a.page_size;
        int pid = -1;
        if (t < a.block_size && slot < a.max_pages) pid = btrow[slot];
        float4_t kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
        if (pid >= 0 && pid < a.num_pages) {
            const long long row =
                (((long long)pid * a.hkv + h) * a.page_size + t % a.page_size) * D + 4 * q;
            kv = *(const float4_t *)(a.kp + row);
            vv = *(const float4_t *)(a.vp + row);
        }
        *(float4_t *)(Ks + t * D + 4 * swz(t, q, KQ)) = kv;
        for (int k = 0; k < 4; ++k) {
            const int r = 4 * q + k;
            Vt[r * BSP + 4 * swz(r, t >> 2, VQ) + (t & 3)] = vv[k];
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g16 = lane >> 4, n16 = lane & 15;
    // Mapped-key masks (wave-uniform): bit t set when key t sits on a mapped page.
    uint64_t mmask[(BSP + 63) / 64];
    for (int hw = 0; hw < (BSP + 63) / 64; ++hw) {
        const int t = 64 * hw + lane;
        const int slot = blk * a.ppb + t / a.page_size;
        bool ok = false;
        if (t < a.block_size && t < BSP && slot < a.max_pages) {
            const int pid = btrow[slot];
            ok = pid >= 0 && pid < a.num_pages;
        }
        mmask[hw] = __ballot(ok);
    }
    const int epg = 16 / a.qhead;          // edges per 16-row group
    const int rows = epg * a.qhead;
    const int hq = a.hkv * a.qhead;
    for (int grp = wave; grp * epg < nE; grp += kThreads / 64) {
        // Row n16 of this group: edge el = n16 / qhead, lane qh = n16 % qhead.
        const int el = n16 / a.qhead, qh = n16 - el * a.qhead;
        const int idx = grp * epg + el;
        const bool vrow = n16 < rows && idx < nE;
        int e = -1, len = 0, qi = 0;
        if (vrow) {
            e = w.perm[ebeg + idx];
            qi = a.edge_meta[5LL * e];
            len = min(a.edge_meta[5LL * e + 4], a.block_size);
        }
        float qf[KD];
        if (vrow) {
            const float *qp = a.q + ((long long)qi * hq + h * a.qhead + qh) * D + KD * g16;
            for (int k = 0; k < KD; k += 4) {
                const float4_t x = *(const float4_t *)(qp + k);
                qf[k] = x[0]; qf[k + 1] = x[1]; qf[k + 2] = x[2]; qf[k + 3] = x[3];
            }
        } else {
            for (int k = 0; k < KD; ++k) qf[k] = 0.f;
        }
        // S^T tiles: lane holds keys 16j + 4g16 + i of row n16.
        float s[NT][4];
        float mx = -INFINITY;
        for (int j = 0; j < NT; ++j) {
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
            const int t = 16 * j + n16;
            for (int k = 0; k < KD; k += 4) {
                const float4_t kk = *(const float4_t *)(Ks + t * D + 4 * swz(t, (KD * g16 + k) >> 2, KQ));
                acc = mfma16x16x4f32(kk[0], qf[k], acc);
                acc = mfma16x16x4f32(kk[1], qf[k + 1], acc);
                acc = mfma16x16x4f32(kk[2], qf[k + 2], acc);
                acc = mfma16x16x4f32(kk[3], qf[k + 3], acc);
            }
            for (int i = 0; i < 4; ++i) {
                const int key = 16 * j + 4 * g16 + i;
                const bool ok = key < len && ((mmask[key >> 6] >> (key & 63)) & 1);
                s[j][i] = ok ? acc[i] * a.scale_log2 : -INFINITY;
                mx = fmaxf(mx, s[j][i]);
            }
        }
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);
        const float mu = (mx == -INFINITY) ? 0.f : mx;
        float ls = 0.f;
        for (int j = 0; j < NT; ++j)
            for (int i = 0; i < 4; ++i) {
                s[j][i] = __builtin_amdgcn_exp2f(s[j][i] - mu);
                ls += s[j][i];
            }
        ls += __shfl_xor(ls, 16, 64);
        ls += __shfl_xor(ls, 32, 64);
        // O = P . V: rows 4g16 + i, dims 16dt + n16.
        float4_t o[NDT];
        for (int dt = 0; dt < NDT; ++dt) o[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < NT; ++j) {
            for (int dt = 0; dt < NDT; ++dt) {
                const int r = 16 * dt + n16;
                const float4_t vv = *(const float4_t *)(Vt + r * BSP + 4 * swz(r, 4 * j + g16, VQ));
                o[dt] = mfma16x16x4f32(s[j][0], vv[0], o[dt]);
                o[dt] = mfma16x16x4f32(s[j][1], vv[1], o[dt]);
                o[dt] = mfma16x16x4f32(s[j][2], vv[2], o[dt]);
                o[dt] = mfma16x16x4f32(s[j][3], vv[3], o[dt]);
            }
        }
        // Stores.
        if (vrow && g16 == 0) {
            const long long p = (long long)e * a.qhead + qh;
            a.m[p] = (mx == -INFINITY) ? kNegLarge : mx * kLn2;
            a.l[p] = ls;
        }
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g16 + i;
            const int er = __shfl(e, r, 64);
            if (r >= rows || er < 0) continue;
            const long long p = (long long)er * a.qhead + (r - (r / a.qhead) * a.qhead);
            for (int dt = 0; dt < NDT; ++dt) a.o[p * D + 16 * dt + n16] = o[dt][i];
        }
    }
}

}  // namespace

size_t sparse_lds_limit() {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        v <= 0)
        return 65536;
    return (size_t)v;
}

size_t sparse_workspace_bytes(int E, int units) {
    const size_t max_items = (size_t)(E + kChunk - 1) / kChunk + units;
    size_t words = al(units) * 2 + al(units + 1) * 2 + al(1) + al(max_items) + al(E);
    return words * 4;
}

pa_status launch_sparse(const SparseArgs &a, hipStream_t stream) {
    LaunchScope scope("sparse_forward", stream);
    SparseWs w = carve(a.ws, a.E, a.units);
    const int nz = (int)(w.offs - w.counts);  // counts and cursor are contiguous
    hipLaunchKernelGGL(sp_zero, dim3((nz + 255) / 256), dim3(256), 0, stream, w.counts, nz);
    const int eg = (a.E + 255) / 256;
    hipLaunchKernelGGL(sp_hist, dim3(eg), dim3(256), 0, stream, a, w);
    hipLaunchKernelGGL(sp_scan, dim3(1), dim3(1024), 0, stream, a, w);
    hipLaunchKernelGGL(sp_scatter, dim3(eg), dim3(256), 0, stream, a, w);
    int nt = 1;
    while (16 * nt < a.block_size) nt *= 2;
    const size_t lds = (size_t)2 * 16 * nt * a.D * sizeof(float);
    if (lds > sparse_lds_limit()) return PA_ERR_UNSUPPORTED;
#define PA_SP_LAUNCH(DD, NN)                                                                 \
    hipLaunchKernelGGL((sp_main<DD, NN>), dim3(w.max_items), dim3(kThreads), lds, stream, a, w)
    if (a.D == 128) {
        if (nt == 1) PA_SP_LAUNCH(128, 1);
        else if (nt == 2) PA_SP_LAUNCH(128, 2);
        else if (nt == 4) PA_SP_LAUNCH(128, 4);
        else PA_SP_LAUNCH(128, 8);
    } else if (a.D == 64) {
        if (nt == 1) PA_SP_LAUNCH(64, 1);
        else if (nt == 2) PA_SP_LAUNCH(64, 2);
        else if (nt == 4) PA_SP_LAUNCH(64, 4);
        else PA_SP_LAUNCH(64, 8);
    } else {
        return PA_ERR_UNSUPPORTED;
    }
#undef PA_SP_LAUNCH
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
