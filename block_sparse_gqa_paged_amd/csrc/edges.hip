// Edge list of the block-sparse forward, built on the device from a kept-block mask.
//
// Operation: the host step of the "alice-llm ... sparse_attention_forward.wgsl" page (its
// layout notes: edge_meta = (q_idx, h, blk, batch, block_len) with block_len computed from
// used_kv_lens and clamped by the block), with the edges ordered by (q_idx, h, blk) and the
// CSR offsets group_ptr[q*hkv + h] of each (q, h) row, which the merge of the partials reads.
//
// Stream compaction in three passes over the mask [tq, hkv, nblk] (one byte per block):
//  * count: each workgroup writes the number of kept blocks in its rows.
//  * eb_scan: one workgroup turns the workgroup totals into exclusive offsets (in place) and
//    writes the edge count into group_ptr[tq*hkv].
//  * emit: the rows are read again, each row's offset is formed, and every kept block writes
//    its edge at the row offset plus its rank within the row.
// On the 16-byte path with at most kEbOwnPrefix workgroups, emit forms its workgroup offset from
// the totals itself and eb_scan is not launched (two passes).
// Power-of-two nblk from 16 to 1024 (16-byte aligned mask): a lane reads 16 mask bytes, a wave
// covers 64*16/nblk rows per load, nonzero bytes are counted four at a time in a register, and
// ranks come from a segmented scan over each row's lanes. Other nblk: a wave reads a row 64
// bytes at a time and counts with the popcount of a ballot; ranks are mbcnt.
#include "common.h"

namespace pa {
namespace {

constexpr int kEbThreads = 256;          // four waves
constexpr int kEbRowsPerWave = 8;
constexpr int kEbRows = 4 * kEbRowsPerWave;  // rows of the mask per workgroup

__device__ __forceinline__ int row_count(const uint8_t *row, int nblk, int lane) {
    int cnt = 0;
    for (int c = 0; c < nblk; c += 64) {
        const bool set = c + lane < nblk && row[c + lane] != 0;
        cnt += __popcll(__ballot(set));
    }
    return cnt;
}

__global__ __launch_bounds__(kEbThreads) void eb_count(EdgeArgs a) {
    __shared__ int s_tot[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long long r0 = (long long)blockIdx.x * kEbRows + wave * kEbRowsPerWave;
    int tot = 0;
    for (int r = 0; r < kEbRowsPerWave; ++r) {
        const long long row = r0 + r;
        if (row >= a.rows) break;
        tot += row_count(a.mask + row * a.nblk, a.nblk, lane);
    }
    if (lane == 0) s_tot[wave] = tot;
    __syncthreads();
    if (threadIdx.x == 0) a.wg[blockIdx.x] = s_tot[0] + s_tot[1] + s_tot[2] + s_tot[3];
}

__global__ __launch_bounds__(1024) void eb_scan(EdgeArgs a, int nwg) {
    __shared__ int sh[16];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    int carry = 0;
    for (int base = 0; base < nwg; base += 1024) {
        const int i = base + tid;
        const int v = i < nwg ? a.wg[i] : 0;
        int x = v;
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (lane >= o) x += y;
        }
        __syncthreads();
        if (lane == 63) sh[wid] = x;
        __syncthreads();
        int before = 0, all = 0;
        for (int k = 0; k < 16; ++k) {
            if (k < wid) before += sh[k];
            all += sh[k];
        }
        if (i < nwg) a.wg[i] = carry + before + x - v;
        carry += all;
    }
    if (tid == 0) a.group_ptr[a.rows] = carry;
}

__global__ __launch_bounds__(kEbThreads) void eb_emit(EdgeArgs a) {
    __shared__ int s_tot[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const long long r0 = (long long)blockIdx.x * kEbRows + wave * kEbRowsPerWave;
    int tot = 0;
    for (int r = 0; r < kEbRowsPerWave; ++r) {
        const long long row = r0 + r;
        if (row >= a.rows) break;
        tot += row_count(a.mask + row * a.nblk, a.nblk, lane);
    }
    if (lane == 0) s_tot[wave] = tot;
    __syncthreads();
    long long e = a.wg[blockIdx.x];
    for (int w = 0; w < wave; ++w) e += s_tot[w];
    for (int r = 0; r < kEbRowsPerWave; ++r) {
        const long long row = r0 + r;
        if (row >= a.rows) break;
        const int q = (int)(row / a.hkv), h = (int)(row - (long long)q * a.hkv);
        const int b = a.q_batch[q];
        const int used = a.used[min(max(b, 0), a.batch - 1)];  // out-of-range batch: any row
        if (lane == 0) a.group_ptr[row] = (int32_t)e;
        const uint8_t *m = a.mask + row * a.nblk;
        for (int c = 0; c < a.nblk; c += 64) {
            const int blk = c + lane;
            const bool set = blk < a.nblk && m[blk] != 0;
            const uint64_t bits = __ballot(set);
            if (set) {
                const long long k = e + __popcll(bits & ((1ull << lane) - 1));
                if (k < a.capacity) {
                    const long long len = (long long)used - (long long)blk * a.block_size;
                    int32_t *o = a.edge_meta + 5 * k;
                    o[0] = q;
                    o[1] = h;
                    o[2] = blk;
                    o[3] = b;
                    o[4] = (int32_t)(len < 0 ? 0 : (len > a.block_size ? a.block_size : len));
                }
            }
            e += __popcll(bits);
        }
    }
}

// ---- 16-byte path. cpr = nblk / 16 lanes per row (a power of two <= 64), rpl = 64 / cpr rows
// per wave load; a wave takes G loads, i.e. G * rpl consecutive rows. G is the smallest of
// 2, 4, 8 with G * rpl >= 8, so that a workgroup covers at least kEbRows rows (the workspace
// holds one total per kEbRows rows) while the grid stays large: with 8 loads per wave the
// 0.99 M-edge mask (32768 rows of 64 blocks) filled only 64 workgroups.

__device__ __forceinline__ int nz_bytes(uint32_t x) {  // nonzero bytes of a word
    uint32_t t = x | (x >> 4);
    t |= t >> 2;
    t |= t >> 1;
    return __popc(t & 0x01010101u);
}

__device__ __forceinline__ int nz16(const uint4 &v) {
    return nz_bytes(v.x) + nz_bytes(v.y) + nz_bytes(v.z) + nz_bytes(v.w);
}

template <int G>
struct VecRows {
    uint4 v[G];
    long long row[G];  // this lane's row in each load (or >= rows)
};

template <int G>
__device__ __forceinline__ VecRows<G> vec_load(const EdgeArgs &a, long long w0, int lcpr,
                                               int lane) {
    VecRows<G> r;
    const int cpr = 1 << lcpr, rpl = 64 >> lcpr;
    for (int g = 0; g < G; ++g) {
        r.row[g] = w0 + (long long)g * rpl + (lane >> lcpr);
        const long long rr = r.row[g] < a.rows ? r.row[g] : a.rows - 1;
        r.v[g] = *(const uint4 *)(a.mask + rr * a.nblk + 16 * (lane & (cpr - 1)));
        if (r.row[g] >= a.rows) r.v[g] = uint4{0u, 0u, 0u, 0u};
    }
    return r;
}

template <int G>
__global__ __launch_bounds__(kEbThreads) void eb_count_vec(EdgeArgs a, int lcpr) {
    __shared__ int s_tot[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wrows = G * (64 >> lcpr);
    const long long w0 = ((long long)blockIdx.x * 4 + wave) * wrows;
    const VecRows<G> r = vec_load<G>(a, w0, lcpr, lane);
    int c = 0;
    for (int g = 0; g < G; ++g) c += nz16(r.v[g]);
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
    if (lane == 0) s_tot[wave] = c;
    __syncthreads();
    if (threadIdx.x == 0) a.wg[blockIdx.x] = s_tot[0] + s_tot[1] + s_tot[2] + s_tot[3];
}

// A grid of at most kEbOwnPrefix workgroups runs without eb_scan: each emit workgroup adds up
// the totals of the workgroups before it (at most 16 KB of reads, issued with its mask loads)
// and the last one writes the edge count; a launch boundary costs more than that.
constexpr int kEbOwnPrefix = 4096;

template <int G>
__global__ __launch_bounds__(kEbThreads) void eb_emit_vec(EdgeArgs a, int lcpr, int own_prefix) {
    __shared__ int s_tot[4], s_pre[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cpr = 1 << lcpr;
    const int wrows = G * (64 >> lcpr);
    const long long w0 = ((long long)blockIdx.x * 4 + wave) * wrows;
    const VecRows<G> r = vec_load<G>(a, w0, lcpr, lane);
    long long wg0;  // this workgroup's first edge
    if (own_prefix) {
        int part = 0;  // a.wg holds the workgroups' totals
        for (int i = threadIdx.x; i < (int)blockIdx.x; i += kEbThreads) part += a.wg[i];
        for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
        if (lane == 0) s_pre[wave] = part;  // published by the barrier below
    } else {
        wg0 = a.wg[blockIdx.x];  // a.wg holds exclusive offsets (eb_scan)
    }
    int cnt[G];
    int wt = 0;
    for (int g = 0; g < G; ++g) {
        cnt[g] = nz16(r.v[g]);
        wt += cnt[g];
    }
    for (int o = 32; o > 0; o >>= 1) wt += __shfl_xor(wt, o, 64);
    if (lane == 0) s_tot[wave] = wt;
    __syncthreads();
    if (own_prefix) {
        wg0 = (long long)s_pre[0] + s_pre[1] + s_pre[2] + s_pre[3];
        if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0)
            a.group_ptr[a.rows] = (int32_t)(wg0 + s_tot[0] + s_tot[1] + s_tot[2] + s_tot[3]);
    }
    long long e = wg0;  // offset of this wave's first row
    for (int w = 0; w < wave; ++w) e += s_tot[w];
    const int seg = lane & (cpr - 1);  // lane's place inside its row
    for (int g = 0; g < G; ++g) {
        // inclusive scan of the counts over each row's cpr lanes
        int x = cnt[g];
        for (int o = 1; o < cpr; o <<= 1) {
            const int y = __shfl_up(x, o, 64);
            if (seg >= o) x += y;
        }
        // rows of this load in order: offset of the lane's row = e + totals of earlier rows
        int before = 0;
        for (int q = 0; q < (64 >> lcpr); ++q) {
            const int tq_ = __shfl(x, (q << lcpr) | (cpr - 1), 64);
            if (q < (lane >> lcpr)) before += tq_;
        }
        int load_tot = 0;
        for (int q = 0; q < (64 >> lcpr); ++q) load_tot += __shfl(x, (q << lcpr) | (cpr - 1), 64);
        const long long row = r.row[g];
        if (row < a.rows) {
            const long long rbase = e + before;
            if (seg == 0) a.group_ptr[row] = (int32_t)rbase;
            long long k = rbase + x - cnt[g];  // first edge of this lane's 16 blocks
            const int q = (int)(row / a.hkv), h = (int)(row - (long long)q * a.hkv);
            const int b = a.q_batch[q];
            const int used = a.used[min(max(b, 0), a.batch - 1)];
            // bit i of `set`: byte i of the lane's 16 is nonzero; visit only those
            const uint32_t wv[4] = {r.v[g].x, r.v[g].y, r.v[g].z, r.v[g].w};
            uint32_t set = 0;
            for (int i = 0; i < 16; ++i)
                set |= (((wv[i >> 2] >> (8 * (i & 3))) & 0xffu) != 0u ? 1u : 0u) << i;
            while (set) {
                const int i = __ffs(set) - 1;
                set &= set - 1;
                if (k < a.capacity) {
                    const int blk = 16 * seg + i;
                    const long long len = (long long)used - (long long)blk * a.block_size;
                    int32_t *o = a.edge_meta + 5 * k;
                    o[0] = q;
                    o[1] = h;
                    o[2] = blk;
                    o[3] = b;
                    o[4] = (int32_t)(len < 0 ? 0 : (len > a.block_size ? a.block_size : len));
                }
                ++k;
            }
        }
        e += load_tot;
    }
}

}  // namespace

size_t edge_workspace_bytes(long long rows) {
    const long long nwg = (rows + kEbRows - 1) / kEbRows;
    return (size_t)((nwg + 63) / 64 * 64) * 4;
}

pa_status launch_build_edges(const EdgeArgs &a, hipStream_t stream) {
    const long long nwg = (a.rows + kEbRows - 1) / kEbRows;
    if (nwg > 0x7fffffff) return PA_ERR_UNSUPPORTED;
    if (nwg == 0) {  // no rows: group_ptr[0] = 0
        LaunchScope scope("build_edges", stream, 1);
        scope.launch(eb_scan, dim3(1), dim3(1024), 0, a, 0);
        return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
    }
    int lcpr = -1;  // 16-byte path when nblk = 16 * 2^lcpr <= 1024 and the mask is aligned
    for (int l = 0; l <= 6; ++l)
        if (a.nblk == 16 << l) lcpr = l;
    if (lcpr >= 0 && ((uintptr_t)a.mask % 16) == 0) {
        const int rpl = 64 >> lcpr;
        const int G = rpl >= 4 ? 2 : 8 / rpl;  // G * rpl >= 8
        const long long wg_rows = 4LL * G * rpl;  // >= kEbRows: nv <= nwg, the workspace fits
        const long long nv = (a.rows + wg_rows - 1) / wg_rows;
        const int own = nv <= kEbOwnPrefix;
        LaunchScope scope("build_edges", stream, own ? 2 : 3);
        const dim3 grid((unsigned)nv), block(kEbThreads);
        if (G == 2) scope.launch(eb_count_vec<2>, grid, block, 0, a, lcpr);
        else if (G == 4) scope.launch(eb_count_vec<4>, grid, block, 0, a, lcpr);
        else scope.launch(eb_count_vec<8>, grid, block, 0, a, lcpr);
        if (!own) scope.launch(eb_scan, dim3(1), dim3(1024), 0, a, (int)nv);
        if (G == 2) scope.launch(eb_emit_vec<2>, grid, block, 0, a, lcpr, own);
        else if (G == 4) scope.launch(eb_emit_vec<4>, grid, block, 0, a, lcpr, own);
        else scope.launch(eb_emit_vec<8>, grid, block, 0, a, lcpr, own);
        return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
    }
    LaunchScope scope("build_edges", stream, 3);
    scope.launch(eb_count, dim3((unsigned)nwg), dim3(kEbThreads), 0, a);
    scope.launch(eb_scan, dim3(1), dim3(1024), 0, a, (int)nwg);
    scope.launch(eb_emit, dim3((unsigned)nwg), dim3(kEbThreads), 0, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
