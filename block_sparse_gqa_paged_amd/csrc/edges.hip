// Edge list of the block-sparse forward, built on the device from a kept-block mask.
//
// Operation: the host step of the "alice-llm ... sparse_attention_forward.wgsl" page (its
// layout notes: edge_meta = (q_idx, h, blk, batch, block_len) with block_len computed from
// used_kv_lens and clamped by the block), with the edges ordered by (q_idx, h, blk) and the
// CSR offsets group_ptr[q*hkv + h] of each (q, h) row, which the merge of the partials reads.
//
// Stream compaction in three passes over the mask [tq, hkv, nblk] (one byte per block):
//  * eb_count: a wave takes rows of the mask 64 bytes at a time; the popcount of a ballot of
//    the nonzero bytes counts a row's edges with no reduction; each workgroup writes the total
//    of its rows.
//  * eb_scan: one workgroup turns the workgroup totals into exclusive offsets (in place) and
//    writes the edge count into group_ptr[tq*hkv].
//  * eb_emit: the count pass again, then each row's offset, and every set byte writes its edge
//    at the row offset plus its rank in the ballot (mbcnt).
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
    LaunchScope scope("build_edges", stream, 3);
    scope.launch(eb_count, dim3((unsigned)nwg), dim3(kEbThreads), 0, a);
    scope.launch(eb_scan, dim3(1), dim3(1024), 0, a, (int)nwg);
    scope.launch(eb_emit, dim3((unsigned)nwg), dim3(kEbThreads), 0, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
