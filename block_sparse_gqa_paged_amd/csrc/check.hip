// Device-side check of the index contract of the paged entry points (a debug aid).
//
// Operation: the inputs section of the "com.microsoft.PagedAttention ... manifest.json" page
// defines cumulative_sequence_length (varlen row offsets of the packed query rows), past_seqlens,
// block_table (logical block -> physical block of each sequence) and slot_mapping (cache slot of
// each new row); its "derive" section fixes tokenCount, blockSize and maxBlocks. The append and
// attention kernels trust these device-resident contents; this pass checks every rule they rely
// on and ORs one bit per violated rule into a caller-owned flag word. It only reads the index
// arrays, inside their declared sizes, and never follows an index, so any contents are safe.
#include "common.h"

#include <algorithm>

namespace pa {
namespace {

struct CheckArgs {
    const int32_t *cu, *past, *bt, *slot;
    int32_t B, T, MB, bs, rot_pos;
    long long NB;
    int32_t *flags;
};

__device__ __forceinline__ void raise_bits(int32_t *flags, int bits) {
    if (bits) atomicOr(flags, bits);
}

__global__ void check_clear(int32_t *flags) { flags[0] = 0; }

// Sequence b's new-token count and total length, when its entries are themselves valid.
__device__ __forceinline__ bool seq_len(const CheckArgs &a, int b, long long &n, long long &L) {
    const long long c0 = a.cu[b], c1 = a.cu[b + 1], p = a.past[b];
    n = c1 - c0;
    L = p + n;
    return n >= 0 && p >= 0;
}

// Three sweeps in one grid-stride launch: sequences (offsets, past lengths, table width),
// block-table entries in use, and new rows (slot_mapping, rotary positions). Duplicate slots are
// a launch of their own (check_slot_dup).
__global__ __launch_bounds__(256) void check_paged(CheckArgs a) {
    const long long stride = (long long)gridDim.x * blockDim.x;
    const long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    int bits = 0;
    for (long long b = tid; b <= a.B; b += stride) {
        const int c = a.cu[b];
        if (b == 0 && c != 0) bits |= PA_CHECK_CU_START;
        if (b == a.B && c != a.T) bits |= PA_CHECK_CU_END;
        if (b < a.B) {
            if (a.cu[b + 1] < c) bits |= PA_CHECK_CU_ORDER;
            if (a.past[b] < 0) bits |= PA_CHECK_PAST;
            long long n, L;
            if (seq_len(a, (int)b, n, L) && (L + a.bs - 1) / a.bs > a.MB)
                bits |= PA_CHECK_TABLE_WIDTH;
        }
    }
    if (a.bt) {
        const long long entries = (long long)a.B * a.MB;
        for (long long e = tid; e < entries; e += stride) {
            const int b = (int)(e / a.MB), j = (int)(e - (long long)b * a.MB);
            long long n, L;
            if (!seq_len(a, b, n, L)) continue;
            if ((long long)j * a.bs >= L) continue;  // entries past the sequence are never read
            const int32_t blk = a.bt[e];
            if (blk < 0 || blk >= a.NB) bits |= PA_CHECK_TABLE_ENTRY;
        }
    }
    for (long long i = tid; i < a.T; i += stride) {
        // sequence of row i: the largest b with cu[b] <= i (a plain search; with disordered
        // offsets it still ends, and the rows are then reported through the offset bits)
        int lo = 0, hi = a.B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu[mid] <= i) lo = mid; else hi = mid - 1;
        }
        const long long pos = (long long)a.past[lo] + (i - a.cu[lo]);
        if (a.rot_pos > 0 && (pos < 0 || pos >= a.rot_pos)) bits |= PA_CHECK_POSITION;
        if (!a.slot) continue;
        const int32_t s = a.slot[i];
        if (s < 0) continue;  // a negative slot is not written
        if (s >= a.NB * a.bs) {
            bits |= PA_CHECK_SLOT;
        } else if (a.bt && pos >= 0 && pos / a.bs < a.MB) {
            const long long want = (long long)a.bt[(long long)lo * a.MB + pos / a.bs] * a.bs +
                                   pos % a.bs;
            if (want != s) bits |= PA_CHECK_SLOT_TABLE;
        }
    }
    raise_bits(a.flags, bits);
}

// The slot new row i writes: its slot_mapping entry, else the slot the block table gives its
// position (only when the position falls inside the table row); -1 when none.
__device__ __forceinline__ long long row_slot(const CheckArgs &a, int i) {
    if (a.slot) return a.slot[i];
    if (!a.bt) return -1;
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const long long pos = (long long)a.past[lo] + (i - a.cu[lo]);
    if (pos < 0 || pos / a.bs >= a.MB) return -1;
    return (long long)a.bt[(long long)lo * a.MB + pos / a.bs] * a.bs + pos % a.bs;
}

// Duplicate written slots: workgroup w takes the w-th pair (k, t), t >= k, of 256-row tiles,
// stages tile t's slots in LDS and compares each of tile k's rows with them (rows j > i only).
// Every non-negative slot takes part.
constexpr int kDupTile = 256;
__global__ __launch_bounds__(kDupTile) void check_slot_dup(CheckArgs a, int ntiles) {
    __shared__ long long sj[kDupTile];
    // pair index -> (k, t): pairs are listed k-major, tile k owning ntiles - k pairs
    long long w = blockIdx.x;
    int k = 0;
    while (w >= ntiles - k) {
        w -= ntiles - k;
        ++k;
    }
    const int t = k + (int)w;
    const int i = k * kDupTile + threadIdx.x;
    const int j0 = t * kDupTile;
    const int jr = j0 + threadIdx.x;
    sj[threadIdx.x] = jr < a.T ? row_slot(a, jr) : -1;
    const long long si = i < a.T ? row_slot(a, i) : -1;
    __syncthreads();
    bool dup = false;
    if (si >= 0)
        for (int x = 0; x < kDupTile; ++x)
            dup |= (j0 + x > i) && sj[x] == si;
    if (__ballot(dup) != 0 && (threadIdx.x & 63) == 0) atomicOr(a.flags, PA_CHECK_SLOT_DUP);
}

}  // namespace

pa_status launch_check_paged(const pa_paged_shape &s, const int32_t *cu, const int32_t *past,
                             const int32_t *bt, const int32_t *slot, int32_t rotary_positions,
                             int32_t *flags, hipStream_t stream) {
    CheckArgs a;
    a.cu = cu;
    a.past = past;
    a.bt = bt;
    a.slot = slot;
    a.B = s.batch;
    a.T = s.num_tokens;
    a.MB = s.max_blocks;
    a.bs = s.block_size;
    a.rot_pos = rotary_positions;
    a.NB = s.num_blocks;
    a.flags = flags;
    const long long work =
        std::max<long long>(std::max<long long>((long long)s.batch * s.max_blocks, s.num_tokens),
                            (long long)s.batch + 1);
    const int grid = (int)std::min<long long>((work + 255) / 256, 1024);
    const long long ntiles = ((long long)s.num_tokens + kDupTile - 1) / kDupTile;
    const long long pairs = (a.slot || a.bt) ? ntiles * (ntiles + 1) / 2 : 0;
    if (pairs > (1LL << 31) - 1) return PA_ERR_UNSUPPORTED;
    LaunchScope scope("check_paged", stream, pairs > 0 ? 3 : 2);
    scope.launch(check_clear, dim3(1), dim3(1), 0, flags);
    scope.launch(check_paged, dim3(grid), dim3(256), 0, a);
    if (pairs > 0)
        scope.launch(check_slot_dup, dim3((unsigned)pairs), dim3(kDupTile), 0, a, (int)ntiles);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
