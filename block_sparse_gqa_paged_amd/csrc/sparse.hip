// Block-sparse "edge" forward in fp32 for gfx950, KV-outer.
//
// Operation: sparse_forward of the "alice-llm ... sparse_attention_forward.wgsl" page. Edge
// e = (q_idx, h, blk, batch, block_len); for each q-head lane qh it scores the query row
// (q_idx, h*qhead + qh) against keys t < block_len of block blk (pages through the batch's
// table row; unmapped pages contribute nothing), and writes the block-local, unnormalised
// (o, m, l) at p = e*qhead + qh. block_len <= 0, or no mapped key, gives o = 0, m = -1e30, l = 0.
//
// MI355X design:
//  * Edges are grouped by their (batch, h, blk) key block with a counting sort on the device:
//    per-chunk LDS histograms that give each edge its rank (no global atomics; a global-atomic
//    histogram for shapes with more key blocks than LDS holds), scans that also write one record
//    per work item, and a scatter of packed edge records (id, query, final key count) into
//    sorted order. One workgroup then stages a key block in LDS once and reuses it for up to
//    kChunk edges; results per edge do not depend on the grouping or the order. A work item
//    starts with two dependent loads: its record (which carries the block's page ids when the
//    block has at most 4 pages, else the table entries are a third), then its edge records
//    beside the block's K and V rows.
//  * fp32 products run as three fp16 MFMAs (v_mfma_f32_16x16x32_f16) on split operands. Before
//    the split, each query row and the block's K are scaled by a power of two that brings their
//    largest magnitude into [0.5, 1), and so is each dimension of the block's V whose largest
//    magnitude is below 0.5 or at least 2^15 (exact; folded back into the scores and, per
//    dimension, into the output, which needs no scaling when no dimension is scaled; capped at
//    2^126 for maxima far below 2^-100, so that the factor stays finite). Q and K are scaled by
//    another 2^11 and split as x = hi + lo, hi = fp16(x), lo = fp16(x - hi): lo stays a normal
//    fp16 number for elements down to 2^-14 of the maximum, so each operand keeps 22
//    significant bits over that range; 2^22 q.k ~ hi.lo + lo.hi + hi.hi, summed in one fp32
//    accumulator. V and P: x = hi + lo with lo = fp16(x - hi), and p.v ~ hi.hi + hi.lo + lo.hi;
//    each element keeps 22 significant bits or an absolute error below 2^-25 in the units of its
//    scaled dimension (half of fp16's subnormal step), which for a V dimension split as it is
//    (largest magnitude in [0.5, 2^15)) is at least as fine as after scaling it down; P <= 1
//    needs no scaling.
//    The dropped lo.lo terms are ~2^-22 of each product.
//  * S^T = K . Q^T has 16 keys as rows and 16 query rows as columns; its accumulator gives each
//    lane 8 keys of one row across two key tiles, exactly the k-slots of the P operand of
//    O^T = V^T . P^T, so P never leaves registers, and O^T gives each lane four consecutive
//    dims of one query row for its stores. K (row-major) and V (transposed, keys ordered so
//    that one 16-byte read is one operand) live in LDS as fp16 hi/lo planes with XOR-swizzled
//    chunks.
//  * Each group of 16 (edge, lane) rows loads its fp32 query rows and scales and splits them in
//    registers (a row's exponent from the maximum over the 4 lanes that hold it); the item's
//    edge list sits in LDS. A separate pass writing split query planes would move the same bytes
//    per row plus its own 200 MB and launch.
//
// Edges whose batch, head, block or query index lie outside the shapes write the sentinel.
// With q_pos (the causal entry), an edge sees only keys at positions <= q_pos[q_idx]: its length
// is cut to that prefix in its sorted record.
#include "common.h"
#include <type_traits>

namespace pa {
namespace {

constexpr int kChunk = 128;    // edges per work item
constexpr int kThreads = 512;  // 8 waves

// The counting sort of the edges by key block takes one of two forms:
//  * chunked (up to kHistUnits key blocks and kMaxChunkCounts chunk counts): each workgroup
//    counts a chunk of kEdgeChunk consecutive edges in an LDS histogram (an edge's rank within
//    its chunk comes from the LDS atomic) and writes the chunk's count of every block; a pass per
//    block turns its counts into offsets over the chunks (the blocks' edges stay in chunk order,
//    that is in edge order up to the order inside a chunk), a workgroup scan per 256 blocks and
//    one small scan give each block's first position, and the scatter adds the three. No global
//    atomics: device-wide atomics with return run at about 17 per ns on MI355X, 58 us for the
//    0.99 M edges of the block-sparse workload.
//  * otherwise, a global histogram whose atomic returns each edge's rank in its block.
constexpr int kHistUnits = 16384;          // LDS histogram: 64 KB
constexpr int kEdgeChunk = 16384;          // edges per histogram workgroup
constexpr int kHistThreads = 1024;
constexpr long long kMaxChunkCounts = 1LL << 24;
constexpr int kUnitsPerScan = 256;         // key blocks per workgroup of the per-block pass

bool sort_chunked(int E, int units) {
    const long long chunks = ((long long)E + kEdgeChunk - 1) / kEdgeChunk;
    return units <= kHistUnits && chunks * units <= kMaxChunkCounts;
}

// Work-item record, two 16-byte words: its key block (unit), first edge in the sorted order and
// edge count; then, for blocks of up to 4 pages, the block's page ids (checked: -1 for an
// unmapped or out-of-range entry), so that the forward kernel reads no table entry itself.
// Sorted edge record: edge id, query index and the edge's key count (clamped to the block,
// cut to the query's causal limit). One 16-byte load for the forward kernel.
struct SparseWs {
    int32_t *counts, *rank, *offs, *nitems;
    int32_t *chunk_counts;  // chunked sort: [chunks][units], then offsets within each block
    int32_t *lo;            // chunked sort: per block, first edge and item within its 256
    int32_t *wtot;          // chunked sort: per 256 blocks, edge and item totals, then bases
    int4_t *items, *edges;
    int max_items, chunks, nscan;
    bool chunked;
};

size_t al(size_t x) { return (x + 63) / 64 * 64; }  // in int32 words (256 bytes)

// Workspace layout in int32 words; returns the total.
size_t layout(SparseWs *w, int32_t *ws, int E, int units) {
    const size_t max_items = (size_t)(E + kChunk - 1) / kChunk + units;
    const bool chunked = sort_chunked(E, units);
    const size_t chunks = chunked ? ((size_t)E + kEdgeChunk - 1) / kEdgeChunk : 0;
    const size_t nscan = ((size_t)units + kUnitsPerScan - 1) / kUnitsPerScan;
    size_t off = 0, o[9];
    o[0] = off; off = al(off + units);             // counts
    o[1] = off; off = al(off + E);                 // rank
    o[2] = off; off = al(off + units + 1);         // offs
    o[3] = off; off = al(off + 1);                 // nitems
    o[4] = off; off = al(off + 8 * max_items);     // items (two 16-byte records each)
    o[5] = off; off = al(off + 4 * (size_t)E);     // edges (sorted)
    o[6] = off; off = al(off + chunks * units);    // chunk counts
    o[7] = off; off = al(off + (chunked ? 2 * (size_t)units : 0));   // lo
    o[8] = off; off = al(off + (chunked ? 2 * nscan : 0));           // wtot
    if (w) {
        w->counts = ws + o[0]; w->rank = ws + o[1]; w->offs = ws + o[2]; w->nitems = ws + o[3];
        w->items = (int4_t *)(ws + o[4]); w->edges = (int4_t *)(ws + o[5]);
        w->chunk_counts = ws + o[6]; w->lo = ws + o[7]; w->wtot = ws + o[8];
        w->max_items = (int)max_items;
        w->chunks = (int)chunks;
        w->nscan = (int)nscan;
        w->chunked = chunked;
    }
    return off;
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

// Block-table page of key t of the block at (b, blk), or -1 (past the block, past the table row,
// or an unmapped or out-of-range entry).
__device__ __forceinline__ int block_page(const SparseArgs &a, const int32_t *btrow, int blk,
                                          int t) {
    const int slot = blk * a.ppb + t / a.page_size;
    int pid = -1;
    if (t < a.block_size && slot < a.max_pages) pid = btrow[slot];
    return (pid >= 0 && pid < a.num_pages) ? pid : -1;
}

// The page ids of key block u's page slots 0..3 (-1 past the block's pages) when a block has at
// most 4 pages; all -1 otherwise (the forward kernel then reads the table).
__device__ int4_t item_pages(const SparseArgs &a, int u) {
    int4_t p = {-1, -1, -1, -1};
    if (a.ppb > 4) return p;
    const int blk = u % a.nblk, b = u / a.nblk / a.hkv;
    const int32_t *btrow = a.bt + (long long)b * a.max_pages;
    for (int sl = 0; sl < a.ppb; ++sl) p[sl] = block_page(a, btrow, blk, sl * a.page_size);
    return p;
}

__global__ void sp_zero(int32_t *p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

// The sentinel partials of an invalid or empty edge.
__device__ void write_sentinel(const SparseArgs &a, int e) {
    for (int qh = 0; qh < a.qhead; ++qh) {
        const long long p = (long long)e * a.qhead + qh;
        for (int d = 0; d < a.D; d += 4)
            *(float4_t *)(a.o + p * a.D + d) = float4_t{0.f, 0.f, 0.f, 0.f};
        a.m[p] = kNegLarge;
        a.l[p] = 0.f;
    }
}

// Histogram of valid edges per key block (the returned count is the edge's rank in its block);
// invalid and empty edges get their sentinel here.
__global__ void sp_hist(SparseArgs a, SparseWs w) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= a.E) return;
    int q, h, blk, b, len, unit;
    if (decode_edge(a, e, q, h, blk, b, len, unit)) {
        w.rank[e] = atomicAdd(&w.counts[unit], 1);
        return;
    }
    write_sentinel(a, e);
}

// Chunked sort, pass 1: workgroup c counts edges [c kEdgeChunk, (c + 1) kEdgeChunk) per key block
// in LDS (rank = the edge's position among its block's edges in the chunk), writes the chunk's
// counts of every block, and the sentinels of invalid edges.
__global__ __launch_bounds__(kHistThreads) void sp_chist(SparseArgs a, SparseWs w) {
    extern __shared__ int hist[];  // units entries
    for (int i = threadIdx.x; i < a.units; i += kHistThreads) hist[i] = 0;
    __syncthreads();
    const int e0 = blockIdx.x * kEdgeChunk;
    for (int k = 0; k < kEdgeChunk / kHistThreads; ++k) {
        const int e = e0 + k * kHistThreads + threadIdx.x;
        if (e >= a.E) break;
        int q, h, blk, b, len, unit;
        if (decode_edge(a, e, q, h, blk, b, len, unit))
            w.rank[e] = atomicAdd(&hist[unit], 1);
        else
            write_sentinel(a, e);
    }
    __syncthreads();
    int32_t *dst = w.chunk_counts + (size_t)blockIdx.x * a.units;
    for (int i = threadIdx.x; i < a.units; i += kHistThreads) dst[i] = hist[i];
}

// Chunked sort, pass 2: thread per key block. Its counts over the chunks become exclusive
// offsets in place; the block's total and item count are scanned over the workgroup's
// kUnitsPerScan blocks (first edge and item within them in lo, the workgroup's totals in wtot).
__global__ __launch_bounds__(kUnitsPerScan) void sp_cprefix(SparseArgs a, SparseWs w) {
    __shared__ int sh[2][kUnitsPerScan / 64];
    const int u = blockIdx.x * kUnitsPerScan + threadIdx.x;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int run = 0;
    if (u < a.units) {
        // 16 chunks at a time: all loads first, then the stores (in place), so that the loads
        // of a batch are in flight together
        int32_t *col = w.chunk_counts + u;
        for (int c0 = 0; c0 < w.chunks; c0 += 16) {
            int v[16];
            for (int j = 0; j < 16; ++j)
                v[j] = c0 + j < w.chunks ? col[(size_t)(c0 + j) * a.units] : 0;
            for (int j = 0; j < 16; ++j) {
                if (c0 + j < w.chunks) col[(size_t)(c0 + j) * a.units] = run;
                run += v[j];
            }
        }
        w.counts[u] = run;
    }
    const int ni = (run + kChunk - 1) / kChunk;
    int xe = run, xi = ni;  // inclusive scans within the wave
    for (int o = 1; o < 64; o <<= 1) {
        const int ye = __shfl_up(xe, o, 64), yi = __shfl_up(xi, o, 64);
        if (lane >= o) { xe += ye; xi += yi; }
    }
    if (lane == 63) { sh[0][wid] = xe; sh[1][wid] = xi; }
    __syncthreads();
    int oe = xe - run, oi = xi - ni, te = 0, ti = 0;
    for (int i = 0; i < kUnitsPerScan / 64; ++i) {
        if (i < wid) { oe += sh[0][i]; oi += sh[1][i]; }
        te += sh[0][i]; ti += sh[1][i];
    }
    if (u < a.units) {
        w.lo[2 * u] = oe;
        w.lo[2 * u + 1] = oi;
    }
    if (threadIdx.x == 0) {
        w.wtot[2 * blockIdx.x] = te;
        w.wtot[2 * blockIdx.x + 1] = ti;
    }
}

// Chunked sort, pass 3: exclusive scan of the per-workgroup totals (in place) and the item
// count. One workgroup.
__global__ __launch_bounds__(1024) void sp_wscan(SparseWs w) {
    __shared__ int sh[2][16];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int per = (w.nscan + 1023) / 1024;
    const int i0 = min(w.nscan, tid * per), i1 = min(w.nscan, i0 + per);
    int se = 0, si = 0;
    for (int i = i0; i < i1; ++i) { se += w.wtot[2 * i]; si += w.wtot[2 * i + 1]; }
    int xe = se, xi = si;
    for (int o = 1; o < 64; o <<= 1) {
        const int ye = __shfl_up(xe, o, 64), yi = __shfl_up(xi, o, 64);
        if (lane >= o) { xe += ye; xi += yi; }
    }
    if (lane == 63) { sh[0][wid] = xe; sh[1][wid] = xi; }
    __syncthreads();
    int oe = xe - se, oi = xi - si, ti = 0;
    for (int i = 0; i < 16; ++i) {
        if (i < wid) { oe += sh[0][i]; oi += sh[1][i]; }
        ti += sh[1][i];
    }
    for (int i = i0; i < i1; ++i) {
        const int ce = w.wtot[2 * i], ci = w.wtot[2 * i + 1];
        w.wtot[2 * i] = oe;
        w.wtot[2 * i + 1] = oi;
        oe += ce;
        oi += ci;
    }
    if (tid == 0) w.nitems[0] = ti;
}

// Chunked sort, pass 4: thread i writes the work items of key block i (i < units) and the sorted
// record of edge i (i < E) at its block's first position + its chunk's offset + its rank.
__global__ void sp_cscatter(SparseArgs a, SparseWs w) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < a.units) {
        const int s = i / kUnitsPerScan;
        const int ebase = w.wtot[2 * s] + w.lo[2 * i], ibase = w.wtot[2 * s + 1] + w.lo[2 * i + 1];
        const int c = w.counts[i];
        if (c > 0) {
            const int4_t pg = item_pages(a, i);
            for (int k = 0; k * kChunk < c; ++k) {
                w.items[2 * (ibase + k)] =
                    int4_t{i, ebase + k * kChunk, min(kChunk, c - k * kChunk), 0};
                w.items[2 * (ibase + k) + 1] = pg;
            }
        }
    }
    if (i >= a.E) return;
    int q, h, blk, b, len, unit;
    if (!decode_edge(a, i, q, h, blk, b, len, unit)) return;
    // causal: keys at positions after the query row's are cut off (a prefix stays)
    if (a.q_pos) len = min(len, a.q_pos[q] - blk * a.block_size + 1);
    const int s = unit / kUnitsPerScan;
    const int pos = w.wtot[2 * s] + w.lo[2 * unit] +
                    w.chunk_counts[(size_t)(i / kEdgeChunk) * a.units + unit] + w.rank[i];
    w.edges[pos] = int4_t{i, q, len, 0};
}

// One workgroup: exclusive scans of edge counts and of work-item counts, and the item records.
// Each thread takes a contiguous run of units: it sums its run, one workgroup-wide scan of the
// run sums gives the run's offsets, and the thread then writes its units' offsets and items.
__global__ __launch_bounds__(1024) void sp_scan(SparseArgs a, SparseWs w) {
    __shared__ int sh[2][16];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int per = (a.units + 1023) / 1024;
    const int u0 = min(a.units, tid * per), u1 = min(a.units, u0 + per);
    int se = 0, si = 0;
    for (int u = u0; u < u1; ++u) {
        const int c = w.counts[u];
        se += c;
        si += (c + kChunk - 1) / kChunk;
    }
    int xe = se, xi = si;  // inclusive scans within the wave
    for (int o = 1; o < 64; o <<= 1) {
        const int ye = __shfl_up(xe, o, 64), yi = __shfl_up(xi, o, 64);
        if (lane >= o) { xe += ye; xi += yi; }
    }
    if (lane == 63) { sh[0][wid] = xe; sh[1][wid] = xi; }
    __syncthreads();
    int oe = xe - se, oi = xi - si, te = 0, ti = 0;
    for (int i = 0; i < 16; ++i) {
        if (i < wid) { oe += sh[0][i]; oi += sh[1][i]; }
        te += sh[0][i]; ti += sh[1][i];
    }
    for (int u = u0; u < u1; ++u) {
        const int c = w.counts[u], ni = (c + kChunk - 1) / kChunk;
        w.offs[u] = oe;
        if (ni > 0) {
            const int4_t pg = item_pages(a, u);
            for (int k = 0; k < ni; ++k) {
                w.items[2 * (oi + k)] = int4_t{u, oe + k * kChunk, min(kChunk, c - k * kChunk), 0};
                w.items[2 * (oi + k) + 1] = pg;
            }
        }
        oe += c;
        oi += ni;
    }
    if (tid == 0) {
        w.offs[a.units] = te;
        w.nitems[0] = ti;
    }
}

__global__ void sp_scatter(SparseArgs a, SparseWs w) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= a.E) return;
    int q, h, blk, b, len, unit;
    if (!decode_edge(a, e, q, h, blk, b, len, unit)) return;
    // causal: keys at positions after the query row's are cut off (a prefix stays)
    if (a.q_pos) len = min(len, a.q_pos[q] - blk * a.block_size + 1);
    w.edges[w.offs[unit] + w.rank[e]] = int4_t{e, q, len, 0};
}

// Split two floats x0 f, x1 f (f a power of two, the results in fp16 range) into fp16 hi and lo
// parts, x f ~ hi + lo: one packed conversion gives both hi parts, and each lo = x f - hi is one
// mixed-precision fused multiply-add that reads hi as fp16 and writes fp16.
typedef float float2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split16x2(float x0, float x1, float f, half2_t &hi, half2_t &lo) {
    hi = __builtin_convertvector(float2_t{x0 * f, x1 * f}, half2_t);
    lo[0] = (half_t)__builtin_fmaf(x0, f, -(float)hi[0]);
    lo[1] = (half_t)__builtin_fmaf(x1, f, -(float)hi[1]);
}
// The same unscaled; one is 1.f hidden from the compiler (with a literal 1 the multiply-adds
// would be rewritten as widen-and-subtract).
__device__ __forceinline__ void split16x2u(float x0, float x1, float one, half2_t &hi,
                                           half2_t &lo) {
    hi = __builtin_convertvector(float2_t{x0, x1}, half2_t);
    lo[0] = (half_t)__builtin_fmaf(x0, one, -(float)hi[0]);
    lo[1] = (half_t)__builtin_fmaf(x1, one, -(float)hi[1]);
}
// Q and K are split after scaling into [-2^11, 2^11) (kOpExp): there hi keeps 11 significant
// bits for every |x| >= 2^-14 and lo = fp16(x - hi), at most half an ulp of hi, stays a normal
// fp16 number for every |x| >= 2^-3, i.e. for elements down to 2^-14 of the row or block maximum,
// with no separate scaling of the remainder.
constexpr int kOpExp = 11;

// Scaling shift 2^sh for a maximum of exponent e (pow2_exp): top - e, capped at 126 so that 2^sh
// stays a finite float (only elements far below 2^-100 reach the cap; they then scale to less
// than the top, which they keep as fp16 subnormals).
__device__ __forceinline__ int scale_shift(int top, int e) { return min(top - e, 126); }

// Item row r -> (edge within the item, q-head lane), r = ix * d + qh, with inv = 1 / d. Rows
// number at most 128 d + 15, so the quotient is at most 143 and its float estimate is off by
// less than 1e-4: truncation is the quotient or one away from it, and one step either way
// corrects it (a few instructions instead of an integer division by the runtime d).
struct RowIx {
    int ix, qh;
};
__device__ __forceinline__ RowIx row_split(int r, int d, float inv) {
    int q = (int)((float)r * inv);
    int rem = r - q * d;
    if (rem < 0) { --q; rem += d; }
    if (rem >= d) { ++q; rem -= d; }
    return RowIx{q, rem};
}

// Power-of-two factor that brings max |x| = mx into [0.5, 1) (1 for mx == 0).
__device__ __forceinline__ int pow2_exp(float mx) {
    int e = 0;
    (void)frexpf(mx, &e);
    return mx > 0.f ? e : 0;
}

// XOR swizzle of 16-byte chunk q in row r of a plane with nq chunks per row (a power of two). A
// 16-lane group reads 16 consecutive rows at one logical chunk, and one pass over the LDS banks
// covers 256 bytes. Rows of 256 bytes or more: the chunk is XORed with r mod 16. Shorter rows
// (nq < 16: 16 / nq rows share a 256-byte span, rows r and r + 16 / nq start on the same bank):
// XORed with (r / (16 / nq)) mod nq, so the rows that share a bank offset take distinct chunks.
__device__ __forceinline__ int swz(int r, int q, int nq) {
    if (nq >= 16) return q ^ (r & 15);
    return q ^ ((r / (16 / nq)) & (nq - 1));
}

// Query operands of group grp: lane (g16, n16) loads fp32 dims 32kb + 8g16 .. +7 of item row
// 16 grp + n16 (a row past the item reads edge 0's query and is dropped later).
template <int D>
__device__ __forceinline__ void load_q(const SparseArgs &a, const int4_t *er, int grp, int nrows,
                                       int h, int lane, float qinv, float4_t (&nq)[D / 32][2]) {
    const int g16 = lane >> 4, n16 = lane & 15;
    const int r = 16 * grp + n16;
    const RowIx x = row_split(r < nrows ? r : 0, a.qhead, qinv);
    const long long qrow = (long long)er[x.ix][1] * (a.hkv * a.qhead) + h * a.qhead + x.qh;
    const float *src = a.q + qrow * D + 8 * g16;
    for (int kb = 0; kb < D / 32; ++kb) {
        nq[kb][0] = gload<float4_t>(src + 32 * kb);
        nq[kb][1] = gload<float4_t>(src + 32 * kb + 4);
    }
}

// The edge groups of one staged key block. The item's rows are its (edge, q-head lane) pairs,
// row r = edge r / qhead, lane r mod qhead; a wave takes 16 consecutive rows at a time (groups
// wave, wave + NW, ...; 16 / qhead whole edges when qhead divides 16). Lane (g16, n16) serves
// row n16 of the group. K (row-major) and V (transposed) are the block's fp16 hi/lo planes, er
// the item's edge records, mmask the mapped-key bits, kshift the block's K scaling shift (K was
// multiplied by 2^kshift) and s_vmul the per-dimension output scales (2^-shift of each V
// dimension); lane and wave are the thread's (a caller may pass values the compiler cannot see
// through, to keep the per-lane offsets from being hoisted out of its loop).
//
// On entry nq holds the query operands of the wave's first group when kPrefetch (loaded and
// waited for by the caller). Each group waits for all of the wave's outstanding memory
// operations right before its stores.
template <int D, int NT, int NW, bool kPrefetch>
__device__ __forceinline__ void edge_groups(const SparseArgs &a, const half_t *Khi,
                                            const half_t *Klo, const half_t *Vhi,
                                            const half_t *Vlo, float *slab, const float *s_vmul,
                                            const int4_t *er, int nrows, int h, int kshift,
                                            const uint64_t (&mmask)[(16 * NT + 63) / 64],
                                            int lane, int wave, float qinv,
                                            float4_t (&nq)[D / 32][2], bool vone) {
    constexpr int BSP = 16 * NT;             // padded keys per block (NT even)
    constexpr int KB = D / 32;               // 32-dim k-blocks of QK^T
    constexpr int NDT = D / 16;              // 16-dim output tiles
    constexpr int KK = NT / 2;               // 32-key k-blocks of PV
    constexpr int KQ = D / 8;                // 16-byte chunks per K row (8 halfs)
    constexpr int VC = BSP / 8;              // 16-byte chunks per V^T row (8 halfs)
    constexpr int MW = (BSP + 63) / 64;      // 64-bit key-mask words
    bool mfull = true;  // every key of the padded block sits on a mapped page
    for (int hw = 0; hw < MW; ++hw) {
        const int nb = BSP - 64 * hw;
        mfull = mfull && mmask[hw] == (nb >= 64 ? ~0ull : (1ull << nb) - 1);
    }
    for (int grp = wave; 16 * grp < nrows; grp += NW) {
        // the lane index through an empty asm statement, once per group: the ~32 per-lane LDS
        // operand offsets are then recomputed in each group rather than held in registers
        // across the loop (which would leave the group's own values short of registers)
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int g16 = ln >> 4, n16 = ln & 15;
        const int row = 16 * grp + n16;
        const bool vrow = row < nrows;
        const RowIx rx = row_split(row, a.qhead, qinv);
        const int ix = vrow ? rx.ix : 0;  // rows past the item read edge 0, then drop it
        const int qh = rx.qh;
        const int e = er[ix][0];
        const int len = vrow ? er[ix][2] : 0;
        if (!kPrefetch) {
            load_q<D>(a, er, grp, nrows, h, ln, qinv, nq);
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        }
        // the row's largest magnitude (its D dims lie in the 4 lanes g16 = 0..3 of column n16),
        // the power of two eQ that brings it into [0.5, 1), and the row scaled by 2^(11 - eQ)
        // and split
        float qmx = 0.f;
        for (int kb = 0; kb < KB; ++kb)
            for (int c = 0; c < 2; ++c)
                for (int i = 0; i < 4; ++i) qmx = fmaxf(qmx, fabsf(nq[kb][c][i]));
        qmx = wave_max_xor(qmx, 16);
        qmx = wave_max_xor(qmx, 32);
        const int eQ = pow2_exp(qmx);
        const int qshift = scale_shift(kOpExp, eQ);
        const float qf = ldexpf(1.f, qshift);
        half8_t qhi[KB], qlo[KB];
        for (int kb = 0; kb < KB; ++kb)
            for (int c = 0; c < 2; ++c)
                for (int i = 0; i < 4; i += 2) {
                    half2_t h2, l2;
                    split16x2(nq[kb][c][i], nq[kb][c][i + 1], qf, h2, l2);
                    qhi[kb][4 * c + i] = h2[0];
                    qhi[kb][4 * c + i + 1] = h2[1];
                    qlo[kb][4 * c + i] = l2[0];
                    qlo[kb][4 * c + i + 1] = l2[1];
                }
        // a score in log2 units is its product sum times mult (> 0)
        const float mult = ldexpf(a.scale_log2, -qshift - kshift);
        // The next group's query operands are loaded here, and the one wait for them sits right
        // before this group's stores. A wait for a load while stores are outstanding has to
        // drain the stores too (loads and stores share the counter and may complete out of
        // order), so loading later would make the next group's first use of its query wait
        // for this group's partial stores to reach memory.
        // (unconditionally: past the last group it reads edge 0's rows, which go unused; a
        // conditional load would make the compiler copy all of nq on both paths)
        if (kPrefetch) load_q<D>(a, er, grp + NW, nrows, h, ln, qinv, nq);
        // S^T tiles: lane holds keys 16j + 4g16 + i of row n16, as product sums.
        float s[NT][4];
        for (int j = 0; j < NT; ++j) {
            // the cross terms hi.lo + lo.hi and hi.hi of each k-block, in one accumulator
            float4_t acc = {0.f, 0.f, 0.f, 0.f};
            const int t = 16 * j + n16;
            for (int kb = 0; kb < KB; ++kb) {
                const int off = t * D + 8 * swz(t, 4 * kb + g16, KQ);
                const half8_t khi = *(const half8_t *)(Khi + off);
                const half8_t klo = *(const half8_t *)(Klo + off);
                acc = mfma16x16x32(khi, qlo[kb], acc);
                acc = mfma16x16x32(klo, qhi[kb], acc);
                acc = mfma16x16x32(khi, qhi[kb], acc);
            }
            for (int i = 0; i < 4; ++i) s[j][i] = acc[i];
            // keep the next tile's LDS operand reads from being hoisted over this tile (each
            // hoisted read holds 4 registers)
            __builtin_amdgcn_sched_barrier(0);
        }
        // Keys past the edge's length or on unmapped pages are excluded (-inf). The test is
        // skipped when every key of the block is mapped and every row of the group sees all of
        // them (the common case; the branch is uniform over the wave).
        if (!(mfull && __ballot(vrow && len < BSP) == 0)) {
            uint64_t lm[MW];  // keys this lane scores (16j + 4g16 + i), mapped and in length
            for (int hw = 0; hw < MW; ++hw) {
                const int rem = len - 64 * hw;
                const uint64_t lenm = rem >= 64 ? ~0ull : (rem <= 0 ? 0ull : (1ull << rem) - 1);
                lm[hw] = (mmask[hw] & lenm) >> (4 * g16);
            }
            for (int j = 0; j < NT; ++j)
                for (int i = 0; i < 4; ++i)
                    if (!((lm[j >> 2] >> (16 * (j & 3) + i)) & 1)) s[j][i] = -INFINITY;
        }
        float mx = -INFINITY;
        for (int j = 0; j < NT; ++j)
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[j][i]);
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);
        // the row maximum in log2 units (0 when every key is excluded)
        const float mu = (mx == -INFINITY) ? 0.f : mx * mult;
        float ls = 0.f;
        float one = 1.f;
        asm volatile("" : "+v"(one));
        half8_t phi[KK], plo[KK];
        for (int j = 0; j < NT; ++j)
            for (int i = 0; i < 4; i += 2) {
                // p = 2^(s mult - mu): an excluded key's exp2(-inf) is 0, and the clamp to [0, 1]
                // (the exp instruction's clamp modifier; p <= 1 up to the rounding of mu) turns a
                // NaN score into 0 (a NaN counts as excluded, as the page's "score >
                // NEG_LARGE/2" test does)
                const float e0 = __builtin_amdgcn_exp2f(fmaf(s[j][i], mult, -mu));
                const float e1 = __builtin_amdgcn_exp2f(fmaf(s[j][i + 1], mult, -mu));
                const float p0 = fminf(fmaxf(e0, 0.f), 1.f);
                const float p1 = fminf(fmaxf(e1, 0.f), 1.f);
                ls += p0;
                ls += p1;
                half2_t h2, l2;
                split16x2u(p0, p1, one, h2, l2);
                phi[j >> 1][4 * (j & 1) + i] = h2[0];
                phi[j >> 1][4 * (j & 1) + i + 1] = h2[1];
                plo[j >> 1][4 * (j & 1) + i] = l2[0];
                plo[j >> 1][4 * (j & 1) + i + 1] = l2[1];
            }
        ls += __shfl_xor(ls, 16, 64);
        ls += __shfl_xor(ls, 32, 64);

        // O^T = V^T . P^T: rows are dims 16dt + 4g16 + i, column n16 is the lane's query row;
        // k-slot (g16, 4u + i) is key 32kk + 16u + 4g16 + i on both operands.
        float4_t o[NDT];
        for (int dt = 0; dt < NDT; ++dt) o[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < KK; ++kk) {
            for (int dt = 0; dt < NDT; ++dt) {
                const int r = 16 * dt + n16;
                const int off = r * BSP + 8 * swz(r, 4 * kk + g16, VC);
                const half8_t vhi = *(const half8_t *)(Vhi + off);
                const half8_t vlo = *(const half8_t *)(Vlo + off);
                o[dt] = mfma16x16x32(vlo, phi[kk], o[dt]);
                o[dt] = mfma16x16x32(vhi, plo[kk], o[dt]);
                o[dt] = mfma16x16x32(vhi, phi[kk], o[dt]);
                if (dt % 2 == 1) __builtin_amdgcn_sched_barrier(0);
            }
        }
        // Stores, o scaled back by each dim's s_vmul. Lane (g16, n16) holds dims 16dt + 4g16 .. +3
        // of row n16, so a direct store instruction would write 64 bytes into each of 16 rows; at
        // this occupancy that writes HBM about 20% slower than whole 128-byte lines. Each
        // 128-byte line j of 8 rows goes through the wave's 1 KB LDS slab instead and leaves as
        // one store of 8 whole lines (lane l: row 8h + l/8, dims 32j + 4(l%8) ..), non-temporal
        // (the 2 GB of partials are read back only by the merge), scaled on the way out. m and
        // l come from g16 == 0.
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the next group's query loads (above)
        if (vrow && g16 == 0) {
            const long long p = (long long)e * a.qhead + qh;
            // 16 bytes per edge and array, scattered: non-temporal, like the o rows
            __builtin_nontemporal_store((mx == -INFINITY) ? kNegLarge : mu * kLn2, a.m + p);
            __builtin_nontemporal_store(ls, a.l + p);
        }
        const int lr = ln >> 3;  // the slab row this lane reads: row 8h + lr of the group
        float *dst[2];
        bool rvalid[2];
        for (int h = 0; h < 2; ++h) {
            const int r = 16 * grp + 8 * h + lr;  // the item row this lane stores
            rvalid[h] = r < nrows;
            const RowIx rs = row_split(rvalid[h] ? r : 0, a.qhead, qinv);
            dst[h] = a.o + ((long long)er[rs.ix][0] * a.qhead + rs.qh) * D + 4 * (ln & 7);
        }
        // slab row r (128 bytes) holds its 16-byte chunk c at c ^ ((r >> 1) & 3): the 8 rows
        // written at one chunk, and the two rows read per 16 lanes, then cover distinct banks
        // (rows r and r + 2 start on the same bank)
        const int wr = n16 & 7, wx = (wr >> 1) & 3;  // the slab row this lane writes
        // (two copies of the loop: with the per-dimension scales, and without them when no
        // dimension of V is scaled)
        auto lines = [&](auto scaled) {
            for (int j = 0; j < NDT / 2; ++j) {
                // the output scales of the 4 dims this lane stores in line j
                float4_t mj;
                if constexpr (decltype(scaled)::value)
                    mj = *(const float4_t *)(s_vmul + 32 * j + 4 * (ln & 7));
                for (int h = 0; h < 2; ++h) {
                    if ((n16 >> 3) == h) {
                        *(float4_t *)(slab + wr * 32 + 4 * (g16 ^ wx)) = o[2 * j];
                        *(float4_t *)(slab + wr * 32 + 16 + 4 * (g16 ^ wx)) = o[2 * j + 1];
                    }
                    float4_t v =
                        *(const float4_t *)(slab + lr * 32 + 4 * ((ln & 7) ^ ((lr >> 1) & 3)));
                    if constexpr (decltype(scaled)::value) v = v * mj;
                    if (rvalid[h]) __builtin_nontemporal_store(v, (float4_t *)(dst[h] + 32 * j));
                }
            }
        };
        if (vone)
            lines(std::false_type{});
        else
            lines(std::true_type{});
    }
}


// Workgroup per work item: stages its key block from HBM into the fp16 planes, then runs the
// edge groups. For the shapes whose planes and raw rows do not both fit in LDS (D = 256, or
// 128-key blocks at D = 128).
template <int D, int NT>
__global__ __launch_bounds__(kThreads, (NT * D <= 512 && D <= 128) ? 4 : 2) void sp_main(
    SparseArgs a, SparseWs w) {
    constexpr int BSP = 16 * NT;             // padded keys per block (NT even)
    constexpr int KQ = D / 8;                // 16-byte chunks per K row (8 halfs)
    constexpr int VC = BSP / 8;              // 16-byte chunks per V^T row (8 halfs)
    constexpr int NW = kThreads / 64;        // waves
    constexpr int MW = (BSP + 63) / 64;      // 64-bit key-mask words
    static_assert(kChunk <= kThreads, "one thread per staged edge");
    extern __shared__ half_t lds[];
    half_t *Khi = lds, *Klo = lds + BSP * D;
    half_t *Vhi = lds + 2 * BSP * D, *Vlo = lds + 3 * BSP * D;
    // per wave: 8 rows x 128 bytes of partial output on their way to a whole-line store; while
    // the block is staged, the same 8 KB hold the per-wave, per-dimension maxima of |V|
    float *slabs = (float *)(lds + 4 * BSP * D);
    float *slab = slabs + (threadIdx.x >> 6) * 256;
    static_assert(NW * D <= NW * 256, "per-wave |V| maxima fit the store slabs");
    __shared__ float s_kmax[NW];                        // per-wave maxima of |K|
    __shared__ int s_len[NW];                           // per-wave longest edge
    __shared__ int s_ev[D];                             // per-dimension scaling shift of V
    __shared__ int s_vscaled;                           // some dimension of V is scaled
    // 2^-s_ev: output scale per dimension, read as float4 (16-byte aligned)
    __shared__ __attribute__((aligned(16))) float s_vmul[D];
    __shared__ __attribute__((aligned(16))) int4_t s_er[kChunk];  // the item's edge records

    // The item's record is read together with the item count (item < max_items: inside the
    // workspace; a record past the count holds no defined value and is not used).
    const int item = blockIdx.x;
    const int nitems = w.nitems[0];
    const int4_t rec = w.items[2 * item], pg = w.items[2 * item + 1];
    if (item >= nitems) return;
    const int u = rec[0], ebeg = rec[1], nE = rec[2];
    const int blk = u % a.nblk;
    const int bh = u / a.nblk;
    const int h = bh % a.hkv;
    const int b = bh / a.hkv;
    const int32_t *btrow = a.bt + (long long)b * a.max_pages;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    // The item's sorted edge records (id, query index, key count) are loaded first; the K and V
    // loads follow at once (page ids from the item record; for blocks of more than 4 pages they
    // wait for the table entries), and the edge records go to LDS after them (loads return in
    // order: this waits for the records only).
    const bool has_edge = (int)threadIdx.x < nE;
    int4_t erec = {0, 0, 0, 0};
    if (has_edge) erec = w.edges[ebeg + threadIdx.x];

    auto row_ptr = [&](const float *base, int pid, int t) {
        return base + (((long long)pid * a.hkv + h) * a.page_size + t % a.page_size) * D;
    };

    // ---- stage the key block. A task is 4 consecutive keys x 8 dims of K and of V (32 + 32
    // floats): dims 4q .. 4q+3 and D/2 + 4q .. +3, so that the 16-byte loads of the D/8 lanes of
    // a key quad read whole contiguous half rows (a load instruction of 16-byte pieces at a
    // 32-byte stride reads HBM more slowly), non-temporal. Pass 1 loads and takes the block-wide
    // max |K| and the per-dimension max |V|; pass 2 scales by the powers of two, splits into
    // fp16 planes and stores K row-major and V transposed. One task per thread: the pass-1
    // registers are reused.
    constexpr int TASKS = BSP / 4 * KQ;                       // (key quad, 8-dim chunk) pairs
    static_assert(TASKS <= kThreads && TASKS % 64 == 0, "one task per thread, whole waves");
    float kr[4][8], vr[4][8];
    const int task = threadIdx.x;
    const bool has_task = task < TASKS;
    const int t4 = task / KQ, q = task - t4 * KQ;
    // page of key t: from the item record (blocks of up to 4 pages) or the table
    auto page_of = [&](int t) {
        if (a.ppb > 4) return block_page(a, btrow, blk, t);
        if (t >= a.block_size) return -1;
        const int sl = t / a.page_size;
        return sl == 0 ? pg[0] : (sl == 1 ? pg[1] : (sl == 2 ? pg[2] : pg[3]));
    };
    int pids[4];
    for (int r = 0; r < 4; ++r) pids[r] = has_task ? page_of(4 * t4 + r) : -1;
    // mapped-key masks (wave-uniform): bit t set when key t sits on a mapped page
    uint64_t mmask[MW];
    for (int hw = 0; hw < MW; ++hw) {
        const int t = 64 * hw + lane;
        mmask[hw] = __ballot(t < BSP && page_of(t) >= 0);
    }
    for (int r = 0; r < 4; ++r) {
        const int t = 4 * t4 + r;
        const int pid = pids[r];
        for (int x = 0; x < 8; ++x) { kr[r][x] = 0.f; vr[r][x] = 0.f; }
        if (pid >= 0) {
            const float *pk = row_ptr(a.kp, pid, t) + 4 * q;
            const float *pv = row_ptr(a.vp, pid, t) + 4 * q;
            const float4_t k0 = gload_nt<float4_t>(pk), k1 = gload_nt<float4_t>(pk + D / 2);
            const float4_t v0 = gload_nt<float4_t>(pv), v1 = gload_nt<float4_t>(pv + D / 2);
            for (int x = 0; x < 4; ++x) {
                kr[r][x] = k0[x]; kr[r][4 + x] = k1[x];
                vr[r][x] = v0[x]; vr[r][4 + x] = v1[x];
            }
        }
    }
    if (has_edge) s_er[threadIdx.x] = erec;
    if (threadIdx.x == 0) s_vscaled = 0;
    // Keys at or past the item's longest edge serve none of its edges; past a sequence's used
    // length a mapped page may hold stale rows, NaN included. Those keys' rows are stored as
    // zeros in the planes (the maxima below skip NaN), so that nothing of them reaches the
    // output, not even as 0 * NaN in the PV products.
    int lmax = has_edge ? erec[2] : 0;
    for (int o = 32; o > 0; o >>= 1) lmax = max(lmax, __shfl_xor(lmax, o, 64));
    if (lane == 0) s_len[wave] = lmax;
    float mk = 0.f, mv[8];
    for (int x = 0; x < 8; ++x) {
        mv[x] = 0.f;
        for (int r = 0; r < 4; ++r) {
            mk = fmaxf(mk, fabsf(kr[r][x]));
            mv[x] = fmaxf(mv[x], fabsf(vr[r][x]));
        }
    }
    for (int o = 32; o > 0; o >>= 1) mk = fmaxf(mk, __shfl_xor(mk, o, 64));
    // lanes l, l + KQ, ... hold the same dims (q = lane mod KQ): reduce over them
    for (int o = KQ; o < 64; o <<= 1)
        for (int x = 0; x < 8; ++x) mv[x] = fmaxf(mv[x], __shfl_xor(mv[x], o, 64));
    if (lane == 0) s_kmax[wave] = mk;
    if (lane < KQ) {
        float *vw = slabs + wave * D;
        for (int x = 0; x < 4; ++x) {
            vw[4 * q + x] = mv[x];
            vw[D / 2 + 4 * q + x] = mv[4 + x];
        }
    }
    __syncthreads();
    // the first group's query rows, loaded while the block is split (the edge records are in
    // LDS since the barrier above)
    constexpr bool kPrefetchQ = D <= 128;
    const int nrows = nE * a.qhead;
    float4_t nq[D / 32][2];
    const float qinv = 1.f / (float)a.qhead;
    if (kPrefetchQ && 16 * wave < nrows) load_q<D>(a, s_er, wave, nrows, h, lane, qinv, nq);
    for (int i = 0; i < NW; ++i) mk = fmaxf(mk, s_kmax[i]);
    const int kshift = scale_shift(kOpExp, pow2_exp(mk));
    if ((int)threadIdx.x < D) {
        float m = 0.f;
        for (int i = 0; i < NW; ++i) m = fmaxf(m, slabs[i * D + threadIdx.x]);
        const int e = pow2_exp(m);
        int vsh = scale_shift(0, e);
        if (e <= 15) vsh = max(vsh, 0);  // from 0.5 up to 2^15: split as it is
        s_ev[threadIdx.x] = vsh;
        s_vmul[threadIdx.x] = ldexpf(1.f, -vsh);
        if (vsh != 0) s_vscaled = 1;
    }
    __syncthreads();
    const bool vone = s_vscaled == 0;  // uniform: no dimension of V is scaled
    if (has_task) {
        const float kf = ldexpf(1.f, kshift);
        lmax = 0;
        for (int i = 0; i < NW; ++i) lmax = max(lmax, s_len[i]);
        lmax = __builtin_amdgcn_readfirstlane(lmax);  // uniform
        if (lmax < BSP)  // uniform: some keys of the block serve no edge
            for (int r = 0; r < 4; ++r)
                if (4 * t4 + r >= lmax)
                    for (int x = 0; x < 8; ++x) { kr[r][x] = 0.f; vr[r][x] = 0.f; }
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * t4 + r;
            half8_t hi, lo;
            for (int x = 0; x < 8; x += 2) {
                half2_t h2, l2;
                split16x2(kr[r][x], kr[r][x + 1], kf, h2, l2);
                hi[x] = h2[0];
                hi[x + 1] = h2[1];
                lo[x] = l2[0];
                lo[x + 1] = l2[1];
            }
            // dims 4q .. are chunk q/2, dims D/2 + 4q .. chunk KQ/2 + q/2, at half (q & 1)
            const int off0 = t * D + 8 * swz(t, q >> 1, KQ) + 4 * (q & 1);
            const int off1 = t * D + 8 * swz(t, KQ / 2 + (q >> 1), KQ) + 4 * (q & 1);
            *(half4_t *)(Khi + off0) = half4_t{hi[0], hi[1], hi[2], hi[3]};
            *(half4_t *)(Klo + off0) = half4_t{lo[0], lo[1], lo[2], lo[3]};
            *(half4_t *)(Khi + off1) = half4_t{hi[4], hi[5], hi[6], hi[7]};
            *(half4_t *)(Klo + off1) = half4_t{lo[4], lo[5], lo[6], lo[7]};
        }
        // V^T row d holds, in 16-byte chunk 4c + g of a 32-key block c, the keys
        // 32c + 4g .. +3 and 32c + 16 + 4g .. +3: the k-slots (g, 0..7) of one PV operand.
        const int vq = 4 * (t4 >> 3) + (t4 & 3), vh = 4 * ((t4 >> 2) & 1);
        for (int x = 0; x < 8; ++x) {
            const int d = x < 4 ? 4 * q + x : D / 2 + 4 * q + (x - 4);
            const float vf = ldexpf(1.f, s_ev[d]);
            half4_t hi, lo;
            for (int r = 0; r < 4; r += 2) {
                half2_t h2, l2;
                split16x2(vr[r][x], vr[r + 1][x], vf, h2, l2);
                hi[r] = h2[0];
                hi[r + 1] = h2[1];
                lo[r] = l2[0];
                lo[r + 1] = l2[1];
            }
            const int off = d * BSP + 8 * swz(d, vq, VC) + vh;
            *(half4_t *)(Vhi + off) = hi;
            *(half4_t *)(Vlo + off) = lo;
        }
    }
    __syncthreads();

    // With D <= 128 each group's query operands are loaded one group ahead (the first during
    // the split above). At D = 256 the second set of query registers does not fit: each group
    // loads its own rows.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    edge_groups<D, NT, NW, kPrefetchQ>(a, Khi, Klo, Vhi, Vlo, slab, s_vmul, s_er, nrows, h,
                                       kshift, mmask, lane, wave, qinv, nq, vone);
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

size_t sparse_workspace_bytes(int E, int units, long long qrows, int D) {
    (void)qrows;  // the query rows are split in registers: no per-row workspace
    (void)D;
    return layout(nullptr, nullptr, E, units) * 4;
}

pa_status launch_sparse(const SparseArgs &a, hipStream_t stream) {
    int nt = 2;
    while (16 * nt < a.block_size) nt *= 2;
    if ((a.D != 64 && a.D != 128 && a.D != 256) || (a.D == 256 && nt > 4))
        return PA_ERR_UNSUPPORTED;
    // the K and V hi/lo planes, then one 1 KB store slab per wave, as dynamic LDS, plus the
    // kernel's static arrays (edge records, maxima, per-dimension V scales: 3.6 KB at D = 128).
    // At D = 256 the planes of a 128-key block exceed the LDS: blocks of up to 64 keys.
    const size_t lds = (size_t)4 * 16 * nt * a.D * sizeof(half_t) + (kThreads / 64) * 1024;
    if (lds + 4096 > sparse_lds_limit()) return PA_ERR_UNSUPPORTED;
    LaunchScope scope("sparse_forward", stream, 5);
    SparseWs w;
    layout(&w, a.ws, a.E, a.units);
    const int eg = (a.E + 255) / 256;
    if (w.chunked) {
        scope.launch(sp_chist, dim3(w.chunks), dim3(kHistThreads), (uint32_t)(4 * a.units), a, w);
        scope.launch(sp_cprefix, dim3(w.nscan), dim3(kUnitsPerScan), 0, a, w);
        scope.launch(sp_wscan, dim3(1), dim3(1024), 0, w);
        scope.launch(sp_cscatter, dim3((std::max(a.E, a.units) + 255) / 256), dim3(256), 0, a, w);
    } else {
        scope.launch(sp_zero, dim3((a.units + 255) / 256), dim3(256), 0, w.counts, a.units);
        scope.launch(sp_hist, dim3(eg), dim3(256), 0, a, w);
        scope.launch(sp_scan, dim3(1), dim3(1024), 0, a, w);
        scope.launch(sp_scatter, dim3(eg), dim3(256), 0, a, w);
    }
#define PA_SP_LAUNCH(DD, NN) \
    scope.launch(sp_main<DD, NN>, dim3(w.max_items), dim3(kThreads), (uint32_t)lds, a, w)
    if (a.D == 256) {
        if (nt == 2) PA_SP_LAUNCH(256, 2);
        else PA_SP_LAUNCH(256, 4);
    } else if (a.D == 128) {
        if (nt == 2) PA_SP_LAUNCH(128, 2);
        else if (nt == 4) PA_SP_LAUNCH(128, 4);
        else PA_SP_LAUNCH(128, 8);
    } else {
        if (nt == 2) PA_SP_LAUNCH(64, 2);
        else if (nt == 4) PA_SP_LAUNCH(64, 4);
        else PA_SP_LAUNCH(64, 8);
    }
#undef PA_SP_LAUNCH
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa
