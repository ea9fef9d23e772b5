// Paged GQA attention for gfx950: the device planner and the MFMA decode kernel (query rows of
// sequences with few new tokens; longer ones go to the prefill kernel).
//
// Operation: the PagedAttention op of the "com.microsoft.PagedAttention ... manifest.json" page
// (passes "main", "split_attention" and "merge"): every query row attends, per kv head, to the
// keys of its sequence that a block table maps into an fp16 cache [NB, bs, G, D]; the key range
// may be cut into chunks whose (o, m, l) partials a log-sum-exp merge combines.
//
// MI355X design (not the page's WebGPU one):
//  * One wave64 per (work item, kv head). A work item is all query rows of a decode-like sequence
//    and a key chunk. The wave serves every query head of the kv group, so each K/V byte of the
//    chunk is read from HBM once per work item.
//  * QK^T and PV run on MFMA v_mfma_f32_16x16x32_f16. The score tile is S^T = K . Q^T with
//    16 keys as rows and 16 (token, head) columns. K rows are copied whole (256 bytes at D = 128,
//    4 rows per copy instruction) from the cache into the wave's own LDS tile and read back in
//    the A-operand layout: loaded straight into that layout, each instruction would fetch 64
//    bytes of 16 different rows, which reads HBM about 8% slower. The tile's C layout already
//    gives each lane 8 keys of one column, exactly the k-slots of the P operand of O = P . V.
//    The V operand wants 8 keys of one dimension per lane; V is loaded as 16-byte row chunks
//    (fully coalesced, 4 rows per load) and transposed in registers with byte permutes.
//  * Online softmax in base 2 (scores pre-multiplied by scale*log2 e); the stored partial max is
//    converted back to natural-log units. Column max/sum reductions are two cross-row shuffles.
//  * A persistent grid walks the planner's item list; the planner (one workgroup) reads the
//    sequence lengths on the device and picks the chunk size, so the host never waits on data.
#include "common.h"
#include "decode_unit.h"
#include "plan.h"

#include <math.h>

namespace pa {

// ============================================================================================
// Device planner (body in plan.h)
// ============================================================================================
template <int TH>  // threads: 64 (one wave) or kPlanThreads
__global__ __launch_bounds__(TH) void plan_kernel(PlanArgs a) {
    plan_body<TH>(a);
}

pa_status launch_plan(const PlanArgs &a, hipStream_t stream) {
    LaunchScope scope("plan", stream);
    // one wave when the batch fits in it: the scans and barriers stay inside the wave
    if (a.B <= 64) scope.launch(plan_kernel<64>, dim3(1), dim3(64), 0, a);
    else scope.launch(plan_kernel<kPlanThreads>, dim3(1), dim3(kPlanThreads), 0, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// ============================================================================================
// Attention kernel
// ============================================================================================
namespace {
// Persistent decode kernel: decode_loop over workgroups of a.gw waves, each with its own LDS
// K tile. At D = 256 a workgroup has at most 4 waves, one per SIMD, so that each can hold its
// 256-dim query, output and V tiles in registers.
template <int D, int NCB, bool POW2, bool NT>
__global__ __launch_bounds__(NCB == 1 ? (D == 256 ? 256 : 512) : 64) void attn_kernel(AttnArgs a) {
    extern __shared__ half_t s_ktile[];  // one 32-key K tile per wave: [gw][32][D]
    __shared__ int s_unit;
    decode_loop<D, NCB, POW2, NT>(a, blockIdx.x, s_ktile + (threadIdx.x >> 6) * (kTileKeys * D),
                                  &s_unit);
}

template <int D, int NCB, bool NT>
pa_status launch_d_ncb(const AttnArgs &a, int blocks, LaunchScope &scope) {
    const dim3 g(blocks), blk(64 * a.gw);
    const uint32_t lds = (uint32_t)(a.gw * kTileKeys * D * sizeof(half_t));  // <= 128 KB
    if (a.log2bs >= 0)
        scope.launch(attn_kernel<D, NCB, true, NT>, g, blk, lds, a);
    else
        scope.launch(attn_kernel<D, NCB, false, NT>, g, blk, lds, a);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

template <int D, bool NT>
pa_status launch_d(const AttnArgs &a, int ncb, int blocks, LaunchScope &scope) {
    if constexpr (D == 256) {  // wider kv groups are split into groups of <= 16 query heads
        if (ncb != 1) return PA_ERR_UNSUPPORTED;
        return launch_d_ncb<D, 1, NT>(a, blocks, scope);
    }
    switch (ncb) {
        case 1: return launch_d_ncb<D, 1, NT>(a, blocks, scope);
        case 2: return launch_d_ncb<D, 2, NT>(a, blocks, scope);
        case 4: return launch_d_ncb<D, 4, NT>(a, blocks, scope);
        default: return PA_ERR_UNSUPPORTED;
    }
}

}  // namespace

pa_status launch_attention(const AttnArgs &a, int D, int ncb, int blocks, const char *name,
                           hipStream_t stream) {
    LaunchScope scope(name, stream);
    if (blocks <= 0) return PA_OK;
    // decode reads each K/V byte once: non-temporal loads
    switch (D) {
        case 64: return launch_d<64, true>(a, ncb, blocks, scope);
        case 128: return launch_d<128, true>(a, ncb, blocks, scope);
        case 256: return launch_d<256, true>(a, ncb, blocks, scope);
        default: return PA_ERR_UNSUPPORTED;
    }
}

}  // namespace pa
