// prefill.hip -- prefill dispatch and the packed-batch schedule.
//
// Packed batches (cu_seqlens) can hold sequences of very different lengths;
// each (sequence, head, value slice) is one chain workgroup that walks its
// chunks in order, so the longest sequence sets the critical path.  A tiny
// kernel ranks the sequences longest first (ties by index, so the schedule is
// deterministic) and the chain kernel maps its workgroups in that order,
// letting the long chains start first.  The same kernel gives each sequence
// its first slot in the per-chunk record array (prefix sum of its chunk
// counts; quadratic in the number of sequences, which is small).
#include <algorithm>

#include "launch.h"
#include "prefill_shapes.h"

namespace gdr {

hipError_t launch_prefill_bf16_gdn(const PrefillArgs &a, hipStream_t st);
hipError_t launch_prefill_bf16_kda(const PrefillArgs &a, hipStream_t st);
hipError_t launch_prefill_f32_gdn(const PrefillArgs &a, hipStream_t st);
hipError_t launch_prefill_f32_kda(const PrefillArgs &a, hipStream_t st);
int chain_blocks_per_cu_bf16_gdn(int dk, int dv_slice, int chunk);
int chain_blocks_per_cu_bf16_kda(int dk, int dv_slice, int chunk);
int chain_blocks_per_cu_f32_gdn(int dk, int dv_slice, int chunk);
int chain_blocks_per_cu_f32_kda(int dk, int dv_slice, int chunk);

__global__ __launch_bounds__(256) void schedule_kernel(const int32_t *__restrict__ cu, int n, int chunk,
                                                       int32_t *__restrict__ order, int32_t *__restrict__ choff) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int li = cu[i + 1] - cu[i];
    int rank = 0, off = 0;
    for (int j = 0; j < n; ++j) {
        const int lj = cu[j + 1] - cu[j];
        rank += (lj > li) || (lj == li && j < i);
        if (j < i) off += (lj + chunk - 1) / chunk;
    }
    order[rank] = i;
    choff[i] = off;
    if (i == n - 1) choff[n] = off + (li + chunk - 1) / chunk;
}

bool prefill_supported(bool bf16, bool kda, int dk, int dv_slice, int chunk) {
#define GDR_CASE(DK_, DVS_, C_) if (dk == DK_ && dv_slice == DVS_ && chunk == C_) return true;
    if (bf16 && kda) {
        GDR_PREFILL_BF16_KDA_SHAPES(GDR_CASE)
    } else if (bf16) {
        GDR_PREFILL_BF16_GDN_SHAPES(GDR_CASE)
    } else if (kda) {
        GDR_PREFILL_F32_KDA_SHAPES(GDR_CASE)
    } else {
        GDR_PREFILL_F32_GDN_SHAPES(GDR_CASE)
    }
#undef GDR_CASE
    return false;
}

// Automatic value-slice width.  A chain workgroup walks all chunks of its
// (sequence, head, slice) in order, so the call takes about one such walk per
// round of workgroups the device holds at once.  The narrower slice gives
// more, lighter workgroups; it is chosen only when it needs no more rounds
// than the wider one (a d_k = 128 chain workgroup fills a CU's LDS, so one
// round is one workgroup per CU).
int auto_dv_slice(bool bf16, bool kda, int dk, int dv, int chunk, long units) {
    if (!bf16 || dv % 32 != 0 || !prefill_supported(bf16, kda, dk, 32, chunk)) return 16;
    if (!prefill_supported(bf16, kda, dk, 16, chunk)) return 32;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;                                   // no device to ask: MI355X
    auto rounds = [&](int dvs) {
        int per_cu = kda ? chain_blocks_per_cu_bf16_kda(dk, dvs, chunk) : chain_blocks_per_cu_bf16_gdn(dk, dvs, chunk);
        const long cap = (long)cus * (per_cu > 0 ? per_cu : 1);
        return (units * (dv / dvs) + cap - 1) / cap;
    };
    // the narrowest width among those that need the fewest rounds (a slice
    // fetches its chunk's whole record whatever its width, so wider slices
    // only pay when they save a round)
    int best = 32;
    long best_r = rounds(32);
    if (dv % 64 == 0 && prefill_supported(bf16, kda, dk, 64, chunk)) {
        const long r64 = rounds(64);
        if (r64 < best_r) best = 64, best_r = r64;
    }
    return rounds(16) <= best_r ? 16 : best;
}

hipError_t launch_schedule(const int32_t *cu, int n, int chunk, int32_t *order, int32_t *chunk_offset,
                           hipStream_t st) {
    hipLaunchKernelGGL(schedule_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, cu, n, chunk, order,
                       chunk_offset);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st) {
    if (a.num_seqs == 0 || a.num_heads == 0) return hipSuccess;
    if (a.cu_seqlens) {
        const hipError_t e = launch_schedule(a.cu_seqlens, a.num_seqs, a.chunk, a.order, a.chunk_offset, st);
        if (e != hipSuccess) return e;
    }
    if (a.bf16) return a.kda ? launch_prefill_bf16_kda(a, st) : launch_prefill_bf16_gdn(a, st);
    return a.kda ? launch_prefill_f32_kda(a, st) : launch_prefill_f32_gdn(a, st);
}

}  // namespace gdr
