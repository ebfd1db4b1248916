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

#include "fused_impl.h"
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
    return rounds(32) < rounds(16) ? 32 : 16;
}

hipError_t launch_schedule(const int32_t *cu, int n, int chunk, int32_t *order, int32_t *chunk_offset,
                           hipStream_t st) {
    hipLaunchKernelGGL(schedule_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, cu, n, chunk, order,
                       chunk_offset);
    return hipGetLastError();
}

hipError_t launch_fused_gdn(const FusedArgs &fa, int dk, int dvs, int grid, hipStream_t st);
hipError_t launch_fused_kda(const FusedArgs &fa, int dk, int dvs, int grid, hipStream_t st);

// Fused prefill: d_k in {32, 64, 128}; value slices of 16 or 32 channels (a
// 64-channel slice needs a fourth chain wave, which leaves too few registers
// per wave).
bool fused_supported(bool kda, int dk, int dvs) {
    (void)kda;
    if (!(dk == 32 || dk == 64 || dk == 128)) return false;
    return dvs == 16 || dvs == 32;
}

namespace {
size_t r256(size_t b) { return (b + 255) & ~size_t(255); }
int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;   // no device to ask: MI355X
    return cus;
}
}  // namespace

// One fused workgroup fills a CU's LDS, so the device holds one per CU; all
// workgroups of a call must be resident together (the slices of a group wait
// on one another), so the grid never exceeds the CU count.  A group of NS
// slices serves units in turn; the groups per XCD cover the largest number of
// units any XCD receives, up to what the CUs hold.  The slice width is the
// narrowest whose groups all fit at once (most workgroups, most record
// producers per unit), else the widest compiled.
FusedPlan fused_plan(bool kda, int dk, int dv, int num_seqs, int num_heads, int num_qk_heads, int dvs_req,
                     bool packed) {
    FusedPlan pl;
    const int cap = device_cus();
    const int G = num_heads / num_qk_heads;
    const long NP = (long)num_seqs * num_qk_heads;
    const long per_xcd = (NP + 7) / 8 * G;              // units on the busiest XCD
    int dvs = dvs_req;
    if (!dvs) {
        for (int cand : {16, 32}) {
            if (dv % cand || !fused_supported(kda, dk, cand)) continue;
            dvs = cand;                                     // widest so far
            if ((long)8 * per_xcd * (dv / cand) <= cap) break;
        }
    }
    if (!dvs || dv % dvs || !fused_supported(kda, dk, dvs)) return pl;
    const int ns = dv / dvs;
    if (8 * ns > cap) return pl;                           // one group per XCD must fit
    pl.dvs = dvs;
    pl.ns = ns;
    // ring depth: the records being built (one per slice) and the ones the
    // loaders and chains still read
    pl.d = ns + 2;
    pl.gpx = (int)std::max<long>(1, std::min<long>(per_xcd, cap / (8 * ns)));
    pl.ngroups = 8 * pl.gpx;
    pl.grid = pl.ngroups * ns;
    size_t off = 0;
    if (packed) {
        pl.order_off = off;
        off += r256(4 * (size_t)num_seqs);
        pl.choff_off = off;
        off += r256(4 * ((size_t)num_seqs + 1));
    }
    pl.ctl_off = off;
    off += r256(4 * ((size_t)pl.ngroups * (pl.d + 2 * ns) + 1));
    pl.ring_off = off;
    off += (size_t)pl.ngroups * pl.d * fused_record_bytes(dk, kda);
    pl.scratch_off = off;
    off += (size_t)pl.grid * fused_scratch_bytes(dk, kda);
    pl.total = off;
    return pl;
}

hipError_t launch_prefill_fused(const PrefillArgs &a, hipStream_t st) {
    if (a.num_seqs == 0 || a.num_heads == 0) return hipSuccess;
    if (a.cu_seqlens) {
        const hipError_t e = launch_schedule(a.cu_seqlens, a.num_seqs, a.chunk, a.order, a.chunk_offset, st);
        if (e != hipSuccess) return e;
    }
    FusedArgs fa;
    fa.T = a.seqlen;
    fa.H = a.num_heads;
    fa.HK = a.num_qk_heads;
    fa.G = a.num_heads / a.num_qk_heads;
    fa.DV = a.dv;
    fa.num_seqs = a.num_seqs;
    fa.NS = a.f_ns;
    fa.D = a.f_d;
    fa.ngroups = a.f_ngroups;
    fa.gpx = a.f_gpx;
    fa.scale = a.scale;
    fa.gate_bf16 = a.gate_bf16;
    fa.out_bf16 = a.out_bf16;
    fa.q = a.q; fa.k = a.k; fa.v = a.v;
    fa.beta = a.beta;
    fa.log_alpha = a.log_alpha;
    fa.state_in = a.initial_state;
    fa.state_out = a.final_state;
    fa.cu = a.cu_seqlens;
    fa.order = a.cu_seqlens ? a.order : nullptr;
    fa.ring = a.f_ring;
    fa.scratch = a.f_scratch;
    fa.ctl = a.f_ctl;
    fa.out = a.out;
    return a.kda ? launch_fused_kda(fa, a.dk, a.dv_slice, a.f_grid, st)
                 : launch_fused_gdn(fa, a.dk, a.dv_slice, a.f_grid, st);
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t st) {
    if (a.fused) return launch_prefill_fused(a, st);
    if (a.num_seqs == 0 || a.num_heads == 0) return hipSuccess;
    if (a.cu_seqlens) {
        const hipError_t e = launch_schedule(a.cu_seqlens, a.num_seqs, a.chunk, a.order, a.chunk_offset, st);
        if (e != hipSuccess) return e;
    }
    if (a.bf16) return a.kda ? launch_prefill_bf16_kda(a, st) : launch_prefill_bf16_gdn(a, st);
    return a.kda ? launch_prefill_f32_kda(a, st) : launch_prefill_f32_gdn(a, st);
}

}  // namespace gdr
