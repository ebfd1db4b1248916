// decode.hip -- fused decode step of the gated delta rule for gfx950.
//
// One token per sequence.  For each (sequence, head) the d_v x d_k fp32 state
// is streamed once from HBM and once back (page "How the New Flash Models
// Work: Inside GLM-5.3-Flash and Qwen3.8-Flash-Next", section "What a
// generated token costs": decode does little arithmetic per byte moved).  Per
// state row i (a value channel), with the decay alpha = exp(log_alpha)
// (scalar per head, or one per key channel):
//     s'   = s * alpha                         (S Diag(alpha))
//     x_i  = s' . k,   y_i = s' . q
//     u_i  = beta (v_i - x_i)
//     s    = s' + u_i k                         (written back in place)
//     o_i  = scale * (y_i + u_i (k . q))        (= (S_new q)_i, no second read)
// which is the Gated DeltaNet / Kimi Delta Attention update of the section
// "Linear attention: a fixed-size memory in place of the cache" of that page,
// applied row by row.
//
// Layout of the work: one 256-thread workgroup per (sequence, head); each row
// is spread over DK/4 consecutive lanes that hold 4 consecutive columns each
// (16-byte loads/stores, so a wave reads 1 KiB of contiguous state per
// instruction).  The two row dot products are finished with cross-lane sums
// inside the row's lane group.  Rows are independent, so a thread keeps RB
// rows in flight at once to cover HBM latency.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace gdr {

// EXACT: d_v is a multiple of the rows one pass covers, so no row index
// needs a bounds check (measured ~5% faster at d = 128); OUTB: bf16 outputs.
template <int DK, bool KDA, typename QT, int RB, bool EXACT, bool OUTB>
__global__ __launch_bounds__(256) void decode_kernel(
    int H, int DV, const QT *__restrict__ q, const QT *__restrict__ k, const QT *__restrict__ v,
    const float *__restrict__ beta, const float *__restrict__ log_alpha, float *__restrict__ state,
    float scale, void *__restrict__ out) {
    constexpr int LPR = DK / 4;          // lanes per state row
    constexpr int RPP = 256 / LPR;       // rows covered by the workgroup per pass
    const int unit = blockIdx.x;         // n * H + h
    const int lane = threadIdx.x % LPR;
    const int rsub = threadIdx.x / LPR;
    const int c0 = lane * 4;

    const float4 kv = load4(k + (size_t)unit * DK + c0);
    const float4 qv = load4(q + (size_t)unit * DK + c0);
    float4 a;
    if constexpr (KDA) {
        const float4 la = *reinterpret_cast<const float4 *>(log_alpha + (size_t)unit * DK + c0);
        a = make_float4(__expf(la.x), __expf(la.y), __expf(la.z), __expf(la.w));
    } else {
        const float s = __expf(log_alpha[unit]);
        a = make_float4(s, s, s, s);
    }
    const float b = beta[unit];
    const float kq = group_sum<LPR>(kv.x * qv.x + kv.y * qv.y + kv.z * qv.z + kv.w * qv.w);

    float *S = state + (size_t)unit * DV * DK;
    const QT *vu = v + (size_t)unit * DV;
    using OT = typename std::conditional<OUTB, __bf16, float>::type;
    OT *ou = static_cast<OT *>(out) + (size_t)unit * DV;

    for (int base = 0; base < DV; base += RPP * RB) {
        f32x4 s[RB];
        float vi[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int i = base + r * RPP + rsub;
            if (EXACT || i < DV) {
                s[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (size_t)i * DK + c0));
                vi[r] = to_f32(vu[i]);
            }
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int i = base + r * RPP + rsub;
            // the group-sum below needs every lane of the row group; i < DV is
            // uniform over the group (all its lanes share rsub), so skipping is safe
            if (EXACT || i < DV) {
                f32x4 t = s[r];
                t[0] *= a.x; t[1] *= a.y; t[2] *= a.z; t[3] *= a.w;
                float x = t[0] * kv.x + t[1] * kv.y + t[2] * kv.z + t[3] * kv.w;
                float y = t[0] * qv.x + t[1] * qv.y + t[2] * qv.z + t[3] * qv.w;
                x = group_sum<LPR>(x);
                y = group_sum<LPR>(y);
                const float u = b * (vi[r] - x);
                t[0] += u * kv.x; t[1] += u * kv.y; t[2] += u * kv.z; t[3] += u * kv.w;
                __builtin_nontemporal_store(t, reinterpret_cast<f32x4 *>(S + (size_t)i * DK + c0));
                if (lane == 0) ou[i] = (OT)(scale * (y + u * kq));
            }
        }
    }
}

template <int DK, bool KDA, typename QT>
static hipError_t launch_decode_t(const DecodeArgs &p, hipStream_t st) {
    constexpr int LPR = DK / 4;
    constexpr int RPP = 256 / LPR;
    constexpr int RB = (RPP >= 64) ? 2 : (RPP >= 32 ? 4 : 8);
    const unsigned grid = (unsigned)((size_t)p.num_seqs * p.num_heads);
    const bool exact = p.dv % (RPP * RB) == 0;
#define GDR_DECODE_LAUNCH(E, O)                                                                        \
    hipLaunchKernelGGL((decode_kernel<DK, KDA, QT, RB, E, O>), dim3(grid), dim3(256), 0, st, p.num_heads, \
                       p.dv, (const QT *)p.q, (const QT *)p.k, (const QT *)p.v, p.beta, p.log_alpha,     \
                       p.state, p.scale, p.out)
    if (exact) {
        if (p.out_bf16) GDR_DECODE_LAUNCH(true, true);
        else GDR_DECODE_LAUNCH(true, false);
    } else {
        if (p.out_bf16) GDR_DECODE_LAUNCH(false, true);
        else GDR_DECODE_LAUNCH(false, false);
    }
#undef GDR_DECODE_LAUNCH
    return hipGetLastError();
}

template <bool KDA, typename QT>
static hipError_t launch_decode_dk(const DecodeArgs &p, hipStream_t st) {
    switch (p.dk) {
        case 16: return launch_decode_t<16, KDA, QT>(p, st);
        case 32: return launch_decode_t<32, KDA, QT>(p, st);
        case 64: return launch_decode_t<64, KDA, QT>(p, st);
        case 128: return launch_decode_t<128, KDA, QT>(p, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeArgs &p, hipStream_t st) {
    if (p.num_seqs == 0 || p.num_heads == 0) return hipSuccess;
    if (p.kda) return p.bf16 ? launch_decode_dk<true, __bf16>(p, st) : launch_decode_dk<true, float>(p, st);
    return p.bf16 ? launch_decode_dk<false, __bf16>(p, st) : launch_decode_dk<false, float>(p, st);
}

}  // namespace gdr
