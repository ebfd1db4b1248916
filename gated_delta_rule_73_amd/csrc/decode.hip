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
// Layout of the work: one workgroup per (sequence, head), 512 threads for
// d_k >= 64.  A state row is spread over LPR = min(8, d_k / 4) lanes, lane l
// holding the VPL four-column groups 4 l + 4 LPR j (j < VPL): a row group's
// loads cover whole 128-byte lines, and each row's two dot products finish in
// log2(LPR) DPP steps inside the lane group.  Every row of the state a thread
// owns is requested before any is used, so the whole state is in flight at
// once.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace gdr {

// Lane layout shared by both decode kernels (see the top of the file).
template <int DK> constexpr int decode_threads() { return DK >= 64 ? 512 : 256; }
template <int DK> constexpr int decode_lpr() { return DK / 4 < 8 ? DK / 4 : 8; }
constexpr int kDecodeTokenBatch = 8;

// Sum over aligned groups of W in {4, 8} lanes by DPP: swap neighbours, swap
// pairs, then (W = 8) mirror each half-row of 8 lanes.
template <int W>
__device__ __forceinline__ float dpp_group_sum(float x) {
    static_assert(W == 4 || W == 8, "DPP lane groups of 4 or 8");
#define GDR_DPP(y, ctrl) __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, y), ctrl, 0xF, 0xF, false))
    x += GDR_DPP(x, 0xB1);                          // quad_perm [1, 0, 3, 2]
    x += GDR_DPP(x, 0x4E);                          // quad_perm [2, 3, 0, 1]
    if constexpr (W == 8) x += GDR_DPP(x, 0x141);   // row_half_mirror
#undef GDR_DPP
    return x;
}

// One token per (sequence, head), layout as described at the top of the file.
// NR: rows per thread (the largest d_v the instance holds is NR x rows per
// pass); OUTB: bf16 outputs.  Value head h reads the q/k head h / G of HK
// (grouped value heads).  GT: storage type of beta and log alpha.
template <int DK, bool KDA, typename QT, typename GT, int NR, bool OUTB>
__global__ __launch_bounds__(decode_threads<DK>()) void decode_kernel(
    int H, int HK, int G, int DV, const QT *__restrict__ q, const QT *__restrict__ k, const QT *__restrict__ v,
    const GT *__restrict__ beta, const GT *__restrict__ log_alpha, float *__restrict__ state,
    float scale, void *__restrict__ out) {
    constexpr int NTH = decode_threads<DK>();
    constexpr int LPR = decode_lpr<DK>();   // lanes per state row
    constexpr int VPL = DK / (4 * LPR);            // four-column groups per lane and row
    constexpr int RPP = NTH / LPR;                 // rows covered by the workgroup per pass
    const int unit = blockIdx.x;                   // n * H + h
    const int qku = (unit / H) * HK + (unit % H) / G;
    const int lane = threadIdx.x % LPR;
    const int rsub = threadIdx.x / LPR;

    float4 kv[VPL], qv[VPL], a[VPL];
    float kq = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int c = 4 * (lane + LPR * j);
        kv[j] = load4(k + (size_t)qku * DK + c);
        qv[j] = load4(q + (size_t)qku * DK + c);
        if constexpr (KDA) {
            const float4 la = load4(log_alpha + (size_t)unit * DK + c);
            a[j] = make_float4(__expf(la.x), __expf(la.y), __expf(la.z), __expf(la.w));
        }
        kq += kv[j].x * qv[j].x + kv[j].y * qv[j].y + kv[j].z * qv[j].z + kv[j].w * qv[j].w;
    }
    if constexpr (!KDA) {
        const float e = __expf(to_f32(log_alpha[unit]));
#pragma unroll
        for (int j = 0; j < VPL; ++j) a[j] = make_float4(e, e, e, e);
    }
    const float b = to_f32(beta[unit]);

    float *S = state + (size_t)unit * DV * DK;
    const QT *vu = v + (size_t)unit * DV;
    using OT = typename std::conditional<OUTB, __bf16, float>::type;
    OT *ou = static_cast<OT *>(out) + (size_t)unit * DV;
    f32x4 s[NR][VPL];
    float vi[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int i = r * RPP + rsub;
        if (i < DV) {
#pragma unroll
            for (int j = 0; j < VPL; ++j)
                s[r][j] = __builtin_nontemporal_load(
                    reinterpret_cast<const f32x4 *>(S + (size_t)i * DK + 4 * (lane + LPR * j)));
            vi[r] = to_f32(vu[i]);
        }
    }
    kq = dpp_group_sum<LPR>(kq);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int i = r * RPP + rsub;
        // i < DV is uniform over a row's lane group (they share rsub), so the
        // DPP sums below see every lane of the group
        if (i < DV) {
            float x = 0.f, y = 0.f;
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                f32x4 &w = s[r][j];
                w[0] *= a[j].x; w[1] *= a[j].y; w[2] *= a[j].z; w[3] *= a[j].w;
                x += w[0] * kv[j].x + w[1] * kv[j].y + w[2] * kv[j].z + w[3] * kv[j].w;
                y += w[0] * qv[j].x + w[1] * qv[j].y + w[2] * qv[j].z + w[3] * qv[j].w;
            }
            x = dpp_group_sum<LPR>(x);
            y = dpp_group_sum<LPR>(y);
            const float u = b * (vi[r] - x);
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                f32x4 &w = s[r][j];
                w[0] += u * kv[j].x; w[1] += u * kv[j].y; w[2] += u * kv[j].z; w[3] += u * kv[j].w;
                __builtin_nontemporal_store(w, reinterpret_cast<f32x4 *>(S + (size_t)i * DK + 4 * (lane + LPR * j)));
            }
            if (lane == 0) ou[i] = (OT)(scale * (y + u * kq));
        }
    }
}

template <int DK, bool KDA, typename QT, typename GT>
static hipError_t launch_decode_t(const DecodeArgs &p, hipStream_t st) {
    constexpr int NTH = decode_threads<DK>();
    constexpr int RPP = NTH / decode_lpr<DK>();
    const unsigned grid = (unsigned)((size_t)p.num_seqs * p.num_heads);
#define GDR_DECODE_LAUNCH(NR, O)                                                                               \
    hipLaunchKernelGGL((decode_kernel<DK, KDA, QT, GT, NR, O>), dim3(grid), dim3(NTH), 0, st, p.num_heads,      \
                       p.num_qk_heads, p.num_heads / p.num_qk_heads, p.dv, (const QT *)p.q, (const QT *)p.k,    \
                       (const QT *)p.v, (const GT *)p.beta, (const GT *)p.log_alpha, p.state, p.scale, p.out)
    // rows per thread: enough for d_v <= 128, or for d_v <= 256
    if (p.dv <= 128) {
        if (p.out_bf16) GDR_DECODE_LAUNCH(div_up(128, RPP), true);
        else GDR_DECODE_LAUNCH(div_up(128, RPP), false);
    } else {
        if (p.out_bf16) GDR_DECODE_LAUNCH(div_up(256, RPP), true);
        else GDR_DECODE_LAUNCH(div_up(256, RPP), false);
    }
#undef GDR_DECODE_LAUNCH
    return hipGetLastError();
}

template <bool KDA, typename QT, typename GT>
static hipError_t launch_decode_dk(const DecodeArgs &p, hipStream_t st) {
    switch (p.dk) {
        case 16: return launch_decode_t<16, KDA, QT, GT>(p, st);
        case 32: return launch_decode_t<32, KDA, QT, GT>(p, st);
        case 64: return launch_decode_t<64, KDA, QT, GT>(p, st);
        case 128: return launch_decode_t<128, KDA, QT, GT>(p, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool KDA, typename QT>
static hipError_t launch_decode_gt(const DecodeArgs &p, hipStream_t st) {
    return p.gate_bf16 ? launch_decode_dk<KDA, QT, __bf16>(p, st) : launch_decode_dk<KDA, QT, float>(p, st);
}

hipError_t launch_decode(const DecodeArgs &p, hipStream_t st) {
    if (p.num_seqs == 0 || p.num_heads == 0) return hipSuccess;
    if (p.kda) return p.bf16 ? launch_decode_gt<true, __bf16>(p, st) : launch_decode_gt<true, float>(p, st);
    return p.bf16 ? launch_decode_gt<false, __bf16>(p, st) : launch_decode_gt<false, float>(p, st);
}

// ---------------------------------------------------------------------------
// Multi-token decode over a pool of state slots.  One workgroup of NTH threads
// per (sequence, value head); the whole d_v x d_k state stays in registers
// while the tokens of the sequence are applied one after another, each as in
// decode_kernel.  A state row is spread over LPR = min(8, d_k / 4) lanes,
// lane l holding the VPL four-column groups 4 l + 4 LPR j (j < VPL), so one
// load instruction reads whole 128-byte lines, and the row's dot products
// finish with log2(LPR) DPP steps inside the lane group (no LDS permutes).
// The inputs of up to TB tokens at a time are staged in LDS as fp32 (with the
// decay already exponentiated), so the token loop waits on no global load;
// the first batch is requested together with the state.  The state is
// written back once, right after token C_n - 1 (the committed prefix), so a
// verify-only call (C_n = 0) never writes it.
struct DecodeTokensKArgs {
    int H, HK, G, DV, K, num_slots;
    const void *q, *k, *v;
    const void *beta, *log_alpha;    // the kernel's GT
    const int32_t *num_tokens, *num_commit, *slots;
    float *pool;
    float scale;
    void *out;
};

template <int DK, bool KDA, typename QT, typename GT, int NR, bool OUTB>
__global__ __launch_bounds__(decode_threads<DK>()) void decode_tokens_kernel(DecodeTokensKArgs p) {
    constexpr int NTH = decode_threads<DK>();
    constexpr int LPR = decode_lpr<DK>();   // lanes per state row
    constexpr int VPL = DK / (4 * LPR);            // four-column groups per lane and row
    constexpr int RPP = NTH / LPR;                 // rows covered by the workgroup per pass
    constexpr int DVM = NR * RPP;                  // largest d_v this instance holds
    constexpr int TB = kDecodeTokenBatch;
    constexpr int NA = KDA ? DK : 1;
    const int unit = blockIdx.x;                   // n * H + h
    const int H = p.H, DV = p.DV, K = p.K;
    const int n = unit / H, h = unit % H;
    const int slot = p.slots ? p.slots[n] : n;
    if (slot < 0 || slot >= p.num_slots) return;           // padding entry: nothing read or written
    const int T = p.num_tokens ? min(max(p.num_tokens[n], 0), K) : K;
    const int Cm = p.num_commit ? min(max(p.num_commit[n], 0), T) : T;
    if (T == 0) return;
    const int tid = threadIdx.x;
    const int lane = tid % LPR;
    const int rsub = tid / LPR;
    const QT *q = static_cast<const QT *>(p.q);
    const QT *k = static_cast<const QT *>(p.k);
    const QT *v = static_cast<const QT *>(p.v);
    const GT *gla = static_cast<const GT *>(p.log_alpha);
    const GT *gbeta = static_cast<const GT *>(p.beta);
    using OT = typename std::conditional<OUTB, __bf16, float>::type;
    OT *out = static_cast<OT *>(p.out);
    float *S = p.pool + ((size_t)slot * H + h) * DV * DK;

    // one batch of token inputs: k, q, alpha = exp(log alpha), beta, v
    __shared__ float4 sk[TB][DK / 4], sq[TB][DK / 4];
    __shared__ float sa[TB][NA], sb[TB], sv[TB][DVM];

    f32x4 s[NR][VPL];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int i = r * RPP + rsub;
        if (i < DV) {
#pragma unroll
            for (int j = 0; j < VPL; ++j)
                s[r][j] = __builtin_nontemporal_load(
                    reinterpret_cast<const f32x4 *>(S + (size_t)i * DK + 4 * (lane + LPR * j)));
        }
    }

    for (int t0 = 0; t0 < T; t0 += TB) {
        const int nb = min(TB, T - t0);
        if (t0 > 0) __syncthreads();              // the previous batch has been read
        for (int e = tid; e < nb * (DK / 4); e += NTH) {
            const int tt = e / (DK / 4), c = (e % (DK / 4)) * 4;
            const size_t tr = (size_t)n * K + t0 + tt;
            const size_t qo = (tr * p.HK + h / p.G) * DK + c;
            sk[tt][c / 4] = load4(k + qo);
            sq[tt][c / 4] = load4(q + qo);
            if constexpr (KDA) {
                const float4 la = load4(gla + (tr * H + h) * DK + c);
                sa[tt][c] = __expf(la.x); sa[tt][c + 1] = __expf(la.y);
                sa[tt][c + 2] = __expf(la.z); sa[tt][c + 3] = __expf(la.w);
            }
        }
        for (int e = tid; e < nb * DV; e += NTH) {
            const int tt = e / DV, i = e % DV;
            sv[tt][i] = to_f32(v[(((size_t)n * K + t0 + tt) * H + h) * DV + i]);
        }
        if (tid < nb) {
            const size_t tr = (size_t)n * K + t0 + tid;
            sb[tid] = to_f32(gbeta[tr * H + h]);
            if constexpr (!KDA) sa[tid][0] = __expf(to_f32(gla[tr * H + h]));
        }
        __syncthreads();
        for (int tt = 0; tt < nb; ++tt) {
            const int t = t0 + tt;
            float4 kv[VPL], qv[VPL], a[VPL];
            float kq = 0.f;
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                const int g = lane + LPR * j;
                kv[j] = sk[tt][g];
                qv[j] = sq[tt][g];
                if constexpr (KDA) a[j] = make_float4(sa[tt][4 * g], sa[tt][4 * g + 1], sa[tt][4 * g + 2], sa[tt][4 * g + 3]);
                else a[j] = make_float4(sa[tt][0], sa[tt][0], sa[tt][0], sa[tt][0]);
                kq += kv[j].x * qv[j].x + kv[j].y * qv[j].y + kv[j].z * qv[j].z + kv[j].w * qv[j].w;
            }
            kq = dpp_group_sum<LPR>(kq);
            const float b = sb[tt];
            OT *ot = out + (((size_t)n * K + t) * H + h) * DV;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int i = r * RPP + rsub;
                // i < DV is uniform over a row's lane group (they share rsub)
                if (i < DV) {
                    float x = 0.f, y = 0.f;
#pragma unroll
                    for (int j = 0; j < VPL; ++j) {
                        f32x4 &w = s[r][j];
                        w[0] *= a[j].x; w[1] *= a[j].y; w[2] *= a[j].z; w[3] *= a[j].w;
                        x += w[0] * kv[j].x + w[1] * kv[j].y + w[2] * kv[j].z + w[3] * kv[j].w;
                        y += w[0] * qv[j].x + w[1] * qv[j].y + w[2] * qv[j].z + w[3] * qv[j].w;
                    }
                    x = dpp_group_sum<LPR>(x);
                    y = dpp_group_sum<LPR>(y);
                    const float u = b * (sv[tt][i] - x);
#pragma unroll
                    for (int j = 0; j < VPL; ++j) {
                        f32x4 &w = s[r][j];
                        w[0] += u * kv[j].x; w[1] += u * kv[j].y; w[2] += u * kv[j].z; w[3] += u * kv[j].w;
                    }
                    if (lane == 0) ot[i] = (OT)(p.scale * (y + u * kq));
                }
            }
            if (t + 1 == Cm) {
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const int i = r * RPP + rsub;
                    if (i < DV) {
#pragma unroll
                        for (int j = 0; j < VPL; ++j)
                            __builtin_nontemporal_store(
                                s[r][j], reinterpret_cast<f32x4 *>(S + (size_t)i * DK + 4 * (lane + LPR * j)));
                    }
                }
            }
        }
    }
}

template <int DK, bool KDA, typename QT, typename GT>
static hipError_t launch_decode_tokens_t(const DecodeArgs &a, hipStream_t st) {
    constexpr int NTH = decode_threads<DK>();
    constexpr int RPP = NTH / decode_lpr<DK>();
    DecodeTokensKArgs p;
    p.H = a.num_heads;
    p.HK = a.num_qk_heads;
    p.G = a.num_heads / a.num_qk_heads;
    p.DV = a.dv;
    p.K = a.max_tokens;
    p.num_slots = a.num_slots;
    p.q = a.q; p.k = a.k; p.v = a.v;
    p.beta = a.beta;
    p.log_alpha = a.log_alpha;
    p.num_tokens = a.num_tokens;
    p.num_commit = a.num_commit;
    p.slots = a.slots;
    p.pool = a.state;
    p.scale = a.scale;
    p.out = a.out;
    const unsigned grid = (unsigned)((size_t)a.num_seqs * a.num_heads);
    // rows per thread: enough for d_v <= 128, or for d_v <= 256
    if (a.dv <= 128) {
        if (a.out_bf16) hipLaunchKernelGGL((decode_tokens_kernel<DK, KDA, QT, GT, div_up(128, RPP), true>), dim3(grid), dim3(NTH), 0, st, p);
        else hipLaunchKernelGGL((decode_tokens_kernel<DK, KDA, QT, GT, div_up(128, RPP), false>), dim3(grid), dim3(NTH), 0, st, p);
    } else {
        if (a.out_bf16) hipLaunchKernelGGL((decode_tokens_kernel<DK, KDA, QT, GT, div_up(256, RPP), true>), dim3(grid), dim3(NTH), 0, st, p);
        else hipLaunchKernelGGL((decode_tokens_kernel<DK, KDA, QT, GT, div_up(256, RPP), false>), dim3(grid), dim3(NTH), 0, st, p);
    }
    return hipGetLastError();
}

template <bool KDA, typename QT, typename GT>
static hipError_t launch_decode_tokens_dk(const DecodeArgs &p, hipStream_t st) {
    switch (p.dk) {
        case 16: return launch_decode_tokens_t<16, KDA, QT, GT>(p, st);
        case 32: return launch_decode_tokens_t<32, KDA, QT, GT>(p, st);
        case 64: return launch_decode_tokens_t<64, KDA, QT, GT>(p, st);
        case 128: return launch_decode_tokens_t<128, KDA, QT, GT>(p, st);
        default: return hipErrorInvalidValue;
    }
}

template <bool KDA, typename QT>
static hipError_t launch_decode_tokens_gt(const DecodeArgs &p, hipStream_t st) {
    return p.gate_bf16 ? launch_decode_tokens_dk<KDA, QT, __bf16>(p, st) : launch_decode_tokens_dk<KDA, QT, float>(p, st);
}

hipError_t launch_decode_tokens(const DecodeArgs &p, hipStream_t st) {
    if (p.num_seqs == 0 || p.num_heads == 0) return hipSuccess;
    if (p.kda) return p.bf16 ? launch_decode_tokens_gt<true, __bf16>(p, st) : launch_decode_tokens_gt<true, float>(p, st);
    return p.bf16 ? launch_decode_tokens_gt<false, __bf16>(p, st) : launch_decode_tokens_gt<false, float>(p, st);
}

}  // namespace gdr
