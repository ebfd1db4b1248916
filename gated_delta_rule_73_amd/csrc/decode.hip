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
// Decode step with the layer prologue fused in: for each (sequence, value
// head) the workgroup forms its own q, k (of its q/k head) and v from the
// token's projected channels x and the convolution state -- the width-4 causal
// convolution, the optional SiLU and per-head q/k L2 norm, in the layer
// prologue's order of operations -- and the gates beta = sigmoid(b),
// log alpha = -softplus(a), then runs the decode update above.  q, k, v and
// the gates never leave the chip and stay fp32 (the unfused calls store them
// in x's dtype in between).  Value heads that share a
// q/k head each recompute it (a few hundred flops).  The convolution state is
// only read here; decode_conv_shift_kernel advances it afterwards on the same
// stream, which keeps an in-place update safe.
struct DecodePrologueKArgs {
    int H, HK, G, DV, C;
    const void *x, *cs_in;
    const float *w, *a_logit, *b_logit;
    float *state;
    float scale;
    void *out;
};

// one channel's convolution inputs for the token: its taps and x_{t-3},
// x_{t-2}, x_{t-1} (convolution state rows 0, 1, 2), x_t
struct ConvIn {
    float4 w;
    float h3, h2, h1, x0;
};
template <typename XT>
__device__ __forceinline__ ConvIn conv_in(const DecodePrologueKArgs &p, int n, int ch) {
    const XT *x = static_cast<const XT *>(p.x);
    const XT *cs = static_cast<const XT *>(p.cs_in);
    ConvIn c;
    c.w = *reinterpret_cast<const float4 *>(p.w + (size_t)ch * 4);
    c.h3 = c.h2 = c.h1 = 0.f;
    if (cs) {
        c.h3 = to_f32(cs[((size_t)n * 3 + 0) * p.C + ch]);
        c.h2 = to_f32(cs[((size_t)n * 3 + 1) * p.C + ch]);
        c.h1 = to_f32(cs[((size_t)n * 3 + 2) * p.C + ch]);
    }
    c.x0 = to_f32(x[(size_t)n * p.C + ch]);
    return c;
}
// the convolution output in the layer prologue's order, then the optional SiLU
template <bool SILU>
__device__ __forceinline__ float conv_out(const ConvIn &c) {
    float y = c.w.x * c.h3 + c.w.y * c.h2 + c.w.z * c.h1 + c.w.w * c.x0;
    if constexpr (SILU) y = y / (1.f + __expf(-y));
    return y;
}

template <int DK, bool KDA, typename XT, int NR, bool SILU, bool NORM, bool OUTB>
__global__ __launch_bounds__(decode_threads<DK>()) void decode_prologue_kernel(DecodePrologueKArgs p) {
    constexpr int NTH = decode_threads<DK>();
    constexpr int LPR = decode_lpr<DK>();
    constexpr int VPL = DK / (4 * LPR);
    constexpr int RPP = NTH / LPR;
    constexpr int DVM = NR * RPP;                  // largest d_v this instance holds
    const int unit = blockIdx.x;                   // n * H + h
    const int n = unit / p.H, h = unit % p.H, hq = h / p.G;
    const int tid = threadIdx.x;
    const int lane = tid % LPR;
    const int rsub = tid / LPR;
    const int DV = p.DV;
    const int qk = p.HK * DK;                      // channels of q (and of k)

    // the prologue, one channel per thread: q, k of head hq, v of head h and,
    // per channel, alpha = exp(-softplus(a)).  The inputs of a thread's first
    // channel are requested before the state (loads complete in order, so the
    // prologue does not wait for the state), the state right after them.
    __shared__ float sq[DK], sk[DK], sv[DVM], sa[KDA ? DK : 1], sn[2];
    auto alpha_of = [](float al) { return __expf(-(fmaxf(al, 0.f) + log1pf(__expf(-fabsf(al))))); };
    auto channel = [&](int c) { return c < DK ? hq * DK + c : c < 2 * DK ? qk + hq * DK + c - DK : 2 * qk + h * DV + c - 2 * DK; };
    auto put = [&](int c, float y) {
        if (c < DK) sq[c] = y;
        else if (c < 2 * DK) sk[c - DK] = y;
        else sv[c - 2 * DK] = y;
    };
    const int total = 2 * DK + DV;
    ConvIn first{};
    if (tid < total) first = conv_in<XT>(p, n, channel(tid));
    const float al0 = (KDA && tid < DK) ? p.a_logit[(size_t)unit * DK + tid] : 0.f;

    float *S = p.state + (size_t)unit * DV * DK;
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

    if (tid < total) put(tid, conv_out<SILU>(first));
    for (int c = tid + NTH; c < total; c += NTH) put(c, conv_out<SILU>(conv_in<XT>(p, n, channel(c))));
    if constexpr (KDA) {
        if (tid < DK) sa[tid] = alpha_of(al0);
        for (int c = tid + NTH; c < DK; c += NTH) sa[c] = alpha_of(p.a_logit[(size_t)unit * DK + c]);
    }
    __syncthreads();
    if constexpr (NORM) {
        // per-head L2 norms of q and k: wave 0 sums q, wave 1 sums k
        if (tid < 128) {
            const float *src = tid < 64 ? sq : sk;
            float ss = 0.f;
            for (int c = tid % 64; c < DK; c += 64) ss += src[c] * src[c];
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
            if (tid % 64 == 0) sn[tid / 64] = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
        }
        __syncthreads();
    }
    const float scq = NORM ? sn[0] : 1.f, sck = NORM ? sn[1] : 1.f;

    float4 kv[VPL], qv[VPL], a[VPL];
    float kq = 0.f;
    const float eh = KDA ? 0.f : alpha_of(p.a_logit[unit]);
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
        const int c = 4 * (lane + LPR * j);
        qv[j] = make_float4(sq[c] * scq, sq[c + 1] * scq, sq[c + 2] * scq, sq[c + 3] * scq);
        kv[j] = make_float4(sk[c] * sck, sk[c + 1] * sck, sk[c + 2] * sck, sk[c + 3] * sck);
        if constexpr (KDA) a[j] = make_float4(sa[c], sa[c + 1], sa[c + 2], sa[c + 3]);
        else a[j] = make_float4(eh, eh, eh, eh);
        kq += kv[j].x * qv[j].x + kv[j].y * qv[j].y + kv[j].z * qv[j].z + kv[j].w * qv[j].w;
    }
    kq = dpp_group_sum<LPR>(kq);
    const float b = 1.f / (1.f + __expf(-p.b_logit[unit]));   // sigmoid(b)

    using OT = typename std::conditional<OUTB, __bf16, float>::type;
    OT *ou = static_cast<OT *>(p.out) + (size_t)unit * DV;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int i = r * RPP + rsub;
        // i < DV is uniform over a row's lane group (they share rsub)
        if (i < DV) {
            float xx = 0.f, yy = 0.f;
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                f32x4 &w = s[r][j];
                w[0] *= a[j].x; w[1] *= a[j].y; w[2] *= a[j].z; w[3] *= a[j].w;
                xx += w[0] * kv[j].x + w[1] * kv[j].y + w[2] * kv[j].z + w[3] * kv[j].w;
                yy += w[0] * qv[j].x + w[1] * qv[j].y + w[2] * qv[j].z + w[3] * qv[j].w;
            }
            xx = dpp_group_sum<LPR>(xx);
            yy = dpp_group_sum<LPR>(yy);
            const float u = b * (sv[i] - xx);
#pragma unroll
            for (int j = 0; j < VPL; ++j) {
                f32x4 &w = s[r][j];
                w[0] += u * kv[j].x; w[1] += u * kv[j].y; w[2] += u * kv[j].z; w[3] += u * kv[j].w;
                __builtin_nontemporal_store(w, reinterpret_cast<f32x4 *>(S + (size_t)i * DK + 4 * (lane + LPR * j)));
            }
            if (lane == 0) ou[i] = (OT)(p.scale * (yy + u * kq));
        }
    }
}

// The new convolution state of each sequence: rows (x_{t-2}, x_{t-1}, x_t),
// i.e. the old rows 1 and 2 and the token's input.  Eight channels per thread,
// both old rows read before any row is written (in place safe).
template <typename XT>
__global__ __launch_bounds__(256) void decode_conv_shift_kernel(int N, int C, const XT *__restrict__ x,
                                                                const XT *cs_in, XT *cs_out) {
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const int CV = C / 8;
    if (i >= (long)N * CV) return;
    const int n = (int)(i / CV), c = (int)(i % CV) * 8;
    XT r[3][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) r[0][e] = r[1][e] = (XT)0.f;
    if (cs_in) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            r[0][e] = cs_in[((size_t)n * 3 + 1) * C + c + e];
            r[1][e] = cs_in[((size_t)n * 3 + 2) * C + c + e];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) r[2][e] = x[(size_t)n * C + c + e];
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) cs_out[((size_t)n * 3 + j) * C + c + e] = r[j][e];
}

template <int DK, bool KDA, typename XT>
static hipError_t launch_decode_prologue_t(const DecodePrologueArgs &a, hipStream_t st) {
    constexpr int NTH = decode_threads<DK>();
    constexpr int RPP = NTH / decode_lpr<DK>();
    DecodePrologueKArgs p;
    p.H = a.num_heads;
    p.HK = a.num_qk_heads;
    p.G = a.num_heads / a.num_qk_heads;
    p.DV = a.dv;
    p.C = 2 * a.num_qk_heads * DK + a.num_heads * a.dv;
    p.x = a.x;
    p.cs_in = a.conv_state_in;
    p.w = a.conv_weight;
    p.a_logit = a.a_logit;
    p.b_logit = a.b_logit;
    p.state = a.state;
    p.scale = a.scale;
    p.out = a.out;
    const unsigned grid = (unsigned)((size_t)a.num_seqs * a.num_heads);
#define GDR_DP(NR, S, N, O) \
    hipLaunchKernelGGL((decode_prologue_kernel<DK, KDA, XT, NR, S, N, O>), dim3(grid), dim3(NTH), 0, st, p)
#define GDR_DP_NR(NR)                                                              \
    do {                                                                           \
        if (a.silu) {                                                              \
            if (a.qk_norm) { if (a.out_bf16) GDR_DP(NR, true, true, true); else GDR_DP(NR, true, true, false); }     \
            else { if (a.out_bf16) GDR_DP(NR, true, false, true); else GDR_DP(NR, true, false, false); }           \
        } else {                                                                   \
            if (a.qk_norm) { if (a.out_bf16) GDR_DP(NR, false, true, true); else GDR_DP(NR, false, true, false); }   \
            else { if (a.out_bf16) GDR_DP(NR, false, false, true); else GDR_DP(NR, false, false, false); }         \
        }                                                                          \
    } while (0)
    if (a.dv <= 128) GDR_DP_NR(div_up(128, RPP));
    else GDR_DP_NR(div_up(256, RPP));
#undef GDR_DP_NR
#undef GDR_DP
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.conv_state_out) return e;
    const long work = (long)a.num_seqs * (p.C / 8);
    hipLaunchKernelGGL((decode_conv_shift_kernel<XT>), dim3((unsigned)((work + 255) / 256)), dim3(256), 0, st,
                       a.num_seqs, p.C, static_cast<const XT *>(a.x), static_cast<const XT *>(a.conv_state_in),
                       static_cast<XT *>(a.conv_state_out));
    return hipGetLastError();
}

template <bool KDA, typename XT>
static hipError_t launch_decode_prologue_dk(const DecodePrologueArgs &a, hipStream_t st) {
    switch (a.dk) {
        case 16: return launch_decode_prologue_t<16, KDA, XT>(a, st);
        case 32: return launch_decode_prologue_t<32, KDA, XT>(a, st);
        case 64: return launch_decode_prologue_t<64, KDA, XT>(a, st);
        case 128: return launch_decode_prologue_t<128, KDA, XT>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_prologue(const DecodePrologueArgs &a, hipStream_t st) {
    if (a.num_seqs == 0 || a.num_heads == 0) return hipSuccess;
    if (a.kda) return a.x_bf16 ? launch_decode_prologue_dk<true, __bf16>(a, st) : launch_decode_prologue_dk<true, float>(a, st);
    return a.x_bf16 ? launch_decode_prologue_dk<false, __bf16>(a, st) : launch_decode_prologue_dk<false, float>(a, st);
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
