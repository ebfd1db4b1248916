// prologue.hip -- the steps of a linear-attention layer between its input
// projections and the recurrence, fused into one pass over the projected
// q/k/v channels (page "Qwen3.8-Flash-Next and GLM-5.3-Flash share a 3:1
// long-context pattern", section "Kimi Delta Attention extends recurrent
// memory control": a short convolution of kernel four on the linear-attention
// path; page "How the New Flash Models Work: Inside GLM-5.3-Flash and
// Qwen3.8-Flash-Next", section "Serving: prefill and decode are different
// problems": a convolution state is handed from prefill to decode with the
// recurrent state).
//
// Per token t of a sequence and channel c of the concatenated q, k, v
// projections x (C = 2 Hk dk + H dv channels):
//     y_t[c] = sum_{j<4} w[c][j] x_{t-3+j}[c]      (causal, per channel; the
//              inputs before the sequence's first token come from its
//              convolution state, the three inputs that preceded it)
//     y <- silu(y)                                  (option)
//     q, k <- y / |y| per head                      (option: L2 norm over d_k)
// and, elementwise, beta = sigmoid(b), log alpha = -softplus(a).
//
// Kernel 1 (conv): a workgroup takes 2048 channels (8 per thread, 16-byte
// vectors) of a block of consecutive tokens and walks them in order with the
// three previous inputs held in registers, so each input row is read once
// (plus a three-row halo per block).  The per-head norm sums over dk / 8
// lanes by DPP.  Kernel 2 (gates and state): the gate activations, then each
// sequence's new convolution state (its last three inputs, older state rows
// when it has fewer than three tokens); it runs after kernel 1 on the same
// stream, so the state may be updated in place.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace gdr {

constexpr int kPrologueThreads = 256;
constexpr int kPrologueTokens = 64;   // tokens per conv workgroup

// eight consecutive channels: one 16-byte access (bf16) or two (fp32)
__device__ __forceinline__ void load8(const __bf16 *p, float (&v)[8]) {
    const bf16x8 x = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)x[i];
}
__device__ __forceinline__ void load8(const float *p, float (&v)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p), b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = a[i];
        v[4 + i] = b[i];
    }
}
__device__ __forceinline__ void store8(__bf16 *p, const float (&v)[8]) {
    bf16x8 x;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (__bf16)v[i];
    *reinterpret_cast<bf16x8 *>(p) = x;
}
__device__ __forceinline__ void store8(float *p, const float (&v)[8]) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// Sum over aligned groups of W in {1, 2, 4, 8, 16} lanes by DPP (within a row
// of 16 lanes): swap neighbours, swap pairs, mirror half-rows, mirror rows.
template <int W>
__device__ __forceinline__ float dpp_sum(float x) {
#define GDR_DPP(y, ctrl) __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, y), ctrl, 0xF, 0xF, false))
    if constexpr (W >= 2) x += GDR_DPP(x, 0xB1);    // quad_perm [1, 0, 3, 2]
    if constexpr (W >= 4) x += GDR_DPP(x, 0x4E);    // quad_perm [2, 3, 0, 1]
    if constexpr (W >= 8) x += GDR_DPP(x, 0x141);   // row_half_mirror
    if constexpr (W >= 16) x += GDR_DPP(x, 0x140);  // row_mirror
#undef GDR_DPP
    return x;
}

struct PrologueKArgs {
    int T, C, QK;                 // tokens per row (dense) or in total (packed); channels; q+k channels
    int num_seqs, total_tokens;
    const void *x;
    const float *w;               // [C][4]
    const void *state_in;         // [num_seqs][3][C] or NULL
    const int32_t *cu;            // packed: [num_seqs + 1]
    void *q, *k, *v;
    int qk_half;                  // Hk dk: channels of q (and of k)
    int dv_total;                 // H dv
};

template <typename XT, int DK, bool SILU, bool NORM>
__global__ __launch_bounds__(kPrologueThreads) void prologue_conv_kernel(PrologueKArgs p) {
    // grid: x = token blocks, y = blocks of 2048 channels
    const int c0 = (blockIdx.y * kPrologueThreads + threadIdx.x) * 8;   // first of this thread's 8 channels
    const bool active = c0 < p.C;     // q/k heads (C multiple of d_k there) are all in or all out
    const int tb = blockIdx.x * kPrologueTokens;
    const int te = min(tb + kPrologueTokens, p.total_tokens);
    const XT *x = static_cast<const XT *>(p.x);
    const XT *st = static_cast<const XT *>(p.state_in);

    float w[8][4];
    if (active) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 wi = *reinterpret_cast<const float4 *>(p.w + (size_t)(c0 + i) * 4);
            w[i][0] = wi.x; w[i][1] = wi.y; w[i][2] = wi.z; w[i][3] = wi.w;
        }
    }
    // the sequence holding token tb: [bos, eos)
    int n, bos, eos;
    if (p.cu) {
        int lo = 0, hi = p.num_seqs - 1;         // last n with cu[n] <= tb
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.cu[mid] <= tb) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
        while (p.cu[n + 1] <= tb) ++n;           // skip empty sequences that start at tb
        bos = p.cu[n];
        eos = p.cu[n + 1];
    } else {
        n = tb / p.T;
        bos = n * p.T;
        eos = bos + p.T;
    }
    // x_{t-1}, x_{t-2}, x_{t-3} of the current token t
    float h1[8], h2[8], h3[8];
    auto input_at = [&](int pos, float (&v)[8]) {   // pos >= bos - 3
        if (pos >= bos) {
            load8(x + (size_t)pos * p.C + c0, v);
        } else if (st) {
            load8(st + ((size_t)n * 3 + (3 + pos - bos)) * p.C + c0, v);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = 0.f;
        }
    };
    auto window = [&](int t) {
        input_at(t - 1, h1);
        input_at(t - 2, h2);
        input_at(t - 3, h3);
    };
    if (active) window(tb);

    const bool is_q = c0 < p.qk_half, is_k = !is_q && c0 < p.QK;
    XT *outp;
    size_t ostride;   // elements per token of the output this channel goes to
    int oc;           // channel within that output
    if (is_q) { outp = static_cast<XT *>(p.q); ostride = p.qk_half; oc = c0; }
    else if (is_k) { outp = static_cast<XT *>(p.k); ostride = p.qk_half; oc = c0 - p.qk_half; }
    else { outp = static_cast<XT *>(p.v); ostride = p.dv_total; oc = c0 - p.QK; }

    // one input row in flight per thread: requesting several rows ahead was
    // measured slower (2 rows: +10%, 4: +15%), the workgroups resident on a
    // CU already keep enough loads in flight
    for (int t = tb; t < te; ++t) {
        if (t == eos) {                           // next sequence (packed: skipping empty ones)
            if (p.cu) {
                do {
                    ++n;
                    bos = p.cu[n];
                    eos = p.cu[n + 1];
                } while (eos == bos);
            } else {
                ++n;
                bos = eos;
                eos = bos + p.T;
            }
            if (active) window(t);
        }
        float y[8];
        if (active) {
            float x0[8];
            load8(x + (size_t)t * p.C + c0, x0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                y[i] = w[i][0] * h3[i] + w[i][1] * h2[i] + w[i][2] * h1[i] + w[i][3] * x0[i];
                if constexpr (SILU) y[i] = y[i] / (1.f + __expf(-y[i]));
                h3[i] = h2[i];
                h2[i] = h1[i];
                h1[i] = x0[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = 0.f;
        }
        if constexpr (NORM) {
            // every lane takes part in the DPP sums; only q/k lanes use them
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += y[i] * y[i];
            ss = dpp_sum<DK / 8>(ss);
            if (is_q || is_k) {
                const float sc = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] *= sc;
            }
        }
        if (active) store8(outp + (size_t)t * ostride + oc, y);
    }
}

struct PrologueGateArgs {
    int H, NA;                    // value heads; log-alpha values per (token, head): 1 or dk
    long tokens;
    const float *a, *b;
    float *beta, *log_alpha;
    // convolution state
    int C, num_seqs, T;
    const void *x, *state_in;
    void *state_out;
    const int32_t *cu;
};

template <typename XT>
__global__ __launch_bounds__(256) void prologue_gate_state_kernel(PrologueGateArgs p) {
    const long stride = (long)gridDim.x * blockDim.x;
    const long i0 = (long)blockIdx.x * blockDim.x + threadIdx.x;
    const long ngate = p.tokens * p.H * p.NA;
    for (long i = i0; i < ngate; i += stride) {
        const float a = p.a[i];
        p.log_alpha[i] = -(fmaxf(a, 0.f) + log1pf(__expf(-fabsf(a))));   // -softplus(a)
    }
    for (long i = i0; i < p.tokens * p.H; i += stride) p.beta[i] = 1.f / (1.f + __expf(-p.b[i]));   // sigmoid(b)
    if (!p.state_out) return;
    // new state of sequence n: the inputs at positions eos-3 .. eos-1, older
    // state rows where the sequence is shorter than three tokens (all three
    // rows of one channel vector read before any is written: in place safe)
    const XT *x = static_cast<const XT *>(p.x);
    const XT *si = static_cast<const XT *>(p.state_in);
    XT *so = static_cast<XT *>(p.state_out);
    const int CV = p.C / 8;
    for (long i = i0; i < (long)p.num_seqs * CV; i += stride) {
        const int n = (int)(i / CV), c = (int)(i % CV) * 8;
        const int bos = p.cu ? p.cu[n] : n * p.T, eos = p.cu ? p.cu[n + 1] : bos + p.T;
        float r[3][8];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int pos = eos - 3 + j;
            if (pos >= bos) load8(x + (size_t)pos * p.C + c, r[j]);
            else if (si) load8(si + ((size_t)n * 3 + (3 + pos - bos)) * p.C + c, r[j]);
            else {
#pragma unroll
                for (int e = 0; e < 8; ++e) r[j][e] = 0.f;
            }
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) store8(so + ((size_t)n * 3 + j) * p.C + c, r[j]);
    }
}

template <typename XT, int DK>
static hipError_t launch_prologue_dk(const PrologueArgs &a, hipStream_t st) {
    const int C = 2 * a.num_qk_heads * a.dk + a.num_heads * a.dv;
    const int total = a.batch * a.seqlen;
    if (total > 0) {
        PrologueKArgs p;
        p.T = a.seqlen;
        p.C = C;
        p.QK = 2 * a.num_qk_heads * a.dk;
        p.num_seqs = a.num_seqs;
        p.total_tokens = total;
        p.x = a.x;
        p.w = a.conv_weight;
        p.state_in = a.state_in;
        p.cu = a.cu_seqlens;
        p.q = a.q; p.k = a.k; p.v = a.v;
        p.qk_half = a.num_qk_heads * a.dk;
        p.dv_total = a.num_heads * a.dv;
        const dim3 grid((unsigned)div_up(total, kPrologueTokens), (unsigned)div_up(C, 8 * kPrologueThreads));
#define GDR_PRO(S, N) hipLaunchKernelGGL((prologue_conv_kernel<XT, DK, S, N>), grid, dim3(kPrologueThreads), 0, st, p)
        if (a.silu) {
            if (a.qk_norm) GDR_PRO(true, true);
            else GDR_PRO(true, false);
        } else {
            if (a.qk_norm) GDR_PRO(false, true);
            else GDR_PRO(false, false);
        }
#undef GDR_PRO
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    PrologueGateArgs g;
    g.H = a.num_heads;
    g.NA = a.kda ? a.dk : 1;
    g.tokens = total;
    g.a = a.a_logit;
    g.b = a.b_logit;
    g.beta = a.beta;
    g.log_alpha = a.log_alpha;
    g.C = C;
    g.num_seqs = a.num_seqs;
    g.T = a.seqlen;
    g.x = a.x;
    g.state_in = a.state_in;
    g.state_out = a.state_out;
    g.cu = a.cu_seqlens;
    const long work = std::max<long>((long)total * a.num_heads * g.NA, (long)a.num_seqs * (C / 8));
    if (work == 0) return hipSuccess;
    const unsigned blocks = (unsigned)std::min<long>(div_up((int)std::min<long>(work, 1L << 30), 256), 8192);
    hipLaunchKernelGGL((prologue_gate_state_kernel<XT>), dim3(blocks), dim3(256), 0, st, g);
    return hipGetLastError();
}

template <typename XT>
static hipError_t launch_prologue_x(const PrologueArgs &a, hipStream_t st) {
    switch (a.dk) {
        case 16: return launch_prologue_dk<XT, 16>(a, st);
        case 32: return launch_prologue_dk<XT, 32>(a, st);
        case 64: return launch_prologue_dk<XT, 64>(a, st);
        case 128: return launch_prologue_dk<XT, 128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prologue(const PrologueArgs &a, hipStream_t st) {
    return a.x_bf16 ? launch_prologue_x<__bf16>(a, st) : launch_prologue_x<float>(a, st);
}

}  // namespace gdr
