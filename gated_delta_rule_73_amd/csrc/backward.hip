// backward.hip -- gradients of the chunked prefill (training).
//
// The recurrence (page "How the New Flash Models Work: Inside GLM-5.3-Flash
// and Qwen3.8-Flash-Next", section "Linear attention: a fixed-size memory in
// place of the cache": the Gated DeltaNet and Kimi Delta Attention
// equations) is trained with the layers around it; the pages describe that
// training but print no backward pass, so what follows is the chain rule of
// the chunked forward form, arranged for the GPU.
//
// Within a chunk of C tokens with incoming state S0 (d_v x d_k), g the
// within-chunk inclusive cumulative log-decay (per key channel; one value per
// row for a per-head decay) and beta, the forward computes
//     U   = T diag(b) V + Wn S0^T,   T = (I + strict_tril(diag(b) (K e^g)(K e^-g)^T))^-1,
//                                    Wn = -T diag(b) (K e^g)
//     O   = scale ((Q e^g) S0^T + M U),  M = tril((Q e^g)(K e^-g)^T)
//     S_C = S0 Diag(e^{g_C}) + U^T (K e^{g_C - g}).
// Its adjoint carries the state gradient backwards without the forward state:
//     dU      = M^T dO' + K_end dS_C^T                  (dO' = scale dO)
//     dS_prev = dS_C Diag(e^{g_C}) + dO'^T (Q e^g) + dU^T Wn
// and each chunk's input gradients follow from its own S0 and dS_C.
//
// Three kernels, fp32 data and accumulation; the products with a d_k or d_v
// contraction run as split bf16 products (split8, mfma_split), the C x C ones
// on the 16x16x4 fp32 MFMA:
//   bwd_prep_kernel  one workgroup per (chunk, head): the chunk record
//                    D = e^{g_C}, T, M, Wn, Q e^g, K_end (fp32, in HBM).
//   bwd_scan_kernel  one workgroup per (sequence, head, 32 or 64 value rows),
//                    walking the sequence's chunks: forward from the initial
//                    state, writing each chunk's incoming state; then
//                    backward from the final-state gradient, writing each
//                    chunk's outgoing state gradient and, at the end, the
//                    initial-state gradient.  Each wave keeps its 16 x d_k
//                    slice of the state transposed in MFMA accumulators, so
//                    the products with the state take it as an operand
//                    straight from registers.
//   bwd_grad_kernel  one workgroup per (chunk, head): every input gradient of
//                    the chunk from its two states (no cross-chunk sums, no
//                    atomics: the result is deterministic).
// The Gram-like products of the gradient pass use operands shifted by a
// per-channel reference exponent m (the midpoint of g over the chunk):
// (K e^{g-m}), (K e^{m-g}), (Q e^{g-m}), so no factor exceeds
// e^{(g_first - g_last)/2}.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace gdr {

constexpr int kBC = 32;                      // chunk length of the backward
constexpr int kGradThreads = 512;            // 8 waves: two per SIMD (the LDS holds one workgroup)

// Record of one (chunk, head), fp32: D[dk] | T[C][C] | M[C][C] | Wn[C][dk] |
// Qg[C][dk] (Q e^g) | Ke[C][dk] (K e^{g_C - g}) | G[C]; stride from launch.h.
// With a per-head decay, Q e^g and K e^{g_C - g} are q and k scaled per row,
// and G holds the rows' cumulative log decay.  When the four-wave state scan
// runs (raw_qk), it stages q and k themselves, scaled as they reach LDS, and
// Qg, Ke are not written: the scan's fetch, which bounds it, shrinks by a
// third.  (With two-wave scans, whose chains are latency-bound, the scattered
// q/k rows cost more than the bytes saved.)
template <int DK> struct BRec {
    static constexpr int D = 0, T = DK, M = T + kBC * kBC, W = M + kBC * kBC, Q = W + kBC * DK,
                         KE = Q + kBC * DK, G = KE + kBC * DK;
};

struct BwdKArgs {
    int batch, seqlen, H, dv, num_seqs;
    int Hk, G;                                // q/k heads; value heads per q/k head (H = Hk G)
    const void *q, *k, *v;
    const void *beta, *log_alpha;             // fp32, or bf16 (the kernels' GT)
    const float *initial_state;
    const int32_t *cu, *order, *choff;
    float scale;
    const float *d_out, *d_final;
    float *dq, *dk, *dv_out, *dbeta, *dla, *d_init;   // dq, dk: per value head ([.., H, dk])
    float *rec, *states, *dstates;
    long rec_stride;                          // floats per record
    int raw_qk;                               // per-head decay, four-wave scans: see BRec
    // Dense batches in time segments: this launch covers chunks [seg_c0,
    // seg_c0 + seg_nc) of every sequence, its records and states indexed
    // from the segment's first chunk (seg_nc = 0: every chunk).  fwd_final:
    // the forward pass also writes the state after its last chunk; no_dump:
    // it writes no per-chunk states.
    int seg_c0, seg_nc;
    float *fwd_final;
    int no_dump;
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// One 16x16 output tile of a product: acc += sum_k A(m, k) B(k, n) for
// k < K <= KMAX, K a multiple of 32 (d_v, d_k or the chunk length), where
// fa(mi, k) = A(m0 + mi, k) and fb(k, ni) = B(k, n0 + ni).  On return acc[i]
// holds the element (m0 + 4 (lane >> 4) + i, n0 + (lane & 15)).  Each block of
// 32 k gathers its operands first (their loads in flight together), then runs
// its eight MFMAs.
template <int KMAX, class FA, class FB>
__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, int K, FA fa, FB fb) {
    static_assert(KMAX % 32 == 0, "k blocks of 32");
    const int l = threadIdx.x & 63, lr = l & 15, lq = l >> 4;
#pragma unroll
    for (int kb = 0; kb < KMAX; kb += 32) {
        if (kb < K) {
            float a[8], b[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                a[s] = fa(lr, kb + 4 * s + lq);
                b[s] = fb(kb + 4 * s + lq, lr);
            }
#pragma unroll
            for (int s = 0; s < 8; ++s) acc = mfma4(a[s], b[s], acc);
        }
    }
    // keep the next product's operand loads behind this one
    __builtin_amdgcn_sched_barrier(0);
    return acc;
}

// NQ tiles at once: acc[q] += sum_k A_q(m, k) B_q(k, n), with
// fa(q, mi, kb, lk) = A_q(m0 + mi, kb + lk) and fb(q, kb, lk, ni) =
// B_q(kb + lk, n0 + ni): kb is the wave-uniform part of k (a constant once
// unrolled, so a buffer load can carry it as its scalar offset), lk the
// lane's part.  The operands of a block of 32 k (every product's;
// identical loads are shared) are gathered one block ahead of its 8 NQ
// MFMAs, so products that read the same slow operand wait for it once and
// the wait overlaps the previous block's MFMAs.
template <int KMAX, int NQ, class FA, class FB>
__device__ __forceinline__ void tile_mma_n(f32x4 (&acc)[NQ], int K, FA fa, FB fb) {
    static_assert(KMAX % 32 == 0, "k blocks of 32");
    constexpr int NB = KMAX / 32;
    const int l = threadIdx.x & 63, lr = l & 15, lq = l >> 4;
    float a[2][NQ][8], b[2][NQ][8];
    auto gather = [&](int blk, int buf) {
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                a[buf][q][s] = fa(q, lr, 32 * blk + 4 * s, lq);
                b[buf][q][s] = fb(q, 32 * blk + 4 * s, lq, lr);
            }
    };
    gather(0, 0);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
        if (32 * blk < K) {
            if (blk + 1 < NB && 32 * (blk + 1) < K) gather(blk + 1, (blk + 1) & 1);
#pragma unroll
            for (int s = 0; s < 8; ++s)
#pragma unroll
                for (int q = 0; q < NQ; ++q) acc[q] = mfma4(a[blk & 1][q][s], b[blk & 1][q][s], acc[q]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Split bf16 operands: x = hi + lo with hi = bf16(x), lo = bf16(x - hi)
// (x - hi is exact in fp32), 16 significant bits with fp32's exponent range.
// A product takes hi*hi + hi*lo + lo*hi on the 16x16x32 bf16 MFMA with fp32
// accumulation; the dropped lo*lo term and the rounding of lo are below
// 2^-16 of each operand product.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
// two values at once (one packed conversion each for hi and lo): the
// returned words hold x0 in their low and x1 in their high half
__device__ __forceinline__ void split2(float x0, float x1, unsigned &hi, unsigned &lo) {
    const unsigned h = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2v){x0, x1}, bf16x2v));
    const float h0 = __builtin_bit_cast(float, h << 16), h1 = __builtin_bit_cast(float, h & 0xffff0000u);
    hi = h;
    lo = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2v){x0 - h0, x1 - h1}, bf16x2v));
}
__device__ __forceinline__ void split4(const f32x4 v, bf16x4 &hi, bf16x4 &lo) {
    unsigned h0, h1, l0, l1;
    split2(v[0], v[1], h0, l0);
    split2(v[2], v[3], h1, l1);
    hi = __builtin_bit_cast(bf16x4, (u32x2){h0, h1});
    lo = __builtin_bit_cast(bf16x4, (u32x2){l0, l1});
}
// the operand of one 32-k MFMA step from two accumulator tiles (k = 4 lq + i
// of tile a, then of tile b)
__device__ __forceinline__ void split8(const f32x4 a, const f32x4 b, bf16x8 &hi, bf16x8 &lo) {
    unsigned h0, h1, h2, h3, l0, l1, l2, l3;
    split2(a[0], a[1], h0, l0);
    split2(a[2], a[3], h1, l1);
    split2(b[0], b[1], h2, l2);
    split2(b[2], b[3], h3, l3);
    hi = __builtin_bit_cast(bf16x8, (u32x4){h0, h1, h2, h3});
    lo = __builtin_bit_cast(bf16x8, (u32x4){l0, l1, l2, l3});
}
__device__ __forceinline__ f32x4 mfma_split(const bf16x8 &ah, const bf16x8 &al, const bf16x8 &bh,
                                            const bf16x8 &bl, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
}
// Raw buffer loads: the byte offset splits into a per-lane VGPR part and a
// uniform scalar part, so a sweep over k needs no per-k address registers.
constexpr int kRawBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const float *base, long floats) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, (int)(floats * 4), kRawBufferWord3);
}
__device__ __forceinline__ float bload(__amdgpu_buffer_rsrc_t r, int lane_bytes, int uniform_bytes) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, lane_bytes, uniform_bytes, 0));
}

// Loads with the non-temporal cache hint, for data a workgroup reads once or
// for the last time: the L2 evicts such lines first, so they do not push out
// lines that are read again (the grad kernel's states, read row-wise for Y and
// K_end dS^T, then column-wise for dq and dk).  Fetch measured with and without
// (KDA 32K): 19.9 against 21.5 GB per call.
constexpr int kNonTemporal = 2;   // the cache-policy operand's nt bit on this chip
__device__ __forceinline__ float bload_last(__amdgpu_buffer_rsrc_t r, int lane_bytes, int uniform_bytes) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, lane_bytes, uniform_bytes, kNonTemporal));
}
__device__ __forceinline__ float4 load4_once(const float *p) {
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float4 load4_once(const __bf16 *p) {
    const bf16x4 v = __builtin_nontemporal_load(reinterpret_cast<const bf16x4 *>(p));
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}
template <typename T> __device__ __forceinline__ float ld1_once(const T *p) { return to_f32(__builtin_nontemporal_load(p)); }

__device__ __forceinline__ f32x4 lds4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f32x4 bload4(__amdgpu_buffer_rsrc_t r, int lane_bytes, int uniform_bytes) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, lane_bytes, uniform_bytes, 0));
}

// NQ tiles of A_q B_q^T products whose operands are both contiguous along k
// (rows of A_q and rows of B_q^T): a lane reads four consecutive k of each as
// one 16-byte access and spends them on four MFMA steps, lane group lq taking
// k = kb + 4 lq + s in step s (the same on both sides, so the sum is the
// same).  fa4(q, mi, kb, lk) = A_q(m0 + mi, kb + lk .. kb + lk + 3) and
// fb4(q, ni, kb, lk) = B_q^T(n0 + ni, kb + lk .. kb + lk + 3); kb is
// wave-uniform.  Blocks of 32 k, gathered one block ahead of their MFMAs;
// each block is one split bf16 product (16x16x32, hi/lo operands, see
// split8): a lane's k = kb + 4 lq + s and kb + 16 + 4 lq + s are the eight
// k it supplies to that MFMA.
template <int KMAX, int NQ, class FA, class FB>
__device__ __forceinline__ void tile_mma_nt(f32x4 (&acc)[NQ], int K, FA fa4, FB fb4) {
    static_assert(KMAX % 32 == 0, "k blocks of 32");
    constexpr int NB = KMAX / 32;
    const int l = threadIdx.x & 63, lr = l & 15, lq = l >> 4;
    f32x4 a[2][NQ][2], b[2][NQ][2];
    auto gather = [&](int blk, int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                a[buf][q][h] = fa4(q, lr, 32 * blk + 16 * h, 4 * lq);
                b[buf][q][h] = fb4(q, lr, 32 * blk + 16 * h, 4 * lq);
            }
    };
    gather(0, 0);
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
        if (32 * blk < K) {                     // K (a multiple of 32) is wave-uniform
            if (blk + 1 < NB && 32 * (blk + 1) < K) gather(blk + 1, (blk + 1) & 1);
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                bf16x8 ah, al, bh, bl;
                split8(a[blk & 1][q][0], a[blk & 1][q][1], ah, al);
                split8(b[blk & 1][q][0], b[blk & 1][q][1], bh, bl);
                acc[q] = mfma_split(ah, al, bh, bl, acc[q]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// e^x for the decay factors: the hardware exponential on x log2(e).  Its
// relative error grows with |x|, to about 5e-6 at the +-80 the chunk decay
// bound allows, far below the gradients' tolerance.
__device__ __forceinline__ float fexp(float x) { return __expf(x); }

template <typename IT> __device__ __forceinline__ float ld1(const IT *p) { return to_f32(*p); }
// gates (beta, log alpha): fp32 or bf16 storage, fp32 arithmetic
template <typename GT> __device__ __forceinline__ float gate1(const void *g, long o) {
    return to_f32(static_cast<const GT *>(g)[o]);
}
template <typename GT> __device__ __forceinline__ float4 gate4(const void *g, long o) {
    return load4(static_cast<const GT *>(g) + o);
}

// Where record chunk rc lies: its sequence, first token (flat index over
// batch x seqlen) and length; len <= 0 past the last chunk of a packed batch.
struct ChunkLoc {
    int n;
    long tok0;
    int len;
};
__device__ __forceinline__ ChunkLoc locate(const BwdKArgs &p, long rc) {
    ChunkLoc L;
    if (!p.cu) {
        const int nct = p.seg_nc ? p.seg_nc : div_up(p.seqlen, kBC);
        L.n = (int)(rc / nct);
        const int c = p.seg_c0 + (int)(rc % nct);
        L.tok0 = (long)L.n * p.seqlen + (long)c * kBC;
        L.len = std::min(kBC, p.seqlen - c * kBC);
        return L;
    }
    if (rc >= p.choff[p.num_seqs]) {
        L.n = 0, L.tok0 = 0, L.len = 0;
        return L;
    }
    int lo = 0, hi = p.num_seqs - 1;          // last n with choff[n] <= rc
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (p.choff[mid] <= rc) lo = mid; else hi = mid - 1;
    }
    const int c = (int)(rc - p.choff[lo]);
    L.n = lo;
    L.tok0 = p.cu[lo] + (long)c * kBC;
    L.len = std::min((long)kBC, (long)p.cu[lo + 1] - L.tok0);
    return L;
}

// Scans over the 32 rows of one column, four adjacent lanes per column and
// eight rows per lane.  seg_scan4: the lane's own running sums over its rows
// of x[.][j] (prefix, or suffix when rev) into v; returns its rows' total.
// scan4_offsets: what the other lanes of the column add (the totals of the
// rows before the lane's, or after them when rev) and the column total.
template <class X>
__device__ __forceinline__ float seg_scan4(X &x, int qd, int j, float (&v)[kBC / 4], bool rev) {
    constexpr int RQ = kBC / 4;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < RQ; ++i) {
        const int rr = rev ? RQ - 1 - i : i;
        s += x[qd * RQ + rr][j];
        v[rr] = s;
    }
    return s;
}
__device__ __forceinline__ void scan4_offsets(float tot, int qd, bool rev, float &other, float &total) {
    // inclusive scan of the four totals in the lane order (or reversed)
    const float a1 = rev ? __shfl_down(tot, 1, 4) : __shfl_up(tot, 1, 4);
    const float s1 = tot + ((rev ? qd < 3 : qd > 0) ? a1 : 0.f);
    const float a2 = rev ? __shfl_down(s1, 2, 4) : __shfl_up(s1, 2, 4);
    const float incl = s1 + ((rev ? qd < 2 : qd > 1) ? a2 : 0.f);
    const float ex = rev ? __shfl_down(incl, 1, 4) : __shfl_up(incl, 1, 4);
    other = (rev ? qd < 3 : qd > 0) ? ex : 0.f;
    total = __shfl(incl, rev ? 0 : 3, 4);
}

// ---------------------------------------------------------------------------
// Chunk records.
template <int DK, bool KDA, typename IT, typename GT>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdKArgs p) {
    constexpr int C = kBC, PK = DK + 4, NT = 256;
    using R = BRec<DK>;
    __shared__ __align__(16) float sK[C][PK], sQ[C][PK], sX[C][PK], sKh[C][PK];
    __shared__ float sA[C][C + 1], sT[C][C + 1];
    __shared__ float sg[C], sb[C], sm[DK], sgl[DK];
    const int H = p.H, h = blockIdx.y, tid = threadIdx.x;
    const long rc = blockIdx.x;
    const ChunkLoc L = locate(p, rc);
    if (L.len <= 0) return;
    const IT *q = static_cast<const IT *>(p.q), *k = static_cast<const IT *>(p.k);
    float *rec = p.rec + (rc * H + h) * p.rec_stride;

    // every load first (clamped rows, all in flight together), then the LDS
    // stores; padding rows are zeroed by a select, not a branch
    constexpr int NL4 = div_up(C * DK / 4, NT);
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 kv[NL4], qv[NL4], gv[NL4];
#pragma unroll
    for (int u = 0; u < NL4; ++u) {
        const int e = min(tid + NT * u, C * DK / 4 - 1), r = e / (DK / 4), j = (e % (DK / 4)) * 4;
        const long t = L.tok0 + min(r, L.len - 1);
        const long o = (t * H + h) * DK + j, oq = (t * p.Hk + h / p.G) * DK + j;
        kv[u] = load4(k + oq);
        qv[u] = load4(q + oq);
        gv[u] = KDA ? gate4<GT>(p.log_alpha, o) : z4;
    }
    const long ob = (L.tok0 + min(tid & (C - 1), L.len - 1)) * H + h;
    const float bb = gate1<GT>(p.beta, ob), gg = KDA ? 0.f : gate1<GT>(p.log_alpha, ob);
#pragma unroll
    for (int u = 0; u < NL4; ++u) {
        const int e = tid + NT * u;
        if (e >= C * DK / 4) continue;
        const int r = e / (DK / 4), j = (e % (DK / 4)) * 4;
        const bool in = r < L.len;
        const float4 k4 = in ? kv[u] : z4, q4 = in ? qv[u] : z4, g4 = in ? gv[u] : z4;
        sK[r][j] = k4.x, sK[r][j + 1] = k4.y, sK[r][j + 2] = k4.z, sK[r][j + 3] = k4.w;
        sQ[r][j] = q4.x, sQ[r][j + 1] = q4.y, sQ[r][j + 2] = q4.z, sQ[r][j + 3] = q4.w;
        if (KDA) sX[r][j] = g4.x, sX[r][j + 1] = g4.y, sX[r][j + 2] = g4.z, sX[r][j + 3] = g4.w;
    }
    if (tid < C) {
        const bool in = tid < L.len;
        sb[tid] = in ? bb : 0.f;
        if (!KDA) sg[tid] = in ? gg : 0.f;
    }
    __syncthreads();
    // inclusive cumulative log-decay (padding rows add zero)
    if (KDA) {
        // four adjacent lanes per channel, eight rows each
        for (int e = tid; e < 4 * DK; e += NT) {
            const int j = e >> 2, qd = e & 3;
            float v[C / 4];
            const float tot = seg_scan4(sX, qd, j, v, false);
            float before, total;
            scan4_offsets(tot, qd, false, before, total);
#pragma unroll
            for (int rr = 0; rr < C / 4; ++rr) sX[qd * (C / 4) + rr][j] = before + v[rr];
            if (qd == 0) {
                sm[j] = 0.5f * (v[0] + total);
                sgl[j] = total;
            }
        }
    } else if (tid < 64) {
        float g = tid < C ? sg[tid] : 0.f;
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
            const float t = __shfl_up(g, o, 32);
            if ((tid & 31) >= o) g += t;
        }
        const float first = __shfl(g, 0), total = __shfl(g, C - 1);
        if (tid < C) sg[tid] = g;
        if (tid == 0) {
            sm[0] = 0.5f * (first + total);
            sgl[0] = total;
        }
    }
    __syncthreads();
    for (int e = tid; e < C * DK; e += NT) {
        const int r = e / DK, j = e % DK;
        const float g = KDA ? sX[r][j] : sg[r], m = KDA ? sm[j] : sm[0], gl = KDA ? sgl[j] : sgl[0];
        const float kk = sK[r][j], qq = sQ[r][j];
        // e^{g} and e^{g_C - g} are at most 1; e^{g - m} and its reciprocal stay
        // within e^{+-(g_first - g_last)/2}
        const float eg = fexp(g), egm = fexp(g - m), emg = 1.f / egm;
        if (KDA || !p.raw_qk) {
            rec[R::Q + e] = qq * eg;
            rec[R::KE + e] = kk * fexp(gl - g);
        }
        sK[r][j] = kk * egm;
        sKh[r][j] = kk * emg;
        sQ[r][j] = qq * egm;
        sX[r][j] = sb[r] * kk * eg;
    }
    for (int j = tid; j < DK; j += NT) rec[R::D + j] = fexp(KDA ? sgl[j] : sgl[0]);
    if (!KDA && tid < C) rec[R::G + tid] = sg[tid];
    __syncthreads();

    const int w = tid >> 6, l = tid & 63, lr = l & 15, lq = l >> 4;
    {   // A = strict_tril(diag(b) Kts Khs^T), M = tril(Qts Khs^T): one tile each per wave
        const int rt = w & 1, ct = w >> 1;
        f32x4 am[2] = {zero4(), zero4()};
        tile_mma_nt<DK, 2>(am, DK, [&](int q, int mi, int kb, int lk) {
                               return lds4(q ? &sQ[16 * rt + mi][kb + lk] : &sK[16 * rt + mi][kb + lk]);
                           },
                           [&](int, int ni, int kb, int lk) { return lds4(&sKh[16 * ct + ni][kb + lk]); });
        const f32x4 a = am[0], mm = am[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * lq + i, c = 16 * ct + lr;
            sA[r][c] = c < r ? sb[r] * a[i] : 0.f;
            rec[R::M + r * C + c] = c <= r ? mm[i] : 0.f;
        }
    }
    __syncthreads();
    // T = (I + A)^-1 by 16 x 16 blocks.  The diagonal blocks by forward
    // substitution row by row: lane j of a half-wave keeps column j of its block
    // in registers and reads A's entries as LDS broadcasts (fully unrolled);
    // then T21 = -T22 (A21 T11) by two MFMA products; T12 = 0.
    if (tid < 32) {
        const int o = 16 * (tid >> 4), j = tid & 15;
        float col[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float t = r == j ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < r; ++i) t -= sA[o + r][o + i] * col[i];
            col[r] = t;                         // zero above the diagonal (col[i] = 0 for i < j)
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            sT[o + r][o + j] = col[r];
            sT[r][16 + j] = 0.f;                // T12 (both half-waves write the same zeros)
        }
    }
    __syncthreads();
    if (w == 0) {   // X = A21 T11 into T12's place (zero again below)
        f32x4 x = zero4();
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) x = mfma4(sA[16 + lr][k0 + lq], sT[k0 + lq][lr], x);
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[4 * lq + i][16 + lr] = x[i];
    }
    __syncthreads();
    if (w == 0) {   // T21 = -T22 X
        f32x4 t21 = zero4();
#pragma unroll
        for (int k0 = 0; k0 < 16; k0 += 4) t21 = mfma4(sT[16 + lr][16 + k0 + lq], sT[k0 + lq][16 + lr], t21);
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[16 + 4 * lq + i][lr] = -t21[i];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[4 * lq + i][16 + lr] = 0.f;
    }
    __syncthreads();
    for (int e = tid; e < C * C; e += NT) rec[R::T + e] = sT[e / C][e % C];
    // Wn = -T (diag(b) K e^g)
    for (int t = w; t < 2 * (DK / 16); t += NT / 64) {
        const int rt = t & 1, jt = t >> 1;
        const f32x4 acc = tile_mma<C>(zero4(), C, [&](int mi, int kk) { return sT[16 * rt + mi][kk]; },
                                   [&](int kk, int ni) { return sX[kk][16 * jt + ni]; });
#pragma unroll
        for (int i = 0; i < 4; ++i) rec[R::W + (16 * rt + 4 * lq + i) * DK + 16 * jt + lr] = -acc[i];
    }
}

// ---------------------------------------------------------------------------
// State scan over a sequence's chunks.  A workgroup of NW waves takes 16 NW
// value rows of one (sequence, head); each wave keeps its 16 x d_k slice of X
// transposed in MFMA accumulators.
//   forward  (BWD = false): X = state;  P = T diag(b) V + Wn X^T,
//            X <- X Diag(D) + P^T K_end; writes X before each chunk.
//   backward (BWD = true):  X = state gradient; Z = scale dO;
//            P = M^T Z + K_end X^T, X <- X Diag(D) + P^T Wn + Z^T (Q e^g);
//            writes X before each chunk (the chunk's outgoing gradient) and
//            the initial-state gradient at the end.
// The workgroup has NW more waves that only load: they fetch chunk s + 2's
// record and inputs into registers and write chunk s + 1's, split, to the
// other half of a double-buffered LDS stage while the NW state waves run
// chunk s: one barrier per chunk, which waits for LDS operations only, so
// the loads stay in flight across it.  (A wave whose loads queue at the CU's
// memory pipeline issues nothing else; with the loads in the state waves,
// the fetch and the products of a chunk took turns.)  The workgroups of one
// (sequence, head) sit on one XCD (block b runs on XCD b mod 8), so its
// records come from HBM once and from that XCD's L2 for the other slices.
//
// Products on the 16x16x32 bf16 MFMA with split operands (split8,
// mfma_split; bf16 rather than fp16 because the state gradient has no
// fp16-sized bound).  The state and P stay in fp32 accumulators and are split
// afresh in registers for each chunk.
//
// Operand planes in LDS are blocks of 32 k (rows x 32, 64 bytes per row).
// Inside a block the k order is permuted so that the eight k one lane
// supplies to one MFMA -- k = 4 lq + i and 16 + 4 lq + i (i < 4): the layout
// of two fp32 accumulator tiles -- sit at eight consecutive positions
// 8 lq .. 8 lq + 7.  The 16 rows one wave reads are then 1 KB of contiguous
// LDS, read as one 16-byte access per lane per plane.
__device__ __forceinline__ int kperm32(int k) { return 8 * ((k & 15) >> 2) + 4 * ((k >> 4) & 1) + (k & 3); }

__device__ __forceinline__ bf16x8 lds8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// 4 x 4 transpose inside each quad of lanes: lane t holds row t of a 4 x 4
// block on entry and column t on return.  Two exchange stages over the DPP
// quad permutations: lanes t and t ^ 2 swap the off-diagonal 2 x 2 blocks,
// then lanes t and t ^ 1 swap the off-diagonal entries of each.
template <int CTRL> __device__ __forceinline__ float quad_perm(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ void quad_transpose(f32x4 &v) {
    const int t = threadIdx.x & 3;
    const bool b1 = t & 2, b0 = t & 1;
    float r0 = quad_perm<0x4E>(b1 ? v[0] : v[2]), r1 = quad_perm<0x4E>(b1 ? v[1] : v[3]);   // lanes t ^ 2
    v = f32x4{b1 ? r0 : v[0], b1 ? r1 : v[1], b1 ? v[2] : r0, b1 ? v[3] : r1};
    r0 = quad_perm<0xB1>(b0 ? v[0] : v[1]), r1 = quad_perm<0xB1>(b0 ? v[2] : v[3]);         // lanes t ^ 1
    v = f32x4{b0 ? r0 : v[0], b0 ? v[1] : r0, b0 ? r1 : v[2], b0 ? v[3] : r1};
}
__device__ __forceinline__ void sts4(__bf16 *p, const bf16x4 v) { *reinterpret_cast<bf16x4 *>(p) = v; }

// LDS of one scan workgroup, two stages; [.][0] hi, [.][1] lo planes.
//   E:  the operand multiplying the state (forward Wn, backward K_end),
//       [key block][chunk row][32 keys];
//   Bt: the state update's left operand (forward K_end, backward Wn),
//       transposed: [key][32 chunk rows];
//   Gt: backward only, (Q e^g) transposed: [key][32 chunk rows];
//   L:  forward T, backward M^T: [chunk row][32 chunk columns];
//   Zt: forward diag(b) V, backward scale dO, transposed:
//       [value row][32 chunk rows].
// Four loader waves beside the NW state waves, eight waves in all (wave w
// runs on SIMD w mod 4).  With four state waves, each SIMD holds one state
// and one loader wave.  With two, the loaders are waves 2, 3, 6 and 7, on the
// two SIMDs without a state wave, and waves 4 and 5 only keep the barrier
// count.  (Loaders sharing a SIMD with a state wave had taken ~35% longer per
// chunk than the others, GDN 8K clock stamps; apart, the GDN 8K backward went
// from 1.17 to 1.16 ms and the grouped GDN 32K one from 10.48 to 10.36 ms.)
constexpr int scan_loader_waves(int) { return 4; }
constexpr int scan_block_waves(int) { return 8; }
template <int NW> __device__ __forceinline__ bool scan_is_loader(int w) { return NW == 4 ? w >= 4 : (w & 3) >= 2; }
// a loader thread's index, 0 .. 255
template <int NW> __device__ __forceinline__ int scan_loader_thread(int tid) {
    const int w = tid >> 6;
    return NW == 4 ? tid - 256 : 64 * (2 * (w >> 2) + (w & 1)) + (tid & 63);
}

template <int DK, int NW> struct ScanLds {
    static constexpr int C = kBC, ZW = 16 * NW;
    __align__(16) __bf16 E[2][2][DK / 32][C][32];
    __align__(16) __bf16 Bt[2][2][DK][32];
    __align__(16) __bf16 Gt[2][2][DK][32];
    __align__(16) __bf16 L[2][2][C][32];
    __align__(16) __bf16 Zt[2][2][ZW][32];
    __align__(16) float D[2][DK];
};

template <int DK, int NW, bool BWD, bool KDA, typename IT, typename GT>
__device__ __forceinline__ void scan_body(const BwdKArgs &p, int block, ScanLds<DK, NW> &lds) {
    constexpr bool RAW = !KDA && NW == 4;     // q, k staged raw (BRec; the launch sets raw_qk to match)
    // column pieces loaded as rows and transposed in quads (see below), for
    // the record fields; the raw q, k rows measured faster with their
    // two-byte column loads
    constexpr bool COLT = !RAW;
    constexpr int C = kBC, NT = 64 * scan_loader_waves(NW), ZW = 16 * NW, NB = DK / 32;
    static_assert(NW == 2 || NW == 4, "scan wave layout");
    // per loader thread (NT of them): NE row pieces of E and NE column
    // pieces of Bt (and Gt), NL pieces of L, NZ column pieces of Zt; four
    // values each
    // (the last round of a count below NT leaves threads idle: their loads
    // are clamped to a valid piece, their LDS stores skipped)
    constexpr int TE = C * DK / 4, TL = C * C / 4, NE = div_up(TE, NT), NL = div_up(TL, NT), NZ = C * ZW / 4 / NT;
    static_assert(C * ZW % (4 * NT) == 0 && TE % NT == 0 && TL % NT == 0 && DK % 32 == 0, "scan tiling");
    using R = BRec<DK>;
    auto &sE = lds.E;
    auto &sBt = lds.Bt;
    auto &sGt = lds.Gt;
    auto &sL = lds.L;
    auto &sZt = lds.Zt;
    auto &sD = lds.D;
    const int H = p.H, DV = p.dv, S = DV / ZW;
    const int xcd = block & 7, kb = block >> 3;
    const int unit = xcd + 8 * (kb / S), slice = kb % S;
    if (unit >= p.num_seqs * H) return;
    const int n = p.cu ? p.order[unit / H] : unit / H, h = unit % H;
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, lr = l & 15, lq = l >> 4;
    const bool state = w < NW;                    // waves 0 .. NW - 1 hold the state
    const bool loader = scan_is_loader<NW>(w);    // (neither: only the barriers)
    int lt = scan_loader_thread<NW>(tid);         // loader thread index (made opaque per chunk below)
    long rc0, tok_base;
    int nc, len;
    if (p.cu) {
        rc0 = p.choff[n], nc = p.choff[n + 1] - p.choff[n];
        tok_base = p.cu[n], len = p.cu[n + 1] - p.cu[n];
    } else {
        nc = p.seg_nc ? p.seg_nc : div_up(p.seqlen, C), rc0 = (long)n * nc;
        tok_base = (long)n * p.seqlen + (long)p.seg_c0 * C, len = p.seqlen - p.seg_c0 * C;
    }
    const int row = ZW * slice + 16 * (w & (NW - 1)) + lr;   // a state lane's value row (as MFMA column)
    const IT *v = static_cast<const IT *>(p.v);
    const IT *kin = static_cast<const IT *>(p.k), *qin = static_cast<const IT *>(p.q);
    const int hq = h / p.G;

    // Thread-to-piece maps (element index e = tid + NT u):
    //  row pieces (E; forward L): four consecutive k of one row; eight
    //    threads cover one row's 32-k block, whose 64 bytes they write whole;
    //  column pieces (Bt, Gt, Zt; backward L): four consecutive rows of one
    //    column; 16 threads take 16 adjacent columns (64 contiguous bytes of
    //    each source row), and a wave writes 16 whole 64-byte LDS rows.  With
    //    COLT they are loaded as rows: each lane of a quad loads four columns
    //    of one of the piece's rows (col_load; a wave reads 64 contiguous
    //    bytes of 16 source rows), and quad_transpose turns the quad's 4 x 4
    //    block into its four column pieces.
    auto row_piece = [](int e, int &r, int &k) {       // k: first of four, 32 k per row block
        const int jj = e & 7;
        r = (e >> 3) & (C - 1);
        k = 32 * (e >> 8) + 4 * (jj >> 1) + 16 * (jj & 1);
    };
    auto col_piece = [](int e, int ncol, int &c, int &r4) {   // ncol: columns in all
        const int rest = e >> 6, nch = ncol / 16;
        c = 16 * (rest % nch) + (e & 15);
        r4 = 16 * (rest / nch) + 4 * ((e >> 4) & 3);
    };
    auto col_load = [](int e, int ncol, int &r, int &c4) {   // row r, columns c4 .. c4 + 3
        const int rest = e >> 6, nch = ncol / 16;
        c4 = 16 * (rest % nch) + 4 * ((e >> 2) & 3);
        r = 16 * (rest / nch) + 4 * ((e >> 4) & 3) + (e & 3);
    };

    f32x4 rE[NE], rB[NE], rG[BWD ? NE : 1], rL[NL], rZ[NZ];
    float rD = 0.f, rZb[NZ] = {};
    // the fetched chunk's length; raw q, k: its row log decays (lane l holds
    // row l mod 32), for scaling them in put
    float rGv = 0.f;
    int rClen = 0;
    auto fetch = [&](int s) {
        const int c = BWD ? nc - 1 - s : s;
        const long rc = rc0 + c, tok0 = tok_base + (long)c * C;
        const int clen = min(C, len - c * C);
        const float *rec = p.rec + (rc * H + h) * p.rec_stride;
        const float *eb = rec + (BWD ? R::KE : R::W), *bb = rec + (BWD ? R::W : R::KE);
        // (raw q, k: K_end and Q e^g come as q and k rows, clamped to valid
        // rows here and scaled or zeroed in put)
        auto qk_off = [&](int r, int c) { return ((tok0 + min(r, clen - 1)) * p.Hk + hq) * DK + c; };
#pragma unroll
        for (int u = 0; u < NE; ++u) {
            const int e = min(lt + NT * u, TE - 1);
            int r, j;
            row_piece(e, r, j);
            if (!RAW || !BWD) {
                rE[u] = *reinterpret_cast<const f32x4 *>(eb + r * DK + j);
            } else {
                const float4 k4 = load4(kin + qk_off(r, j));
                rE[u] = f32x4{k4.x, k4.y, k4.z, k4.w};
            }
            if (COLT) {
                int rr, c4;
                col_load(e, DK, rr, c4);
                rB[u] = *reinterpret_cast<const f32x4 *>(bb + rr * DK + c4);
                if (BWD) rG[u] = *reinterpret_cast<const f32x4 *>(rec + R::Q + rr * DK + c4);
            } else {
                int jc, r4;
                col_piece(e, DK, jc, r4);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    rB[u][t] = !RAW || BWD ? bb[(r4 + t) * DK + jc] : ld1(kin + qk_off(r4 + t, jc));
                    if (BWD) rG[u][t] = !RAW ? rec[R::Q + (r4 + t) * DK + jc] : ld1(qin + qk_off(r4 + t, jc));
                }
            }
        }
        if (RAW) rGv = rec[R::G + (l & (C - 1))];
        rClen = clen;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int e = min(lt + NT * u, TL - 1);
            if (BWD && COLT) {                // L = M^T: column pieces of M^T are row pieces of M
                int mr, mc4;
                col_load(e, C, mr, mc4);
                rL[u] = *reinterpret_cast<const f32x4 *>(rec + R::M + mr * C + mc4);
            } else if (BWD) {
                int r, c4;
                col_piece(e, C, r, c4);
#pragma unroll
                for (int t = 0; t < 4; ++t) rL[u][t] = rec[R::M + (c4 + t) * C + r];
            } else {
                int r, c4;
                row_piece(e, r, c4);
                rL[u] = *reinterpret_cast<const f32x4 *>(rec + R::T + r * C + c4);
            }
        }
        // loads from clamped, always-valid rows and a select for padding rows:
        // a load under a lane-dependent branch would make the compiler wait for
        // every load in flight, the record loads above included
        // (COLT: scaled and masked in put, after the loads have landed)
#pragma unroll
        for (int u = 0; u < NZ; ++u) {
            if (COLT) {
                int zr, zc4;
                col_load(lt + NT * u, ZW, zr, zc4);
                const long tr = (tok0 + min(zr, clen - 1)) * H + h, o = tr * DV + ZW * slice + zc4;
                if (BWD) {
                    rZ[u] = *reinterpret_cast<const f32x4 *>(p.d_out + o);
                } else {
                    const float4 v4 = load4(v + o);
                    rZ[u] = f32x4{v4.x, v4.y, v4.z, v4.w};
                    rZb[u] = gate1<GT>(p.beta, tr);
                }
            } else {
                int i, r4;
                col_piece(lt + NT * u, ZW, i, r4);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int r = r4 + t;
                    const long tr = (tok0 + min(r, clen - 1)) * H + h, o = tr * DV + ZW * slice + i;
                    const float z = BWD ? p.scale * p.d_out[o] : gate1<GT>(p.beta, tr) * ld1(v + o);
                    rZ[u][t] = r < clen ? z : 0.f;
                }
            }
        }
        rD = rec[R::D + (lt & (DK - 1))];
    };
    auto put = [&](int b) {
        if (COLT) {
            // the column pieces: Z scaled by its row's factor (zero past the
            // chunk's end), then every quad's rows turned into columns
#pragma unroll
            for (int u = 0; u < NZ; ++u) {
                int zr, zc4;
                col_load(lt + NT * u, ZW, zr, zc4);
                const float f = BWD ? p.scale : rZb[u];
#pragma unroll
                for (int t = 0; t < 4; ++t) rZ[u][t] = zr < rClen ? f * rZ[u][t] : 0.f;
                quad_transpose(rZ[u]);
            }
#pragma unroll
            for (int u = 0; u < NE; ++u) {
                quad_transpose(rB[u]);
                if (BWD) quad_transpose(rG[u]);
            }
            if (BWD) {
#pragma unroll
                for (int u = 0; u < NL; ++u) quad_transpose(rL[u]);
            }
        }
        if (RAW) {
            // K_end = k e^{g_C - g_r}, Q e^g = q e^{g_r}, zero past the chunk's
            // end: lane r forms row r's two factors, the pieces read them across
            // lanes (before any lane skips)
            const int rr = l & (C - 1);
            const float gC = __shfl(rGv, C - 1), in = rr < rClen ? 1.f : 0.f;
            const float fk = in * fexp(gC - rGv), fq = in * fexp(rGv);
#pragma unroll
            for (int u = 0; u < NE; ++u) {
                const int e = min(lt + NT * u, TE - 1);
                int r, j, jc, r4;
                row_piece(e, r, j);
                col_piece(e, DK, jc, r4);
                if (BWD) {
                    const float f = __shfl(fk, r);
#pragma unroll
                    for (int t = 0; t < 4; ++t) rE[u][t] *= f;
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (BWD) rG[u][t] *= __shfl(fq, r4 + t);
                    else rB[u][t] *= __shfl(fk, r4 + t);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < NE; ++u) {
            const int e = lt + NT * u;
            if (TE % NT != 0 && e >= TE) continue;
            bf16x4 hi, lo;
            int r, j;
            row_piece(e, r, j);
            split4(rE[u], hi, lo);
            sts4(&sE[b][0][j >> 5][r][kperm32(j)], hi);
            sts4(&sE[b][1][j >> 5][r][kperm32(j)], lo);
            int jc, r4;
            col_piece(e, DK, jc, r4);
            split4(rB[u], hi, lo);
            sts4(&sBt[b][0][jc][kperm32(r4)], hi);
            sts4(&sBt[b][1][jc][kperm32(r4)], lo);
            if (BWD) {
                split4(rG[u], hi, lo);
                sts4(&sGt[b][0][jc][kperm32(r4)], hi);
                sts4(&sGt[b][1][jc][kperm32(r4)], lo);
            }
        }
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int e = lt + NT * u;
            if (TL % NT != 0 && e >= TL) continue;
            int r, c4;
            if (BWD) col_piece(e, C, r, c4);
            else row_piece(e, r, c4);
            bf16x4 hi, lo;
            split4(rL[u], hi, lo);
            sts4(&sL[b][0][r][kperm32(c4)], hi);
            sts4(&sL[b][1][r][kperm32(c4)], lo);
        }
#pragma unroll
        for (int u = 0; u < NZ; ++u) {
            int i, r4;
            col_piece(lt + NT * u, ZW, i, r4);
            bf16x4 hi, lo;
            split4(rZ[u], hi, lo);
            sts4(&sZt[b][0][i][kperm32(r4)], hi);
            sts4(&sZt[b][1][i][kperm32(r4)], lo);
        }
        if (lt < DK) sD[b][lt] = rD;
    };

    f32x4 x[DK / 16];
    if (state) {
        const float *init = BWD ? p.d_final : p.initial_state;
#pragma unroll
        for (int jt = 0; jt < DK / 16; ++jt)
            x[jt] = init ? *reinterpret_cast<const f32x4 *>(init + (((long)n * H + h) * DV + row) * DK + 16 * jt + 4 * lq)
                         : zero4();
    } else if (loader) {
        if (nc > 0) {
            fetch(0);
            put(0);
        }
        if (nc > 1) fetch(1);
    }
    lds_barrier();
    // The two roles run separate loops, one barrier per chunk each (a barrier
    // counts waves, wherever they wait).  In one shared loop body the compiler
    // merged the roles' wait counters at the loop head, and a state wave, whose
    // only memory operations are its state dumps, waited there for those
    // stores to complete (GDN 8K backward 1.24 -> 1.17 ms when separated).
    if (loader) {
        for (int s = 0; s < nc; ++s) {
            // chunk s + 1 into the stage chunk s - 1 used, then chunk s + 2's
            // loads.  The thread index is made opaque each chunk, so the
            // pieces' addresses are formed where they are used rather than
            // kept in registers across the loop.
            int opaque_zero;
            asm volatile("v_mov_b32 %0, 0" : "=v"(opaque_zero));
            lt = scan_loader_thread<NW>((int)threadIdx.x + opaque_zero) & (NT - 1);   // (the mask keeps lt's range known)
            if (s + 1 < nc) {
                put((s & 1) ^ 1);
                if (s + 2 < nc) fetch(s + 2);
            }
            lds_barrier();
        }
    } else if (!state) {
        for (int s = 0; s < nc; ++s) lds_barrier();
    } else for (int s = 0; s < nc; ++s) {
        const int b = s & 1;
        const int c = BWD ? nc - 1 - s : s;
        const long rc = rc0 + c;
        if (!p.no_dump) {
            float *dump = (BWD ? p.dstates : p.states) + ((rc * H + h) * DV + row) * DK;
#pragma unroll
            for (int jt = 0; jt < DK / 16; ++jt) *reinterpret_cast<f32x4 *>(dump + 16 * jt + 4 * lq) = x[jt];
        }

        // the state as B operand of the products over keys (k = key)
        bf16x8 xh[NB], xl[NB];
#pragma unroll
        for (int kb2 = 0; kb2 < NB; ++kb2) split8(x[2 * kb2], x[2 * kb2 + 1], xh[kb2], xl[kb2]);
        const bf16x8 zh = lds8(&sZt[b][0][16 * w + lr][8 * lq]), zl = lds8(&sZt[b][1][16 * w + lr][8 * lq]);
        f32x4 pc[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4 acc = mfma_split(lds8(&sL[b][0][16 * rt + lr][8 * lq]), lds8(&sL[b][1][16 * rt + lr][8 * lq]), zh,
                                   zl, zero4());
#pragma unroll
            for (int kb2 = 0; kb2 < NB; ++kb2)
                acc = mfma_split(lds8(&sE[b][0][kb2][16 * rt + lr][8 * lq]), lds8(&sE[b][1][kb2][16 * rt + lr][8 * lq]),
                                 xh[kb2], xl[kb2], acc);
            pc[rt] = acc;
        }
        // P as B operand of the state update (k = chunk row)
        bf16x8 ph, pl;
        split8(pc[0], pc[1], ph, pl);
#pragma unroll
        for (int jt = 0; jt < DK / 16; ++jt) {
            f32x4 acc = x[jt];
            const f32x4 dv4 = *reinterpret_cast<const f32x4 *>(&sD[b][16 * jt + 4 * lq]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] *= dv4[i];
            acc = mfma_split(lds8(&sBt[b][0][16 * jt + lr][8 * lq]), lds8(&sBt[b][1][16 * jt + lr][8 * lq]), ph, pl, acc);
            if (BWD)
                acc = mfma_split(lds8(&sGt[b][0][16 * jt + lr][8 * lq]), lds8(&sGt[b][1][16 * jt + lr][8 * lq]), zh,
                                 zl, acc);
            x[jt] = acc;
        }
        lds_barrier();
    }
    float *fin = BWD ? p.d_init : p.fwd_final;
    if (state && fin) {
#pragma unroll
        for (int jt = 0; jt < DK / 16; ++jt)
            *reinterpret_cast<f32x4 *>(fin + (((long)n * H + h) * DV + row) * DK + 16 * jt + 4 * lq) = x[jt];
    }
}

// Both state passes in one launch: the first half of the grid walks the
// states forward, the second half the state gradients backward.  The two
// recurrences are independent, so each half fills the CUs the other leaves.
template <int DK, int NW, bool KDA, typename IT, typename GT>
__global__ __launch_bounds__(64 * scan_block_waves(NW)) void bwd_scan_kernel(BwdKArgs p, int half) {
    __shared__ ScanLds<DK, NW> lds;
    if ((int)blockIdx.x < half)
        scan_body<DK, NW, false, KDA, IT, GT>(p, blockIdx.x, lds);
    else
        scan_body<DK, NW, true, KDA, IT, GT>(p, blockIdx.x - half, lds);
}

// ---------------------------------------------------------------------------
// Input gradients of one (chunk, head) from its incoming state S0 and its
// outgoing state gradient dS.  Eight waves; C x n outputs are 16x16 tiles
// (row tile rt, column tile).  The products with the states give a wave one
// column tile and both row tiles (each state row or column is then read
// once); the others deal the tiles round-robin to the waves.
template <int DK, bool KDA, typename IT, typename GT>
__global__ __launch_bounds__(kGradThreads) void bwd_grad_kernel(BwdKArgs p, long nitems) {
    constexpr int C = kBC, NT = kGradThreads, NW = NT / 64, PK = DK + 4, PV = 128 + 4, PB = PK > PV ? PK : PV;
    constexpr int UV = div_up(2 * 128 / 16, NW);   // C x d_v tiles per wave (max)
    static_assert(NW >= 8 && NW % 2 == 0, "the C x C phases deal tiles to waves 0-7");
    using R = BRec<DK>;
    // K e^g, then K e^{g-m}       | raw K, then K e^{m-g}      | g, then dg (per channel)
    // (16-byte aligned: the A B^T products read four floats at a time)
    __shared__ __align__(16) float sX1[C][PK], sX2[C][PK], sGg[KDA ? C : 1][PK];
    // V -> Y, then Q e^{g-m}      | U                          | dU -> dY      | scale dO
    __shared__ __align__(16) float sB1[C][PB], sB2[C][PV], sB3[C][PV], sB4[C][PV];
    __shared__ float sT[C][C + 1], sM[C][C + 1], sdT[C][C + 1], sdA[C][C + 1], sdM[C][C + 1], sE1[C][C + 1];
    __shared__ float sb[C], sg[C], sm[DK], sgl[DK], sdgc[DK], sdb[C];
    __shared__ float sPb[8][C], sPb2[2][C];   // d beta partials (per value tile / column tile)
    __shared__ float sPc[2][DK];              // column partials of gK3 o K
    __shared__ float sPr[DK / 16][C];         // row partials of dg (per-head decay)
    const int H = p.H, DV = p.dv;
    const IT *q = static_cast<const IT *>(p.q), *k = static_cast<const IT *>(p.k), *v = static_cast<const IT *>(p.v);
    const int ntv = 2 * (DV / 16);

    // Persistent workgroups: items (chunk slot rc, head h), item = rc H + h,
    // blockIdx.x, + gridDim.x, ...  While one item's phases run, the next
    // item's inputs and its S0 rows for Y are already in flight into
    // registers (and, once Y has used those registers, the item's own dS
    // rows for K_end dS^T): the LDS holds one workgroup per CU, so without
    // this a CU's loads and its products would take turns.  (Barriers wait
    // only for LDS operations, so those loads stay in flight across them.)
    constexpr int NKL = div_up(C * DK / 4, NT), NVL = div_up(C * 128 / 4, NT), NTL = C * C / NT;
    constexpr int NSB = DK / 32;                   // 32-wide k blocks of a state row
    static_assert(NTL >= 1 && C * C % NT == 0, "load tiling");
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 kv[NKL], qv[NKL], gv[NKL], vv[NVL], dd[NVL];
    float tv[NTL], mv[NTL], bb = 0.f, gg = 0.f;
    // wave w's rows 16 w + lr of S0, k = 32 blk + 16 hh + 4 lq .. + 3: the B
    // operand of its Y product
    f32x4 s0r[NSB][2];
    auto item_loc = [&](long it) {
        ChunkLoc L;
        L.n = 0, L.tok0 = 0, L.len = 0;
        if (it < nitems) L = locate(p, it / H);
        return L;
    };
    auto fetch_inputs = [&](long it, const ChunkLoc &L) {
        const int tid = threadIdx.x;
        const long rc = it / H;
        const int h = (int)(it % H), hq = h / p.G;
        const float *rec = p.rec + (rc * H + h) * p.rec_stride;
#pragma unroll
        for (int u = 0; u < NKL; ++u) {
            const int e = min(tid + NT * u, C * DK / 4 - 1), r = e / (DK / 4), j = (e % (DK / 4)) * 4;
            const long t = L.tok0 + min(r, L.len - 1);
            kv[u] = load4_once(k + (t * p.Hk + hq) * DK + j);
            qv[u] = load4_once(q + (t * p.Hk + hq) * DK + j);
            gv[u] = KDA ? load4_once(static_cast<const GT *>(p.log_alpha) + (t * H + h) * DK + j) : z4;
        }
#pragma unroll
        for (int u = 0; u < NVL; ++u) {
            const int e = min(tid + NT * u, C * DV / 4 - 1), r = e / (DV / 4), i = (e % (DV / 4)) * 4;
            const long o = ((L.tok0 + min(r, L.len - 1)) * H + h) * DV + i;
            vv[u] = load4_once(v + o);
            dd[u] = load4_once(p.d_out + o);
        }
#pragma unroll
        for (int u = 0; u < NTL; ++u) {
            tv[u] = ld1_once(rec + R::T + tid + NT * u);
            mv[u] = ld1_once(rec + R::M + tid + NT * u);
        }
        const long obg = (L.tok0 + min(tid & (C - 1), L.len - 1)) * H + h;
        bb = gate1<GT>(p.beta, obg);
        gg = KDA ? 0.f : gate1<GT>(p.log_alpha, obg);
    };
    auto fetch_rows = [&](const float *base, f32x4 (&r)[NSB][2]) {
        const int w = threadIdx.x >> 6, lr = threadIdx.x & 15, lq = (threadIdx.x >> 4) & 3;
        if (w >= DV / 16) return;
        const __amdgpu_buffer_rsrc_t rs = buffer_of(base, (long)DV * DK);
#pragma unroll
        for (int blk = 0; blk < NSB; ++blk)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) r[blk][hh] = bload4(rs, ((16 * w + lr) * DK + 4 * lq) * 4, (32 * blk + 16 * hh) * 4);
    };
    auto states_of = [&](long it) { return p.states + it * (long)DV * DK; };    // item = rc H + h
    auto dstates_of = [&](long it) { return p.dstates + it * (long)DV * DK; };
    (void)dstates_of;

    long item = blockIdx.x;
    ChunkLoc L = item_loc(item);
    if (L.len > 0) {
        fetch_inputs(item, L);
        fetch_rows(states_of(item), s0r);
    }
    // (an empty chunk slot ends the packed batch's slots, so every later item is empty too)
    while (L.len > 0) {
    // The lane index, opaque to the compiler once per item: the per-lane LDS
    // addresses of the phases are then formed where they are used, as in a
    // workgroup that runs one item, instead of being hoisted out of the loop
    // and held in registers across it.
    int opaque_zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(opaque_zero));
    const int tid = ((int)threadIdx.x + opaque_zero) & (NT - 1);   // (the mask keeps tid's range known)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, lr = l & 15, lq = l >> 4;
    const bool has_v = w < DV / 16;
    const long rc = item / H;
    const int h = (int)(item % H);
    const float *rec = p.rec + (rc * H + h) * p.rec_stride;
    const float *S0 = states_of(item);
    const float *dS = dstates_of(item);
    const __amdgpu_buffer_rsrc_t rS0 = buffer_of(S0, (long)DV * DK), rdS = buffer_of(dS, (long)DV * DK);
    const long nxt = item + gridDim.x;
    const ChunkLoc Ln = item_loc(nxt);
    const bool more = Ln.len > 0;

    // ---- the item's inputs from registers into LDS
#pragma unroll
    for (int u = 0; u < NKL; ++u) {
        const int e = tid + NT * u;
        if (e >= C * DK / 4) continue;
        const int r = e / (DK / 4), j = (e % (DK / 4)) * 4;
        const float4 kk4 = r < L.len ? kv[u] : z4, gg4 = r < L.len ? gv[u] : z4;
        sX2[r][j] = kk4.x, sX2[r][j + 1] = kk4.y, sX2[r][j + 2] = kk4.z, sX2[r][j + 3] = kk4.w;
        if (KDA) sGg[r][j] = gg4.x, sGg[r][j + 1] = gg4.y, sGg[r][j + 2] = gg4.z, sGg[r][j + 3] = gg4.w;
    }
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
        const int e = tid + NT * u;
        if (e >= C * DV / 4) continue;
        const int r = e / (DV / 4), i = (e % (DV / 4)) * 4;
        const float4 v4 = r < L.len ? vv[u] : z4, d4 = r < L.len ? dd[u] : z4;
        sB1[r][i] = v4.x, sB1[r][i + 1] = v4.y, sB1[r][i + 2] = v4.z, sB1[r][i + 3] = v4.w;
        sB4[r][i] = p.scale * d4.x, sB4[r][i + 1] = p.scale * d4.y;
        sB4[r][i + 2] = p.scale * d4.z, sB4[r][i + 3] = p.scale * d4.w;
    }
#pragma unroll
    for (int u = 0; u < NTL; ++u) {
        const int e = tid + NT * u;
        sT[e / C][e % C] = tv[u];
        sM[e / C][e % C] = mv[u];
    }
    if (tid < C) {
        sb[tid] = tid < L.len ? bb : 0.f;
        if (!KDA) sg[tid] = tid < L.len ? gg : 0.f;
    }
    // q stays in registers for the last phases (raw q from its LDS copy there)
    float4 qkeep[NKL];
#pragma unroll
    for (int u = 0; u < NKL; ++u) qkeep[u] = qv[u];
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (more) fetch_inputs(nxt, Ln);
    // inclusive cumulative sums of the log decay over the chunk's rows
    if (KDA) {
        // four adjacent lanes per channel, eight rows each
        for (int e = tid; e < 4 * DK; e += NT) {
            const int j = e >> 2, qd = e & 3;
            float v[C / 4];
            const float tot = seg_scan4(sGg, qd, j, v, false);
            float before, total;
            scan4_offsets(tot, qd, false, before, total);
#pragma unroll
            for (int rr = 0; rr < C / 4; ++rr) sGg[qd * (C / 4) + rr][j] = before + v[rr];
            if (qd == 0) {
                sm[j] = 0.5f * (v[0] + total);
                sgl[j] = total;
            }
        }
    } else if (w == 0) {
        float g = l < C ? sg[l] : 0.f;
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
            const float t = __shfl_up(g, o, 32);
            if ((l & 31) >= o) g += t;
        }
        const float first = __shfl(g, 0), total = __shfl(g, C - 1);
        if (l < C) sg[l] = g;
        if (l == 0) {
            sm[0] = 0.5f * (first + total);
            sgl[0] = total;
        }
    }
    lds_barrier();
    auto gval = [&](int r, int j) { return KDA ? sGg[r][j] : sg[r]; };
    auto mval = [&](int j) { return KDA ? sm[j] : sm[0]; };
    auto glast = [&](int j) { return KDA ? sgl[j] : sgl[0]; };
    for (int e = tid; e < C * DK; e += NT) {
        const int r = e / DK, j = e % DK;
        sX1[r][j] = sX2[r][j] * fexp(gval(r, j));
    }
    lds_barrier();

    // Phases over C x d_v tiles: wave w takes value tile w (16 value rows)
    // and both row tiles, so each state row is read from memory once.
    const int nvt = DV / 16;
    // ---- Y = V - (K e^g) S0^T
    if (has_v) {
        f32x4 acc[2] = {zero4(), zero4()};
        tile_mma_nt<DK, 2>(acc, DK, [&](int q, int mi, int kb, int lk) { return lds4(&sX1[16 * q + mi][kb + lk]); },
                           [&](int, int, int kb, int) { return s0r[kb >> 5][(kb >> 4) & 1]; });
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) sB1[16 * q + 4 * lq + i][16 * w + lr] -= acc[q][i];
    }
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // the same registers now take this item's dS rows, for K_end dS^T below
    fetch_rows(dS, s0r);
    // ---- U = T diag(b) Y;  dU = M^T dO' (then + K_end dS^T below);
    //      K_end = K e^{g_C - g} built in place of K e^g (no longer read)
    f32x4 u[2] = {zero4(), zero4()}, du[2] = {zero4(), zero4()};
    if (has_v) {
        tile_mma_n<C, 2>(u, C, [&](int q, int mi, int kb, int lk) { return sT[16 * q + mi][kb + lk]; },
                         [&](int, int kb, int lk, int ni) { return sb[kb + lk] * sB1[kb + lk][16 * w + ni]; });
        tile_mma_n<C, 2>(du, C, [&](int q, int mi, int kb, int lk) { return sM[kb + lk][16 * q + mi]; },
                         [&](int, int kb, int lk, int ni) { return sB4[kb + lk][16 * w + ni]; });
    }
    for (int e = tid; e < C * DK; e += NT) {
        const int r = e / DK, j = e % DK;
        sX1[r][j] = sX2[r][j] * fexp(glast(j) - gval(r, j));
    }
    lds_barrier();
    if (has_v) {
        tile_mma_nt<DK, 2>(du, DK, [&](int q, int mi, int kb, int lk) { return lds4(&sX1[16 * q + mi][kb + lk]); },
                           [&](int, int, int kb, int) { return s0r[kb >> 5][(kb >> 4) & 1]; });
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * q + 4 * lq + i;
                sB2[r][16 * w + lr] = u[q][i];
                sB3[r][16 * w + lr] = du[q][i];
            }
    }
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (more) fetch_rows(states_of(nxt), s0r);
    // ---- dT = dU (diag(b) Y)^T;  Z = T^T dU (kept in registers);  d beta (value part)
    if (w < 4) {
        const int rt = w & 1, ct = w >> 1;
        f32x4 t1[1] = {zero4()};
        tile_mma_nt<128, 1>(t1, DV, [&](int, int mi, int kb, int lk) { return lds4(&sB3[16 * rt + mi][kb + lk]); },
                            [&](int, int ni, int kb, int lk) { return sb[16 * ct + ni] * lds4(&sB1[16 * ct + ni][kb + lk]); });
        const f32x4 a = t1[0];
#pragma unroll
        for (int i = 0; i < 4; ++i) sdT[16 * rt + 4 * lq + i][16 * ct + lr] = a[i];
    }
    f32x4 z[UV];
#pragma unroll
    for (int u = 0; u < UV; ++u) {
        const int t = w + NW * u;
        z[u] = zero4();
        if (t < ntv) {
            const int rt = t & 1, it = t >> 1;
            z[u] = tile_mma<C>(zero4(), C, [&](int mi, int kk) { return sT[kk][16 * rt + mi]; },
                            [&](int kk, int ni) { return sB3[kk][16 * it + ni]; });
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rt + 4 * lq + i;
                const float s = group_sum<16>(z[u][i] * sB1[r][16 * it + lr]);
                if (lr == 0) sPb[it][r] = s;
            }
        }
    }
    lds_barrier();
    // ---- dV = dY = diag(b) Z (written out and kept in place of dU);
    //      E1 = dT T^T;  shifted operands;  Q e^{g-m} in place of Y
#pragma unroll
    for (int u = 0; u < UV; ++u) {
        const int t = w + NW * u;
        if (t < ntv) {
            const int rt = t & 1, it = t >> 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rt + 4 * lq + i, c = 16 * it + lr;
                const float dy = sb[r] * z[u][i];
                sB3[r][c] = dy;
                if (r < L.len) p.dv_out[((L.tok0 + r) * H + h) * DV + c] = dy;
            }
        }
    }
    if (w < 4) {
        const int rt = w & 1, ct = w >> 1;
        const f32x4 a = tile_mma<C>(zero4(), C, [&](int mi, int kk) { return sdT[16 * rt + mi][kk]; },
                                 [&](int kk, int ni) { return sT[16 * ct + ni][kk]; });
#pragma unroll
        for (int i = 0; i < 4; ++i) sE1[16 * rt + 4 * lq + i][16 * ct + lr] = a[i];
    }
    for (int e = tid; e < C * DK; e += NT) {
        const int r = e / DK, j = e % DK;
        const float kk = sX2[r][j], g = gval(r, j), m = mval(j);
        sX1[r][j] = kk * fexp(g - m);
        sX2[r][j] = kk * fexp(m - g);
    }
#pragma unroll
    for (int u = 0; u < NKL; ++u) {               // q as loaded at the start
        const int e = tid + NT * u;
        if (e >= C * DK / 4) continue;
        const int r = e / (DK / 4), j = (e % (DK / 4)) * 4;
        const float4 q4 = r < L.len ? qkeep[u] : z4;
        sB1[r][j] = q4.x * fexp(gval(r, j) - mval(j));
        sB1[r][j + 1] = q4.y * fexp(gval(r, j + 1) - mval(j + 1));
        sB1[r][j + 2] = q4.z * fexp(gval(r, j + 2) - mval(j + 2));
        sB1[r][j + 3] = q4.w * fexp(gval(r, j + 3) - mval(j + 3));
    }
    if (tid < C) {
        float s = 0.f;
        for (int it = 0; it < DV / 16; ++it) s += sPb[it][tid];
        sdb[tid] = s;
    }
    lds_barrier();
    // ---- dA = strict_tril(-T^T E1), d beta (Gram part), diag(b) dA;  dM = tril(dO' U^T)
    if (w < 4) {
        const int rt = w & 1, ct = w >> 1;
        const f32x4 a = tile_mma<C>(zero4(), C, [&](int mi, int kk) { return sT[kk][16 * rt + mi]; },
                                 [&](int kk, int ni) { return sE1[kk][16 * ct + ni]; });
        f32x4 g1[1] = {zero4()};
        tile_mma_nt<DK, 1>(g1, DK, [&](int, int mi, int kb, int lk) { return lds4(&sX1[16 * rt + mi][kb + lk]); },
                           [&](int, int ni, int kb, int lk) { return lds4(&sX2[16 * ct + ni][kb + lk]); });
        const f32x4 gm = g1[0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * lq + i, c = 16 * ct + lr;
            // the Gram's upper triangle (i > r) carries e^{g_r - g_i} >= 1 and may
            // overflow; only the strictly lower part enters
            const float d = c < r ? -a[i] : 0.f;
            const float s = group_sum<16>(c < r ? d * gm[i] : 0.f);
            if (lr == 0) sPb2[ct][r] = s;
            sdA[r][c] = sb[r] * d;
        }
    } else if (w < 8) {
        const int rt = (w - 4) & 1, ct = (w - 4) >> 1;
        f32x4 m1[1] = {zero4()};
        tile_mma_nt<128, 1>(m1, DV, [&](int, int mi, int kb, int lk) { return lds4(&sB4[16 * rt + mi][kb + lk]); },
                            [&](int, int ni, int kb, int lk) { return lds4(&sB2[16 * ct + ni][kb + lk]); });
        const f32x4 a = m1[0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * rt + 4 * lq + i, c = 16 * ct + lr;
            sdM[r][c] = c <= r ? a[i] : 0.f;
        }
    }
    lds_barrier();
    // ---- dO' (sB4), dY (sB3) and U (sB2) as split bf16 operands, in place:
    //      each row's 528 bytes become [hi of its 128 values | lo | unused],
    //      the value index permuted within blocks of 32 (kperm32).  One wave
    //      converts a whole row (one read, then the writes), so no other wave
    //      touches a row while it changes form.
    static_assert(PV * 4 >= 2 * 128 * 2, "a row holds its split form");
    {
        // (all of the wave's row reads are issued before the first write, so
        // their LDS latencies overlap; a row is written only by the wave
        // that read it, after its read)
        static_assert(3 * C % NW == 0, "rows per wave");
        constexpr int NRR = 3 * C / NW;
        auto row_of = [&](int rr) { return rr < C ? sB4[rr] : rr < 2 * C ? sB3[rr - C] : sB2[rr - 2 * C]; };
        float2 xs[NRR];
#pragma unroll
        for (int i = 0; i < NRR; ++i) xs[i] = *reinterpret_cast<const float2 *>(row_of(w + NW * i) + 2 * l);
        const int pos = (2 * l & ~31) + kperm32(2 * l);
#pragma unroll
        for (int i = 0; i < NRR; ++i) {
            unsigned hu, lu;
            split2(xs[i].x, xs[i].y, hu, lu);
            __bf16 *rb = reinterpret_cast<__bf16 *>(row_of(w + NW * i));
            *reinterpret_cast<unsigned *>(rb + pos) = hu;
            *reinterpret_cast<unsigned *>(rb + 128 + pos) = lu;
        }
    }
    lds_barrier();
    auto plane = [&](float (*buf)[PV], int r) { return reinterpret_cast<const __bf16 *>(buf[r]); };

    // ---- per (row, key channel): dq, dk and the log-decay gradient dg.
    //      Wave w takes key tile w and both row tiles, so each state column is
    //      read once; the same values give the column sums of dS o S0 (the
    //      decay's share of the outgoing gradient).
    if (w < DK / 16) {
        const int jt = w, j = 16 * jt + lr;
        // the three products with the states, dO' S0, dY S0 and U dS, as
        // split bf16 products over blocks of 32 value rows; lane group lq
        // takes rows i = kb + 4 lq + t and kb + 16 + 4 lq + t (t < 4).  The
        // states' rows run along j, so a lane's rows come from eight loads
        // per state, fetched one block ahead.
        f32x4 st[2][3];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int q = 0; q < 3; ++q) st[rt][q] = zero4();
        float cs = 0.f;
        f32x4 sa[2][2], sd[2][2];   // [buffer][half]: S0 and dS values of one block
        auto gather = [&](int kb, int buf) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int lane_bytes = ((4 * lq + t) * DK + j) * 4, ub = (kb + 16 * hf) * DK * 4;
                    sa[buf][hf][t] = bload_last(rS0, lane_bytes, ub);
                    sd[buf][hf][t] = bload_last(rdS, lane_bytes, ub);
                }
        };
        gather(0, 0);
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const int kb = 32 * blk, buf = blk & 1;
            if (kb < DV) {                      // DV (a multiple of 32) is wave-uniform
                if (blk + 1 < 4 && kb + 32 < DV) gather(kb + 32, buf ^ 1);
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int t = 0; t < 4; ++t) cs += sa[buf][hf][t] * sd[buf][hf][t];
                bf16x8 s0h, s0l, dsh, dsl;
                split8(sa[buf][0], sa[buf][1], s0h, s0l);
                split8(sd[buf][0], sd[buf][1], dsh, dsl);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const int r = 16 * rt + lr, c = kb + 8 * lq;
                    const __bf16 *a0 = plane(sB4, r), *a1 = plane(sB3, r), *a2 = plane(sB2, r);
                    st[rt][0] = mfma_split(lds8(a0 + c), lds8(a0 + 128 + c), s0h, s0l, st[rt][0]);
                    st[rt][1] = mfma_split(lds8(a1 + c), lds8(a1 + 128 + c), s0h, s0l, st[rt][1]);
                    st[rt][2] = mfma_split(lds8(a2 + c), lds8(a2 + 128 + c), dsh, dsl, st[rt][2]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        cs += __shfl_xor(cs, 16);
        cs += __shfl_xor(cs, 32);
        if (lq == 0) sdgc[j] = cs * rec[R::D + j];
#pragma unroll 1
        for (int rt = 0; rt < 2; ++rt) {
            // the chunk-local products: dM Khs, dA Khs, dM^T Qts + dA^T Kts
            f32x4 gm[4] = {zero4(), zero4(), zero4(), zero4()};
            tile_mma_n<C, 4>(gm, C, [&](int q, int mi, int kb, int lk) {
                                 const int kk = kb + lk;
                                 return q == 0 ? sdM[16 * rt + mi][kk] : q == 1 ? sdA[16 * rt + mi][kk]
                                      : q == 2 ? sdM[kk][16 * rt + mi] : sdA[kk][16 * rt + mi];
                             },
                             [&](int q, int kb, int lk, int ni) {
                                 const int kk = kb + lk;
                                 return q < 2 ? sX2[kk][16 * jt + ni] : q == 2 ? sB1[kk][16 * jt + ni] : sX1[kk][16 * jt + ni];
                             });
            const f32x4 dq0 = rt ? st[1][0] : st[0][0], dy0 = rt ? st[1][1] : st[0][1], uds = rt ? st[1][2] : st[0][2];
            const f32x4 dmk = gm[0], dak = gm[1];
            f32x4 tq;
#pragma unroll
            for (int i = 0; i < 4; ++i) tq[i] = gm[2][i] + gm[3][i];
            float colk = 0.f;
            float rowg[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rt + 4 * lq + i;
                const float g = gval(r, j), m = mval(j);
                const float eg = fexp(g), egm = fexp(g - m), emg = fexp(m - g), egc = fexp(glast(j) - g);
                const float dQ = dq0[i] * eg + dmk[i] * egm;
                const float gk1 = -dy0[i] * eg + dak[i] * egm;
                const float gk2 = tq[i] * emg;
                const float gk3 = uds[i] * egc;
                const long t = L.tok0 + min(r, L.len - 1), o = (t * H + h) * DK + j;
                // raw k and q from their shifted copies in LDS (zero on padding rows)
                const float kk = sX1[r][j] * emg, qq = sB1[r][j] * emg;
                if (r < L.len) {
                    p.dq[o] = dQ;
                    p.dk[o] = gk1 + gk2 + gk3;
                }
                const float dg = kk * (gk1 - gk2 - gk3) + qq * dQ;
                colk += gk3 * kk;
                if (KDA) sGg[r][j] = dg;
                rowg[i] = dg;
            }
            colk += __shfl_xor(colk, 16);
            colk += __shfl_xor(colk, 32);
            if (lq == 0) sPc[rt][j] = colk;
            if (!KDA) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float s = group_sum<16>(rowg[i]);
                    if (lr == 0) sPr[jt][16 * rt + 4 * lq + i] = s;
                }
            }
        }
    }
    lds_barrier();
    // ---- log-decay gradient: reverse cumulative sum of dg, plus the
    //      chunk-end terms (through e^{g_C}) on every row; d beta
    if (KDA) {
        // four adjacent lanes per channel, eight rows each (suffix sums)
        for (int e = tid; e < 4 * DK; e += NT) {
            const int j = e >> 2, qd = e & 3;
            float v[C / 4];
            const float tot = seg_scan4(sGg, qd, j, v, true);
            float after, total;
            scan4_offsets(tot, qd, true, after, total);
            const float base = sdgc[j] + sPc[0][j] + sPc[1][j] + after;
#pragma unroll
            for (int rr = 0; rr < C / 4; ++rr) {
                const int r = qd * (C / 4) + rr;
                if (r < L.len) p.dla[((L.tok0 + r) * H + h) * DK + j] = base + v[rr];
            }
        }
    } else if (w == 0) {
        // one head-wide decay per row: sum the channel terms, then a suffix
        // scan over the rows (row r on lane r)
        float gc = 0.f;
        for (int j = l; j < DK; j += 64) gc += sdgc[j] + sPc[0][j] + sPc[1][j];
        for (int m = 32; m >= 1; m >>= 1) gc += __shfl_xor(gc, m);
        float d = 0.f;
        if (l < C)
            for (int jt = 0; jt < DK / 16; ++jt) d += sPr[jt][l];
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
            const float t = __shfl_down(d, o, 32);
            if ((l & 31) + o < 32) d += t;
        }
        if (l < L.len) p.dla[(L.tok0 + l) * H + h] = gc + d;
    }
    if (tid < L.len) p.dbeta[(L.tok0 + tid) * H + h] = sdb[tid] + sPb2[0][tid] + sPb2[1][tid];
    lds_barrier();   // the next item's inputs overwrite this one's LDS
    item = nxt;
    L = Ln;
    }
}

// ---------------------------------------------------------------------------
// Grouped q/k heads: the gradient of a q/k head is the sum of those of the G
// value heads that read it (value head h reads q/k head h / G).
__global__ __launch_bounds__(256) void bwd_group_sum_kernel(const float *__restrict__ dqv,
                                                            const float *__restrict__ dkv, float *__restrict__ dq,
                                                            float *__restrict__ dk, long n4, int G, int dk4) {
    const long e = (long)blockIdx.x * 256 + threadIdx.x;   // one float4 of [tokens, Hk, dk]
    if (e >= n4) return;
    const long row = e / dk4, c = e % dk4;                  // row = token * Hk + hk
    f32x4 sq = zero4(), sk = zero4();
    for (int g = 0; g < G; ++g) {
        const long src = (row * G + g) * dk4 + c;
        const f32x4 a = reinterpret_cast<const f32x4 *>(dqv)[src], b = reinterpret_cast<const f32x4 *>(dkv)[src];
#pragma unroll
        for (int i = 0; i < 4; ++i) sq[i] += a[i], sk[i] += b[i];
    }
    reinterpret_cast<f32x4 *>(dq)[e] = sq;
    reinterpret_cast<f32x4 *>(dk)[e] = sk;
}

template <int DK, bool KDA, typename IT, typename GT>
static hipError_t run_backward(const BackwardArgs &a, const BwdKArgs &kp0, hipStream_t st) {
    const long nrc = a.record_chunks;
    // A scan workgroup fills a CU's LDS, so the grid runs in rounds of one
    // workgroup per CU, each round one full chain.  Two waves (32 value rows)
    // per workgroup when both passes then fit in one round, else four.
    const long units = (long)a.num_seqs * a.num_heads;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const bool four = a.dv % 64 == 0 && 2 * 8 * ((units + 7) / 8) * (a.dv / 32) > cus;
    BwdKArgs base = kp0;
    base.raw_qk = !KDA && four;                 // the four-wave scan stages q, k raw with a per-head decay
    const long per_unit = a.dv / (four ? 64 : 32);
    const unsigned scan_blocks = (unsigned)(8 * ((units + 7) / 8) * per_unit);
    // records of chunk slots [0, nrc): prep; then the two state passes
    // (forward: grid [0, half); backward: [half, 2 half)); then the gradients
    auto prep = [&](const BwdKArgs &kp, long nrc_) -> hipError_t {
        if (nrc_ <= 0) return hipSuccess;
        hipLaunchKernelGGL((bwd_prep_kernel<DK, KDA, IT, GT>), dim3((unsigned)nrc_, (unsigned)a.num_heads), dim3(256), 0, st, kp);
        return hipGetLastError();
    };
    auto scan = [&](const BwdKArgs &kp, bool fwd, bool bwd) -> hipError_t {
        const unsigned grid = (fwd ? scan_blocks : 0) + (bwd ? scan_blocks : 0);
        const int half = fwd ? (int)scan_blocks : 0;
        if (four)
            hipLaunchKernelGGL((bwd_scan_kernel<DK, 4, KDA, IT, GT>), dim3(grid), dim3(64 * scan_block_waves(4)), 0, st,
                               kp, half);
        else
            hipLaunchKernelGGL((bwd_scan_kernel<DK, 2, KDA, IT, GT>), dim3(grid), dim3(64 * scan_block_waves(2)), 0, st,
                               kp, half);
        return hipGetLastError();
    };
    auto grad = [&](const BwdKArgs &kp, long nrc_) -> hipError_t {
        if (nrc_ <= 0) return hipSuccess;
        // one grad workgroup fills a CU's LDS: one persistent workgroup per CU
        const long nitems = nrc_ * a.num_heads;
        const unsigned ggrid = (unsigned)std::min<long>(nitems, cus);
        hipLaunchKernelGGL((bwd_grad_kernel<DK, KDA, IT, GT>), dim3(ggrid), dim3(kGradThreads), 0, st, kp, nitems);
        return hipGetLastError();
    };
    hipError_t e = hipSuccess;
    if (a.num_segments <= 1) {
        if ((e = prep(base, nrc)) != hipSuccess || (e = scan(base, true, true)) != hipSuccess ||
            (e = grad(base, nrc)) != hipSuccess)
            return hipErrorLaunchFailure;
    } else {
        // Dense batch in time segments of S chunks: a forward pass over the
        // segments keeps only the state entering each segment; then, last
        // segment first, each segment's records and per-chunk states are
        // rebuilt from that state, its state gradients run backward from the
        // one carried out of the segment after it, and its gradients follow.
        // The chunks see the same arithmetic as in one pass, so the results
        // are the same bit for bit.
        const long nct = div_up(a.seqlen, kBC), S = a.segment_chunks;
        const int NS = a.num_segments;
        const size_t SZ = (size_t)a.num_seqs * a.num_heads * a.dv * DK;   // floats of one set of states
        auto seg = [&](int sgi) {
            BwdKArgs kp = base;
            kp.seg_c0 = (int)(sgi * S);
            kp.seg_nc = (int)std::min<long>(S, nct - sgi * S);
            kp.initial_state = sgi == 0 ? a.initial_state : a.boundary_states + (size_t)(sgi - 1) * SZ;
            return kp;
        };
        for (int sgi = 0; sgi + 1 < NS; ++sgi) {
            BwdKArgs kp = seg(sgi);
            kp.fwd_final = a.boundary_states + (size_t)sgi * SZ;
            kp.no_dump = 1;
            if ((e = prep(kp, (long)a.batch * kp.seg_nc)) != hipSuccess || (e = scan(kp, true, false)) != hipSuccess)
                return hipErrorLaunchFailure;
        }
        for (int sgi = NS - 1; sgi >= 0; --sgi) {
            BwdKArgs kp = seg(sgi);
            kp.d_final = sgi == NS - 1 ? a.d_final_state : a.carry + (size_t)((sgi + 1) & 1) * SZ;
            kp.d_init = sgi == 0 ? a.d_initial_state : a.carry + (size_t)(sgi & 1) * SZ;
            const long nrc_s = (long)a.batch * kp.seg_nc;
            if ((e = prep(kp, nrc_s)) != hipSuccess || (e = scan(kp, true, true)) != hipSuccess ||
                (e = grad(kp, nrc_s)) != hipSuccess)
                return hipErrorLaunchFailure;
        }
    }
    if (nrc > 0 && base.G > 1) {
        const long n4 = (long)a.batch * a.seqlen * base.Hk * (DK / 4);
        hipLaunchKernelGGL(bwd_group_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, base.dq, base.dk,
                           a.dq, a.dk_out, n4, base.G, DK / 4);
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    return hipSuccess;
}

template <int DK>
static hipError_t dispatch_dk(const BackwardArgs &a, const BwdKArgs &kp, hipStream_t st) {
    if (a.gate_bf16) {
        if (a.bf16)
            return a.kda ? run_backward<DK, true, __bf16, __bf16>(a, kp, st) : run_backward<DK, false, __bf16, __bf16>(a, kp, st);
        return a.kda ? run_backward<DK, true, float, __bf16>(a, kp, st) : run_backward<DK, false, float, __bf16>(a, kp, st);
    }
    if (a.bf16)
        return a.kda ? run_backward<DK, true, __bf16, float>(a, kp, st) : run_backward<DK, false, __bf16, float>(a, kp, st);
    return a.kda ? run_backward<DK, true, float, float>(a, kp, st) : run_backward<DK, false, float, float>(a, kp, st);
}

bool backward_supported(int dk, int dv) {
    return (dk == 32 || dk == 64 || dk == 128) && dv >= 32 && dv <= 128 && dv % 32 == 0;
}

hipError_t launch_backward(const BackwardArgs &a, hipStream_t st) {
    if (a.num_seqs == 0 || a.num_heads == 0) return hipSuccess;
    if (a.cu_seqlens) {
        const hipError_t e = launch_schedule(a.cu_seqlens, a.num_seqs, kBC, a.order, a.chunk_offset, st);
        if (e != hipSuccess) return e;
    }
    BwdKArgs kp;
    kp.batch = a.batch, kp.seqlen = a.seqlen, kp.H = a.num_heads, kp.dv = a.dv, kp.num_seqs = a.num_seqs;
    kp.q = a.q, kp.k = a.k, kp.v = a.v, kp.beta = a.beta, kp.log_alpha = a.log_alpha;
    kp.initial_state = a.initial_state;
    kp.cu = a.cu_seqlens, kp.order = a.order, kp.choff = a.chunk_offset;
    kp.scale = a.scale, kp.d_out = a.d_out, kp.d_final = a.d_final_state;
    kp.Hk = a.num_qk_heads, kp.G = a.num_heads / a.num_qk_heads;
    // per-value-head q/k gradients go straight to dq, dk, or (grouped heads)
    // to the workspace, summed over each group afterwards
    kp.dq = kp.G > 1 ? a.dq_heads : a.dq;
    kp.dk = kp.G > 1 ? a.dk_heads : a.dk_out;
    kp.dv_out = a.dv_out, kp.dbeta = a.dbeta, kp.dla = a.dlog_alpha;
    kp.d_init = a.d_initial_state;
    kp.rec = a.records, kp.states = a.states, kp.dstates = a.dstates;
    kp.rec_stride = (long)(backward_record_bytes(a.dk) / sizeof(float));
    kp.raw_qk = 0;
    kp.seg_c0 = 0, kp.seg_nc = 0, kp.fwd_final = nullptr, kp.no_dump = 0;
    switch (a.dk) {
        case 32: return dispatch_dk<32>(a, kp, st);
        case 64: return dispatch_dk<64>(a, kp, st);
        case 128: return dispatch_dk<128>(a, kp, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdr
