// prefill_impl.h -- chunked prefill of the gated delta rule for gfx950.
//
// The recurrence (page "How the New Flash Models Work: Inside GLM-5.3-Flash
// and Qwen3.8-Flash-Next", section "Linear attention: a fixed-size memory in
// place of the cache"):  S_t = S_{t-1} Diag(a_t)(I - b_t k_t k_t^T) + b_t v_t k_t^T,
// o_t = S_t q_t, with a scalar decay per head (Gated DeltaNet) or one per key
// channel (Kimi Delta Attention).
//
// Chunked form (algebra derived from that equation; the pages give no
// algorithm).  For a chunk of C tokens entering with state S0 and the
// inclusive in-chunk cumulative log-decay g_r (per key channel),
//     A   = strict_tril(diag(b) (K e^g)(K e^-g)^T)           Gram with decay
//     T   = (I + A)^-1                                        UT transform
//     X   = (K e^g) S0^T,   W = diag(b)(V - X),   U = T W
//     O   = (Q e^g) S0^T + M U,   M = tril((Q e^g)(K e^-g)^T)
//     S_C = S0 Diag(e^{g_C}) + U^T (K e^{g_C - g}).
//
// Work split.  One workgroup owns a slice of DVS value channels of one
// (sequence, head): rows of S evolve independently, so slices never talk.
// Inside the workgroup, four "prologue" waves build everything a chunk needs
// that does not depend on the state (gate prefix sums, decayed operands,
// Gram matrices, T), one chunk ahead, into a double buffer; one "chain" wave
// per 16 value channels walks the chunks in order, holding its part of the
// state transposed (S^T: key rows x value columns) as fp32 MFMA accumulators.
// In that layout the state, W and U feed the next product straight from
// registers (each lane's accumulator rows are exactly the k-indices its
// MFMA operand fragment needs), so the sequential chain X -> W -> U -> (O, S)
// touches LDS only to read the prologue's shared operands.  Global inputs of
// chunk j+1 are prefetched into registers while chunk j is built.
//
// Precision (bf16 q/k/v).  Outputs reach ~15x their RMS, so an error bound of
// 2e-2 x RMS on the largest element needs ~1e-3 relative accuracy on the
// terms that carry v; one bf16 rounding (2^-8) of those terms is too coarse.
// The products run on fp16 MFMA (11-bit operands) with the value-carrying
// operands W and U split into an fp16 hi + lo pair (two MFMAs each), and the
// per-channel-decay Gram M from bf16 hi + lo pairs (three MFMAs: hi.hi +
// hi.lo + lo.hi).  The Gram A that feeds T keeps single bf16 operands: the
// delta rule's erase step corrects what an error in T leaves behind.  fp32
// q/k/v use fp32 MFMA throughout.
//
// Exponent range.  Gated DeltaNet: the decay is a per-row scalar; raw k/q
// (exact in fp16) feed the products and e^{g_r - g_i} <= 1 scales the fp32
// results.  Kimi Delta Attention: the decay sits inside the key-channel sum,
// so the Gram operands carry it around a per-channel reference
// m = (g_first + g_last)/2: k e^{g-m}, q e^{g-m}, k e^{m-g} stay within
// e^{+-half the chunk's decay} in bf16 (fp32 exponent range).  The state-side
// operands k e^g, q e^g, k e^{g_C-g} are all <= 1 in magnitude.
#pragma once

#include "common.h"
#include "launch.h"

namespace gdr {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

// ---- MFMA traits: 16x16 fp32 tile, K advanced KSTEP per instruction -------
// Lane l holds row (l & 15) of each 16-row operand and KPL consecutive
// k-values from (l >> 4) * KPL; A and B share that k-assignment, so the
// k-order inside one instruction is irrelevant.  The result gives lane l
// rows 4*(l>>4)+i (i < 4) of column l&15.
template <typename OT> struct Mfma;
template <> struct Mfma<__bf16> {
    static constexpr int KSTEP = 32, KPL = 8;
    using frag = bf16x8;
    __device__ static __forceinline__ frag load(const __bf16 *p) { return *reinterpret_cast<const frag *>(p); }
    __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<_Float16> {
    static constexpr int KSTEP = 32, KPL = 8;
    using frag = f16x8;
    __device__ static __forceinline__ frag load(const _Float16 *p) { return *reinterpret_cast<const frag *>(p); }
    __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    static constexpr int KSTEP = 4, KPL = 1;
    using frag = float;
    __device__ static __forceinline__ frag load(const float *p) { return *p; }
    __device__ static __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// acc += A[16 rows] * B[16 rows]^T over k in [0, K); both row-major in LDS
// with k contiguous (leading dimensions lda, ldb, in elements).
template <typename OT, int K>
__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, const OT *A, int lda, const OT *B, int ldb, int lane) {
    using M = Mfma<OT>;
    const OT *pa = A + (lane & 15) * lda + (lane >> 4) * M::KPL;
    const OT *pb = B + (lane & 15) * ldb + (lane >> 4) * M::KPL;
#pragma unroll
    for (int k = 0; k < K; k += M::KSTEP) acc = M::mma(M::load(pa + k), M::load(pb + k), acc);
    return acc;
}

// ---- operands held in registers in the accumulator layout ------------------
// A k-dimension of NBLK 16-blocks held as fp32 accumulator tiles v[blk]
// (lane: k-indices 16*blk + 4*lg + i).  As an MFMA B operand it is consumed
// with the A operand read from LDS at the same k-indices.
template <typename ST, int NBLK> struct RegB;
template <int NBLK> struct RegB<_Float16, NBLK> {
    static_assert(NBLK % 2 == 0, "fp16 k-steps span two 16-blocks");
    f16x8 f[NBLK / 2];
    __device__ __forceinline__ void set(const f32x4 *v) {
#pragma unroll
        for (int s = 0; s < NBLK / 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f[s][i] = (_Float16)v[2 * s][i];
                f[s][4 + i] = (_Float16)v[2 * s + 1][i];
            }
    }
    // split v = hi + lo: this object takes hi, `lo` takes the remainder
    __device__ __forceinline__ void set_split(const f32x4 *v, RegB &lo) {
#pragma unroll
        for (int s = 0; s < NBLK / 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const _Float16 h0 = (_Float16)v[2 * s][i], h1 = (_Float16)v[2 * s + 1][i];
                f[s][i] = h0;
                f[s][4 + i] = h1;
                lo.f[s][i] = (_Float16)(v[2 * s][i] - (float)h0);
                lo.f[s][4 + i] = (_Float16)(v[2 * s + 1][i] - (float)h1);
            }
    }
    // acc += A * B, A given as preloaded fragments (RowA) of the same k-range
    template <class RA>
    __device__ __forceinline__ f32x4 mma(f32x4 acc, const RA &a, int nsteps = 1 << 20) const {
#pragma unroll
        for (int s = 0; s < NBLK / 2; ++s)
            if (s < nsteps) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.f[s], f[s], acc, 0, 0, 0);
        return acc;
    }
};

template <int NBLK> struct RegB<float, NBLK> {
    f32x4 f[NBLK];
    __device__ __forceinline__ void set(const f32x4 *v) {
#pragma unroll
        for (int b = 0; b < NBLK; ++b) f[b] = v[b];
    }
    __device__ __forceinline__ void set_split(const f32x4 *v, RegB &lo) {
        set(v);
        (void)lo;
    }
    // nsteps counts 32-wide k-steps (two 16-blocks), as for fp16 operands
    template <class RA>
    __device__ __forceinline__ f32x4 mma(f32x4 acc, const RA &a, int nsteps = 1 << 20) const {
        const int nblk = nsteps < NBLK ? 2 * nsteps : NBLK;
#pragma unroll
        for (int b = 0; b < NBLK; ++b)
            if (b < nblk)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[b][i], f[b][i], acc, 0, 0, 0);
        return acc;
    }
};

// A-operand fragments of one 16-row tile read from LDS at the k-indices a
// RegB of the same NBLK supplies (lane row = lr, k = 16*blk + 4*lg + i).
template <typename ST, int NBLK> struct RowA;
template <int NBLK> struct RowA<_Float16, NBLK> {
    f16x8 f[NBLK / 2];
    __device__ __forceinline__ void load(const _Float16 *arow, int lg, int nsteps = 1 << 20) {
#pragma unroll
        for (int s = 0; s < NBLK / 2; ++s) {
            if (s < nsteps) {
                const f16x4 a0 = *reinterpret_cast<const f16x4 *>(arow + 32 * s + 4 * lg);
                const f16x4 a1 = *reinterpret_cast<const f16x4 *>(arow + 32 * s + 16 + 4 * lg);
                f[s] = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
    }
};
template <int NBLK> struct RowA<float, NBLK> {
    f32x4 f[NBLK];
    __device__ __forceinline__ void load(const float *arow, int lg, int nsteps = 1 << 20) {
        const int nblk = nsteps < NBLK ? 2 * nsteps : NBLK;
#pragma unroll
        for (int b = 0; b < NBLK; ++b)
            if (b < nblk) f[b] = *reinterpret_cast<const f32x4 *>(arow + 16 * b + 4 * lg);
    }
};

// ---- precision policy per input type --------------------------------------
template <typename IT> struct Prec;
template <> struct Prec<__bf16> {
    using ST = _Float16;   // state-side operands
    using GT = __bf16;     // per-channel-decay Gram operands (fp32 exponent range)
    static constexpr bool SPLIT = true;
};
template <> struct Prec<float> {
    using ST = float;
    using GT = float;
    static constexpr bool SPLIT = false;
};

template <typename T, int N> struct VecT { typedef T type __attribute__((ext_vector_type(N))); };

// ---- shared memory ----------------------------------------------------------
template <int DK, int DVS, int C, bool KDA, typename IT>
struct PrefillSmem {
    using ST = typename Prec<IT>::ST;
    using GT = typename Prec<IT>::GT;
    static constexpr bool SPLIT = Prec<IT>::SPLIT;
    static constexpr int PAD = 16 / sizeof(ST);   // 16-byte row padding spreads LDS banks
    static constexpr int LDK = DK + PAD;          // [*][DK] operand rows (ST and GT have equal size)
    static constexpr int LDC = C + PAD;           // [*][C] operand rows
    static constexpr int LDV = DVS + PAD;         // value-slice rows
    static constexpr int LDA = C + 4;             // fp32 [C][C]
    static constexpr int NB = C / 16;
    static constexpr int KG = KDA ? C : 1;
    static constexpr int KGS = (KDA && SPLIT) ? C : 1;

    // per-chunk operands, double-buffered (prologue writes chunk j+1 while
    // the chain reads chunk j)
    struct alignas(16) Buf {
        float dec[KDA ? DK : 4];  // decay over the chunk: e^{g_C} (per key channel for KDA)
        ST Kt[C][LDK];          // GDN: k              KDA: k e^g
        ST Qt[C][LDK];          // GDN: q              KDA: q e^g
        ST KeT[DK][LDC];        // (k e^{g_C - g})^T
        ST Tm[C][LDC];          // T = (I + A)^-1 (zero above the diagonal)
        ST Mm[C][LDC];          // M (zero above the diagonal)
        IT V[C][LDV];           // value slice
        float beta[C];
        float eg[KDA ? 1 : C];  // GDN: e^{g_r}
    } buf[2];
    // prologue scratch
    union alignas(16) {
        float G[KDA ? C : 1][DK];   // KDA: log-decay, then e^{g - m}
        struct {
            float A[C][LDA];        // strict_tril(diag(b) Gram)
            float Tf[C][LDA];       // (I + A)^-1, fp32
        } at;
    } u;
    float P[256];                   // T_10 intermediate (two 16-blocks)
    alignas(16) GT Lk[KG][LDK];     // KDA: k e^{g-m}
    GT Lq[KG][LDK];                 // KDA: q e^{g-m} (hi)
    GT Lql[KGS][LDK];               //                (lo)
    GT Rh[KG][LDK];                 // KDA: k e^{m-g} (hi)
    GT Rl[KGS][LDK];                //                (lo)
    float em[KDA ? DK : 1], egcm[KDA ? DK : 1];   // KDA: e^m, e^{g_C - m}
    float g[KDA ? 1 : C], egc[KDA ? 1 : C];       // GDN: g, e^{g_C - g}
};

struct PrefillKArgs {
    int T, H, DV, num_seqs;
    const void *q, *k, *v;
    const float *beta, *log_alpha, *initial_state;
    const int32_t *cu, *order;
    float scale;
    void *out;
    float *final_state;
    bool out_bf16;
};

template <typename ST>
__device__ __forceinline__ void split2(float x, ST &hi, ST &lo) {
    hi = (ST)x;
    lo = (ST)(x - (float)hi);
}

constexpr int kPrologueWaves = 4;

// Barriers per pipeline iteration.  Per-head decay: (1) inputs to LDS,
// (2) Gram + T + K_end^T, chain alongside.  Per-channel decay: (1) prefix sums
// and e^{g-m}, (2) decayed operands, chain alongside, (3) Gram + T + K_end^T.
template <bool KDA>
constexpr int pipeline_barriers() { return KDA ? 3 : 2; }

template <int DK, int DVS, int C, bool KDA, typename IT>
__global__ __launch_bounds__(64 * (kPrologueWaves + DVS / 16)) void prefill_kernel(PrefillKArgs p) {
    using SM = PrefillSmem<DK, DVS, C, KDA, IT>;
    using Buf = typename SM::Buf;
    using ST = typename SM::ST;
    using GT = typename SM::GT;
    constexpr bool SPLIT = SM::SPLIT;
    constexpr int NPW = kPrologueWaves;
    constexpr int EPV = 16 / sizeof(IT);           // elements per 16-byte input vector
    using IV = typename VecT<IT, EPV>::type;
    using SV = typename VecT<ST, EPV>::type;
    using GV = typename VecT<GT, EPV>::type;
    constexpr int LDK = SM::LDK;
    constexpr int NB = C / 16;                     // 16-token blocks per chunk
    constexpr int NKB = DK / 16;                   // 16-channel key blocks
    constexpr int KV = C * (DK / EPV);             // 16-byte k (or q) vectors per chunk
    constexpr int KVPT = (KV + 255) / 256;
    constexpr int VV = C * (DVS / EPV);            // 16-byte value vectors per chunk
    constexpr int NSEG = 256 / DK;                 // KDA prefix sum: lanes per key channel
    constexpr int SEGL = C / NSEG;                 //   tokens per lane
    constexpr int NBAR = pipeline_barriers<KDA>();
    constexpr int CHAIN_STAGE = 1;                 // barriers the chain waits for before its work
    static_assert(NB <= 2, "the inverse below handles at most two 16-token blocks");
    static_assert(NB * (NB + 1) / 2 <= kPrologueWaves - 1, "one M tile per prologue wave");
    static_assert(sizeof(SM) <= 160 * 1024, "LDS budget");
    static_assert(C % Mfma<ST>::KSTEP == 0 && DK % Mfma<ST>::KSTEP == 0, "tile sizes");
    static_assert(VV <= 256 && C <= 64 && SEGL >= 1, "prologue thread mapping");
    static_assert(sizeof(ST) == sizeof(IT) && sizeof(GT) == sizeof(IT), "operand sizes");

    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index in a scalar register: the chain / prologue split below is a
    // uniform branch, so each wave executes only its own path's barriers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int H = p.H, DV = p.DV;

    // ---- block -> (sequence, head, value slice); the slices of one
    // (sequence, head) share blockIdx % 8, i.e. one XCD and its L2.
    const int NS = DV / DVS;
    const int xcd = blockIdx.x & 7, qd = blockIdx.x >> 3;
    const int urank = (qd / NS) * 8 + xcd, slice = qd % NS;
    if (urank >= p.num_seqs * H) return;
    const int srank = urank / H, h = urank % H;
    const int n = p.order ? p.order[srank] : srank;
    int bos, eos;
    if (p.cu) { bos = p.cu[n]; eos = p.cu[n + 1]; }
    else { bos = n * p.T; eos = bos + p.T; }
    const int v0 = slice * DVS;
    const int nchunks = (eos - bos + C - 1) / C;

    if (wave >= NPW) {
        // =================== chain wave: 16 value channels ===================
        const int cb = wave - NPW;
        // S^T of this wave's value block (lane: value column v0 + 16 cb + lr,
        // key rows 16 kb + 4 lg + i)
        f32x4 St[NKB];
        const size_t srow = ((size_t)n * H + h) * DV * DK + (size_t)(v0 + 16 * cb + lr) * DK + 4 * lg;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            St[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (p.initial_state) St[kb] = *reinterpret_cast<const f32x4 *>(p.initial_state + srow + 16 * kb);
        }
        float *gof = static_cast<float *>(p.out);
        __bf16 *gob = static_cast<__bf16 *>(p.out);

        for (int it = 0; it <= nchunks; ++it) {
#pragma unroll
            for (int b = 0; b < CHAIN_STAGE; ++b) __syncthreads();
            if (it >= 1) {
                const Buf &bc = sm.buf[(it + 1) & 1];
                const int jc = it - 1;
                const int t0 = bos + jc * C;
                const int nv = min(C, eos - t0);
                // every LDS operand of the chunk, read up front
                RowA<ST, NKB> ka[NB], qa[NB];
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    ka[rb].load(&bc.Kt[16 * rb + lr][0], lg);
                    qa[rb].load(&bc.Qt[16 * rb + lr][0], lg);
                }
                float vv[NB][4], bt[NB][4], eg[NB][4];
#pragma unroll
                for (int rb = 0; rb < NB; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * rb + 4 * lg + i;
                        vv[rb][i] = (float)bc.V[t][16 * cb + lr];
                        bt[rb][i] = bc.beta[t];
                        eg[rb][i] = KDA ? 1.f : bc.eg[KDA ? 0 : t];
                    }
                RegB<ST, NKB> sop;
                sop.set(St);
                f32x4 X[NB], Y[NB], W[NB];
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    X[rb] = sop.mma(f32x4{0.f, 0.f, 0.f, 0.f}, ka[rb]);
                    Y[rb] = sop.mma(f32x4{0.f, 0.f, 0.f, 0.f}, qa[rb]);
                }
                RowA<ST, NB> ta[NB], ma[NB];
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    const int ns = (16 * rb + 16 + 31) / 32;   // T and M are lower triangular
                    ta[rb].load(&bc.Tm[16 * rb + lr][0], lg, ns);
                    ma[rb].load(&bc.Mm[16 * rb + lr][0], lg, ns);
                }
#pragma unroll
                for (int rb = 0; rb < NB; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        Y[rb][i] *= eg[rb][i];
                        W[rb][i] = bt[rb][i] * (vv[rb][i] - X[rb][i] * eg[rb][i]);
                    }
                RegB<ST, NB> wh, wl;
                wh.set_split(W, wl);
                f32x4 U[NB];
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    const int ns = (16 * rb + 16 + 31) / 32;
                    U[rb] = wh.mma(f32x4{0.f, 0.f, 0.f, 0.f}, ta[rb], ns);
                    if constexpr (SPLIT) U[rb] = wl.mma(U[rb], ta[rb], ns);
                }
                RowA<ST, NB> kea[NKB];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) kea[kb].load(&bc.KeT[16 * kb + lr][0], lg);
                RegB<ST, NB> uh, ul;
                uh.set_split(U, ul);
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    const int ns = (16 * rb + 16 + 31) / 32;
                    f32x4 o = uh.mma(Y[rb], ma[rb], ns);
                    if constexpr (SPLIT) o = ul.mma(o, ma[rb], ns);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * rb + 4 * lg + i;
                        if (t < nv) {
                            const size_t off = ((size_t)(t0 + t) * H + h) * DV + v0 + 16 * cb + lr;
                            if (p.out_bf16) gob[off] = (__bf16)(p.scale * o[i]);
                            else gof[off] = p.scale * o[i];
                        }
                    }
                }
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    f32x4 acc = St[kb];
                    if constexpr (KDA) {
                        const f32x4 d = *reinterpret_cast<const f32x4 *>(&bc.dec[16 * kb + 4 * lg]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[i] *= d[i];
                    } else {
                        const float d = bc.dec[0];
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[i] *= d;
                    }
                    acc = uh.mma(acc, kea[kb]);
                    if constexpr (SPLIT) acc = ul.mma(acc, kea[kb]);
                    St[kb] = acc;
                }
            }
#pragma unroll
            for (int b = CHAIN_STAGE; b < NBAR; ++b) __syncthreads();
        }
        if (p.final_state) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                *reinterpret_cast<f32x4 *>(p.final_state + srow + 16 * kb) = St[kb];
        }
        return;
    }

    // ======================= prologue waves (256 threads) ====================
    const IT *gq = static_cast<const IT *>(p.q);
    const IT *gk = static_cast<const IT *>(p.k);
    const IT *gv = static_cast<const IT *>(p.v);
    IV kreg[KVPT], qreg[KVPT], vreg;
    float greg[KDA ? SEGL : 1];                    // KDA: this lane's (channel, token segment) of log-decay
    float gsc = 0.f, breg = 0.f;
    const int gc = tid / NSEG, gseg = tid % NSEG;  // KDA prefix-sum lane: key channel, token segment
    // raw inputs of chunk j into registers (zeros past the sequence end)
    auto prefetch = [&](int j) {
        const int t0 = bos + j * C;
        const int nv = j < nchunks ? min(C, eos - t0) : 0;
#pragma unroll
        for (int x = 0; x < KVPT; ++x) {
            const int e = tid + 256 * x;
            const int t = e / (DK / EPV), c = (e % (DK / EPV)) * EPV;
            kreg[x] = IV{};
            qreg[x] = IV{};
            if (e < KV && t < nv) {
                const size_t off = ((size_t)(t0 + t) * H + h) * DK + c;
                kreg[x] = *reinterpret_cast<const IV *>(gk + off);
                qreg[x] = *reinterpret_cast<const IV *>(gq + off);
            }
        }
        if constexpr (KDA) {
#pragma unroll
            for (int x = 0; x < SEGL; ++x) {
                const int t = gseg * SEGL + x;
                greg[x] = t < nv ? p.log_alpha[((size_t)(t0 + t) * H + h) * DK + gc] : 0.f;
            }
        } else {
            gsc = tid < nv ? p.log_alpha[(size_t)(t0 + tid) * H + h] : 0.f;
        }
        vreg = IV{};
        if (tid < VV) {
            const int t = tid / (DVS / EPV), c = (tid % (DVS / EPV)) * EPV;
            if (t < nv) vreg = *reinterpret_cast<const IV *>(gv + ((size_t)(t0 + t) * H + h) * DV + v0 + c);
        }
        breg = tid < nv ? p.beta[(size_t)(t0 + tid) * H + h] : 0.f;
    };

    // Gram tiles of the lower block triangle.  M (operand, zero above the
    // diagonal) goes to waves 0..NLT-1, one tile each; the last prologue wave
    // computes the A tiles and then T = (I + A)^-1 by itself, so the A -> T
    // dependency needs no barrier (a wave's LDS accesses complete in order).
    auto gram_inverse = [&](Buf &bp) {
        constexpr int NLT = NB * (NB + 1) / 2;     // lower tiles
        const int I0[3] = {0, 1, 1}, J0[3] = {0, 0, 1};
        if (wave < NLT) {
            const int I = I0[wave], J = J0[wave];
            f32x4 a0{0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0;
            if constexpr (KDA) {
                a0 = tile_mma<GT, DK>(a0, &sm.Lq[16 * I][0], LDK, &sm.Rh[16 * J][0], LDK, lane);
                if constexpr (SPLIT) {
                    a1 = tile_mma<GT, DK>(a1, &sm.Lq[16 * I][0], LDK, &sm.Rl[16 * J][0], LDK, lane);
                    a2 = tile_mma<GT, DK>(a2, &sm.Lql[16 * I][0], LDK, &sm.Rh[16 * J][0], LDK, lane);
                }
            } else {
                a0 = tile_mma<ST, DK>(a0, &bp.Qt[16 * I][0], LDK, &bp.Kt[16 * J][0], LDK, lane);
            }
            const f32x4 acc = a0 + a1 + a2;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * I + 4 * lg + i, c = 16 * J + lr;
                float val = 0.f;
                if (c <= r) {
                    val = acc[i];
                    if constexpr (!KDA) val *= __expf(sm.g[r] - sm.g[c]);
                }
                bp.Mm[r][c] = (ST)val;
                if (NB == 2 && I == 0) bp.Mm[r][16 + lr] = (ST)0.f;
            }
        }
        if (wave == NPW - 1) {
#pragma unroll
            for (int x = 0; x < NLT; ++x) {
                const int I = I0[x], J = J0[x];
                f32x4 a{0.f, 0.f, 0.f, 0.f};
                if constexpr (KDA) a = tile_mma<GT, DK>(a, &sm.Lk[16 * I][0], LDK, &sm.Rh[16 * J][0], LDK, lane);
                else a = tile_mma<ST, DK>(a, &bp.Kt[16 * I][0], LDK, &bp.Kt[16 * J][0], LDK, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * I + 4 * lg + i, c = 16 * J + lr;
                    float val = 0.f;
                    if (c < r) {
                        val = a[i] * bp.beta[r];
                        if constexpr (!KDA) val *= __expf(sm.g[r] - sm.g[c]);
                    }
                    sm.u.at.A[r][c] = val;
                }
            }
            // diagonal 16x16 blocks by forward substitution, one column per
            // lane: t_i = delta_ij - sum_{m<i} A_im t_m, row i of A read from LDS
            if (lane < C) {
                const int I = lane / 16, jc = lane % 16;
                float tcol[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float acc0 = (i == jc) ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
                    for (int m4 = 0; m4 < i; m4 += 4) {
                        const f32x4 v = *reinterpret_cast<const f32x4 *>(&sm.u.at.A[16 * I + i][16 * I + m4]);
#pragma unroll
                        for (int y = 0; y < 4; ++y)
                            if (m4 + y < i) {
                                if (y & 1) acc1 -= v[y] * tcol[m4 + y];
                                else acc0 -= v[y] * tcol[m4 + y];
                            }
                    }
                    tcol[i] = acc0 + acc1;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    sm.u.at.Tf[16 * I + i][16 * I + jc] = tcol[i];
                    bp.Tm[16 * I + i][16 * I + jc] = (ST)tcol[i];
                }
            }
            if constexpr (NB == 2) {
                // T_10 = -T_11 (A_10 T_00); four entries per lane
#pragma unroll
                for (int y = 0; y < 4; ++y) {
                    const int e = lane + 64 * y, r = e / 16, c = e % 16;
                    float acc = 0.f;
#pragma unroll
                    for (int m = 0; m < 16; ++m) acc += sm.u.at.A[16 + r][m] * sm.u.at.Tf[m][c];
                    sm.P[e] = acc;
                }
#pragma unroll
                for (int y = 0; y < 4; ++y) {
                    const int e = lane + 64 * y, r = e / 16, c = e % 16;
                    float acc = 0.f;
#pragma unroll
                    for (int m = 0; m < 16; ++m) acc += sm.u.at.Tf[16 + r][16 + m] * sm.P[m * 16 + c];
                    bp.Tm[16 + r][c] = (ST)(-acc);
                    bp.Tm[r][16 + c] = (ST)0.f;
                }
            }
        }
    };
    // K_end^T (key rows, token columns) via column reads of row-major data
    auto transpose_kend = [&](Buf &bp) {
        if (wave == NPW - 1) return;
        for (int e = tid; e < DK * (C / EPV); e += 64 * (NPW - 1)) {
            const int c = e % DK, t0 = (e / DK) * EPV;
            SV o;
#pragma unroll
            for (int x = 0; x < EPV; ++x) {
                float val;
                if constexpr (KDA) {
                    val = (float)sm.Rh[t0 + x][c];
                    if constexpr (SPLIT) val += (float)sm.Rl[t0 + x][c];
                    val *= sm.egcm[c];
                } else {
                    val = (float)bp.Kt[t0 + x][c] * sm.egc[t0 + x];
                }
                o[x] = (ST)val;
            }
            *reinterpret_cast<SV *>(&bp.KeT[c][t0]) = o;
        }
    };

    prefetch(0);
    // iteration `it` builds chunk it; the chain waves consume chunk it-1
    for (int it = 0; it <= nchunks; ++it) {
        const bool pro = it < nchunks;
        Buf &bp = sm.buf[it & 1];
        if (pro) {
            if (tid < VV) {
                const int t = tid / (DVS / EPV), c = (tid % (DVS / EPV)) * EPV;
                *reinterpret_cast<IV *>(&bp.V[t][c]) = vreg;
            }
            if (tid < C) bp.beta[tid] = breg;
        }
        if constexpr (!KDA) {
            // ---- stage 1: inputs to LDS, per-head decay prefix sums
            if (pro) {
                if (wave == 0) {
                    float x = gsc;
#pragma unroll
                    for (int off = 1; off < 64; off <<= 1) {
                        const float y = __shfl_up(x, off);
                        if (lane >= off) x += y;
                    }
                    const float gC = __shfl(x, C - 1);
                    if (lane < C) {
                        sm.g[lane] = x;
                        bp.eg[lane] = __expf(x);
                        sm.egc[lane] = __expf(gC - x);
                    }
                    if (lane == 0) bp.dec[0] = __expf(gC);
                }
#pragma unroll
                for (int x = 0; x < KVPT; ++x) {
                    const int e = tid + 256 * x;
                    if (e < KV) {
                        const int t = e / (DK / EPV), c = (e % (DK / EPV)) * EPV;
                        SV kt, qt;
#pragma unroll
                        for (int y = 0; y < EPV; ++y) {
                            kt[y] = (ST)(float)kreg[x][y];
                            qt[y] = (ST)(float)qreg[x][y];
                        }
                        *reinterpret_cast<SV *>(&bp.Kt[t][c]) = kt;
                        *reinterpret_cast<SV *>(&bp.Qt[t][c]) = qt;
                    }
                }
            }
            __syncthreads();
            // ---- stage 2: Gram, T, K_end^T; next chunk's inputs requested
            if (pro) {
                gram_inverse(bp);
                transpose_kend(bp);
                prefetch(it + 1);
            }
            __syncthreads();
        } else {
            // ---- stage 1: per-channel prefix sums and e^{g-m}
            if (pro) {
                float gv_[SEGL];
#pragma unroll
                for (int s2 = 0; s2 < SEGL; ++s2) gv_[s2] = greg[s2];
#pragma unroll
                for (int s2 = 1; s2 < SEGL; ++s2) gv_[s2] += gv_[s2 - 1];
                float incl = gv_[SEGL - 1];
#pragma unroll
                for (int off = 1; off < NSEG; off <<= 1) {
                    const float y = __shfl_up(incl, off, NSEG);
                    if (gseg >= off) incl += y;
                }
                const float carry = incl - gv_[SEGL - 1];
                const float gC = __shfl(incl, NSEG - 1, NSEG);
                const float g0 = __shfl(gv_[0], 0, NSEG);
                const float m = 0.5f * (g0 + gC);
#pragma unroll
                for (int s2 = 0; s2 < SEGL; ++s2) sm.u.G[gseg * SEGL + s2][gc] = __expf(gv_[s2] + carry - m);
                if (gseg == 0) {
                    sm.em[gc] = __expf(m);
                    sm.egcm[gc] = __expf(gC - m);
                    bp.dec[gc] = __expf(gC);
                }
            }
            __syncthreads();
            // ---- stage 2: decayed operands; next chunk's inputs requested
            if (pro) {
#pragma unroll
                for (int x = 0; x < KVPT; ++x) {
                    const int e = tid + 256 * x;
                    if (e < KV) {
                        const int t = e / (DK / EPV), c = (e % (DK / EPV)) * EPV;
                        SV kt, qt;
                        GV lk, lq, lql, rh, rl;
#pragma unroll
                        for (int y = 0; y < EPV; ++y) {
                            const float kf = (float)kreg[x][y], qf = (float)qreg[x][y];
                            const float e1 = sm.u.G[t][c + y];
                            const float e2 = __builtin_amdgcn_rcpf(e1);
                            lk[y] = (GT)(kf * e1);
                            GT hi, lo;
                            split2<GT>(qf * e1, hi, lo);
                            lq[y] = hi;
                            lql[y] = lo;
                            split2<GT>(kf * e2, hi, lo);
                            rh[y] = hi;
                            rl[y] = lo;
                            const float eg = e1 * sm.em[c + y];
                            kt[y] = (ST)(kf * eg);
                            qt[y] = (ST)(qf * eg);
                        }
                        *reinterpret_cast<GV *>(&sm.Lk[t][c]) = lk;
                        *reinterpret_cast<GV *>(&sm.Lq[t][c]) = lq;
                        *reinterpret_cast<GV *>(&sm.Rh[t][c]) = rh;
                        if constexpr (SPLIT) {
                            *reinterpret_cast<GV *>(&sm.Lql[t][c]) = lql;
                            *reinterpret_cast<GV *>(&sm.Rl[t][c]) = rl;
                        }
                        *reinterpret_cast<SV *>(&bp.Kt[t][c]) = kt;
                        *reinterpret_cast<SV *>(&bp.Qt[t][c]) = qt;
                    }
                }
                prefetch(it + 1);
            }
            __syncthreads();
            // ---- stage 3: Gram, T, K_end^T
            if (pro) {
                gram_inverse(bp);
                transpose_kend(bp);
            }
            __syncthreads();
        }
    }
}

template <int DK, int DVS, int C, bool KDA, typename IT>
hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t st) {
    PrefillKArgs p;
    p.T = a.seqlen;
    p.H = a.num_heads;
    p.DV = a.dv;
    p.num_seqs = a.num_seqs;
    p.q = a.q; p.k = a.k; p.v = a.v;
    p.beta = a.beta; p.log_alpha = a.log_alpha; p.initial_state = a.initial_state;
    p.cu = a.cu_seqlens; p.order = a.cu_seqlens ? a.order : nullptr;
    p.scale = a.scale;
    p.out = a.out;
    p.final_state = a.final_state;
    p.out_bf16 = a.out_bf16;
    const long units = (long)a.num_seqs * a.num_heads;
    const long grid = ((units + 7) / 8) * 8 * (a.dv / DVS);
    hipLaunchKernelGGL((prefill_kernel<DK, DVS, C, KDA, IT>), dim3((unsigned)grid),
                       dim3(64 * (kPrologueWaves + DVS / 16)), 0, st, p);
    return hipGetLastError();
}

}  // namespace gdr
