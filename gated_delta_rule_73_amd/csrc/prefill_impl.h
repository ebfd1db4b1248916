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
// Rows of S (value channels) evolve independently, so a workgroup owns a
// slice of DVS value channels of one (sequence, head) and walks its chunks in
// order; the key-side work (Gram, T) is recomputed by each slice.
//
// Precision (bf16 q/k/v).  Outputs reach ~15x their RMS, so an error bound of
// 2e-2 x RMS on the largest element needs ~1e-3 relative accuracy on the
// terms that carry v; one bf16 rounding (2^-8) of those terms is too coarse.
// The products therefore run on fp16 MFMA (11-bit operands) with the value-
// carrying operands W and U split into an fp16 hi + lo pair (two MFMAs each),
// and the per-channel decay Gram M of Kimi Delta Attention from bf16 hi + lo
// pairs (three MFMAs: hi.hi + hi.lo + lo.hi).  The Gram A that feeds T keeps
// single bf16 operands: the delta rule's erase step corrects what an error in
// T leaves behind.  fp32 q/k/v use fp32 MFMA throughout.
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

// acc += A[16 rows] * B[16 rows]^T over k in [k0, k1); both row-major in LDS
// with k contiguous (leading dimensions lda, ldb, in elements).
template <typename OT>
__device__ __forceinline__ f32x4 tile_mma(f32x4 acc, const OT *A, int lda, const OT *B, int ldb, int k0, int k1,
                                          int lane) {
    using M = Mfma<OT>;
    const OT *pa = A + (lane & 15) * lda + (lane >> 4) * M::KPL;
    const OT *pb = B + (lane & 15) * ldb + (lane >> 4) * M::KPL;
    for (int k = k0; k < k1; k += M::KSTEP) acc = M::mma(M::load(pa + k), M::load(pb + k), acc);
    return acc;
}

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

// ---- shared-memory layout ---------------------------------------------------
template <int DK, int DVS, int C, bool KDA, typename IT>
struct PrefillSmem {
    using ST = typename Prec<IT>::ST;
    using GT = typename Prec<IT>::GT;
    static constexpr bool SPLIT = Prec<IT>::SPLIT;
    static constexpr int PAD = 16 / sizeof(ST);   // 16-byte row padding spreads LDS banks
    static constexpr int LDK = DK + PAD;          // [*][DK] operand rows (ST and GT have equal size)
    static constexpr int LDC = C + PAD;           // [*][C] operand rows
    static constexpr int LDA = C + 4;             // fp32 [C][C]
    static constexpr int NB = C / 16;
    static constexpr int KG = KDA ? C : 1;        // rows of per-channel Gram operands
    static constexpr int KGS = (KDA && SPLIT) ? C : 1;
    static constexpr int SP = SPLIT ? DVS : 1;

    ST Kt[C][LDK];          // GDN: k            KDA: k e^g
    ST Qt[C][LDK];          // GDN: q            KDA: q e^g
    ST KeT[DK][LDC];        // (k e^{g_C - g})^T
    GT Lk[KG][LDK];         // KDA: k e^{g-m}
    GT Lq[KG][LDK];         // KDA: q e^{g-m} (hi)
    GT Lql[KGS][LDK];       //                (lo)
    GT Rh[KG][LDK];         // KDA: k e^{m-g} (hi)
    GT Rl[KGS][LDK];        //                (lo)
    union {
        float G[KDA ? C : 1][DK];   // KDA: log-decay, then its in-chunk prefix sum
        struct {
            float A[C][LDA];        // strict_tril(diag(b) Gram)
            float Tf[C][LDA];       // (I + A)^-1
        } at;
        float O[C][DVS + 4];        // output slice, staged for the store
    } u;
    float P[(NB > 1 ? NB - 1 : 1) * 256];  // inverse scratch
    ST M[C][LDC];           // tril(Q K^T) with decay
    ST T[C][LDC];           // (I + A)^-1
    ST S[DVS][LDK];         // state slice operand
    ST Wh[DVS][LDC];        // diag(b)(V - X), transposed [value][token]  (hi)
    ST Wl[SP][LDC];         //                                              (lo)
    ST Uh[DVS][LDC];        // U, transposed (hi)
    ST Ul[SP][LDC];         //               (lo)
    IT V[C][DVS];           // value slice
    float beta[C];
    float g[C], eg[C], egc[C];                      // GDN: g, e^g, e^{g_C - g}
    float m[KDA ? DK : 1], em[KDA ? DK : 1];        // KDA: reference m, e^m
    float egcm[KDA ? DK : 1], egC[KDA ? DK : 1];    // KDA: e^{g_C - m}, e^{g_C}
    float egCs;                                     // GDN: e^{g_C}
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

// hi/lo split of x in ST: hi = ST(x), lo = ST(x - hi) (lo unused without SPLIT)
template <typename ST>
__device__ __forceinline__ void split2(float x, ST &hi, ST &lo) {
    hi = (ST)x;
    lo = (ST)(x - (float)hi);
}

template <int DK, int DVS, int C, bool KDA, typename IT>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillKArgs p) {
    using SM = PrefillSmem<DK, DVS, C, KDA, IT>;
    using ST = typename SM::ST;
    using GT = typename SM::GT;
    constexpr bool SPLIT = SM::SPLIT;
    constexpr int EPV = 16 / sizeof(IT);           // elements per 16-byte input vector
    using IV = typename VecT<IT, EPV>::type;
    using SV = typename VecT<ST, EPV>::type;
    using GV = typename VecT<GT, EPV>::type;
    using MS = Mfma<ST>;
    constexpr int LDK = SM::LDK, LDC = SM::LDC;
    constexpr int NB = C / 16;                     // 16-token blocks
    constexpr int NCB = DVS / 16;                  // 16-channel value blocks
    constexpr int NKB = DK / 16;                   // 16-channel key blocks
    constexpr int NST = NCB * NKB;                 // state tiles
    constexpr int STPW = (NST + 3) / 4;            // state tiles per wave
    constexpr int NOT = NB * NCB;                  // output tiles per chunk
    constexpr int OTPW = (NOT + 3) / 4;
    constexpr int KV = C * (DK / EPV);             // 16-byte k (or q) vectors per chunk
    constexpr int KVPT = (KV + 255) / 256;         // ... per thread
    static_assert(sizeof(SM) <= 160 * 1024, "LDS budget");
    static_assert(C % MS::KSTEP == 0 && DK % MS::KSTEP == 0, "tile sizes");
    static_assert(sizeof(ST) == sizeof(IT) && sizeof(GT) == sizeof(IT), "operand sizes");

    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

    const IT *gq = static_cast<const IT *>(p.q);
    const IT *gk = static_cast<const IT *>(p.k);
    const IT *gv = static_cast<const IT *>(p.v);
    float *gof = static_cast<float *>(p.out);
    __bf16 *gob = static_cast<__bf16 *>(p.out);

    // ---- state slice in registers (fp32, MFMA accumulator layout)
    f32x4 Sreg[STPW];
    const size_t sbase = ((size_t)n * H + h) * DV * DK;
#pragma unroll
    for (int j = 0; j < STPW; ++j) {
        const int tile = wave + 4 * j;
        Sreg[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tile < NST && p.initial_state) {
            const int cb = tile / NKB, kb = tile % NKB;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                Sreg[j][i] = p.initial_state[sbase + (size_t)(v0 + 16 * cb + 4 * lg + i) * DK + 16 * kb + lr];
        }
    }

    for (int t0 = bos; t0 < eos; t0 += C) {
        const int nv = min(C, eos - t0);

        // ================= L: loads, gates, prefix sums, operands ===========
        IV kreg[KVPT], qreg[KVPT];
#pragma unroll
        for (int j = 0; j < KVPT; ++j) {
            const int e = tid + 256 * j;
            const int t = e / (DK / EPV), c = (e % (DK / EPV)) * EPV;
            kreg[j] = IV{};
            qreg[j] = IV{};
            if (e < KV && t < nv) {
                const size_t off = ((size_t)(t0 + t) * H + h) * DK + c;
                kreg[j] = *reinterpret_cast<const IV *>(gk + off);
                qreg[j] = *reinterpret_cast<const IV *>(gq + off);
            }
        }
        if (tid < C) sm.beta[tid] = tid < nv ? p.beta[(size_t)(t0 + tid) * H + h] : 0.f;
        for (int e = tid; e < C * (DVS / EPV); e += 256) {
            const int t = e / (DVS / EPV), c = (e % (DVS / EPV)) * EPV;
            IV vv{};
            if (t < nv) vv = *reinterpret_cast<const IV *>(gv + ((size_t)(t0 + t) * H + h) * DV + v0 + c);
            *reinterpret_cast<IV *>(&sm.V[t][c]) = vv;
        }
        if constexpr (!KDA) {
            if (wave == 0) {
                float x = (lane < nv) ? p.log_alpha[(size_t)(t0 + lane) * H + h] : 0.f;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float y = __shfl_up(x, off);
                    if (lane >= off) x += y;
                }
                const float gC = __shfl(x, C - 1);
                if (lane < C) {
                    sm.g[lane] = x;
                    sm.eg[lane] = __expf(x);
                    sm.egc[lane] = __expf(gC - x);
                }
                if (lane == 0) sm.egCs = __expf(gC);
            }
        } else {
            for (int e = tid; e < C * (DK / 4); e += 256) {
                const int t = e / (DK / 4), c = (e % (DK / 4)) * 4;
                f32x4 a{0.f, 0.f, 0.f, 0.f};
                if (t < nv) a = *reinterpret_cast<const f32x4 *>(p.log_alpha + ((size_t)(t0 + t) * H + h) * DK + c);
                *reinterpret_cast<f32x4 *>(&sm.u.G[t][c]) = a;
            }
            __syncthreads();
            for (int c = tid; c < DK; c += 256) {
                float run = 0.f;
                for (int t = 0; t < C; ++t) {
                    run += sm.u.G[t][c];
                    sm.u.G[t][c] = run;
                }
                const float m = 0.5f * (sm.u.G[0][c] + run);
                sm.m[c] = m;
                sm.em[c] = __expf(m);
                sm.egcm[c] = __expf(run - m);
                sm.egC[c] = __expf(run);
            }
        }
        // state operand of this chunk
#pragma unroll
        for (int j = 0; j < STPW; ++j) {
            const int tile = wave + 4 * j;
            if (tile < NST) {
                const int cb = tile / NKB, kb = tile % NKB;
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.S[16 * cb + 4 * lg + i][16 * kb + lr] = (ST)Sreg[j][i];
            }
        }
        __syncthreads();

        // operands from the registers holding k and q
#pragma unroll
        for (int j = 0; j < KVPT; ++j) {
            const int e = tid + 256 * j;
            if (e >= KV) break;
            const int t = e / (DK / EPV), c = (e % (DK / EPV)) * EPV;
            SV kt, qt;
            if constexpr (!KDA) {
                const float ec = sm.egc[t];
#pragma unroll
                for (int x = 0; x < EPV; ++x) {
                    const float kf = (float)kreg[j][x];
                    kt[x] = (ST)kf;
                    qt[x] = (ST)(float)qreg[j][x];
                    sm.KeT[c + x][t] = (ST)(kf * ec);
                }
            } else {
                GV lk, lq, lql, rh, rl;
#pragma unroll
                for (int x = 0; x < EPV; ++x) {
                    const float kf = (float)kreg[j][x], qf = (float)qreg[j][x];
                    const float d = sm.u.G[t][c + x] - sm.m[c + x];
                    const float e1 = __expf(d), e2 = __expf(-d);
                    lk[x] = (GT)(kf * e1);
                    GT hi, lo;
                    split2<GT>(qf * e1, hi, lo);
                    lq[x] = hi;
                    lql[x] = lo;
                    split2<GT>(kf * e2, hi, lo);
                    rh[x] = hi;
                    rl[x] = lo;
                    const float eg = e1 * sm.em[c + x];
                    kt[x] = (ST)(kf * eg);
                    qt[x] = (ST)(qf * eg);
                    sm.KeT[c + x][t] = (ST)(kf * e2 * sm.egcm[c + x]);
                }
                *reinterpret_cast<GV *>(&sm.Lk[t][c]) = lk;
                *reinterpret_cast<GV *>(&sm.Lq[t][c]) = lq;
                *reinterpret_cast<GV *>(&sm.Rh[t][c]) = rh;
                if constexpr (SPLIT) {
                    *reinterpret_cast<GV *>(&sm.Lql[t][c]) = lql;
                    *reinterpret_cast<GV *>(&sm.Rl[t][c]) = rl;
                }
            }
            *reinterpret_cast<SV *>(&sm.Kt[t][c]) = kt;
            *reinterpret_cast<SV *>(&sm.Qt[t][c]) = qt;
        }
        __syncthreads();

        // ================= G: Gram matrices A (fp32) and M (operand) ========
        for (int job = wave; job < 2 * NB * NB; job += 4) {
            const bool isM = job >= NB * NB;
            const int I = (job % (NB * NB)) / NB, J = job % NB;
            f32x4 acc{0.f, 0.f, 0.f, 0.f};
            if (J <= I) {
                if constexpr (!KDA) {
                    acc = tile_mma(acc, isM ? &sm.Qt[16 * I][0] : &sm.Kt[16 * I][0], LDK, &sm.Kt[16 * J][0], LDK, 0,
                                   DK, lane);
                } else if (!isM) {
                    acc = tile_mma(acc, &sm.Lk[16 * I][0], LDK, &sm.Rh[16 * J][0], LDK, 0, DK, lane);
                } else {
                    acc = tile_mma(acc, &sm.Lq[16 * I][0], LDK, &sm.Rh[16 * J][0], LDK, 0, DK, lane);
                    if constexpr (SPLIT) {
                        acc = tile_mma(acc, &sm.Lq[16 * I][0], LDK, &sm.Rl[16 * J][0], LDK, 0, DK, lane);
                        acc = tile_mma(acc, &sm.Lql[16 * I][0], LDK, &sm.Rh[16 * J][0], LDK, 0, DK, lane);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * I + 4 * lg + i, c = 16 * J + lr;
                float val = 0.f;
                if (isM ? (c <= r) : (c < r)) {
                    val = acc[i];
                    if constexpr (!KDA) val *= __expf(sm.g[r] - sm.g[c]);
                    if (!isM) val *= sm.beta[r];
                }
                if (isM) sm.M[r][c] = (ST)val;
                else sm.u.at.A[r][c] = val;
            }
        }
        __syncthreads();

        // ================= I: T = (I + A)^-1 =================================
        // diagonal 16x16 blocks by forward substitution, one column per thread
        if (tid < C) {
            const int I = tid / 16, jc = tid % 16;
            float tcol[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = (i == jc) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) acc -= sm.u.at.A[16 * I + i][16 * I + m] * tcol[m];
                tcol[i] = acc;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.u.at.Tf[16 * I + i][16 * I + jc] = tcol[i];
        }
        __syncthreads();
        // off-diagonal blocks by distance d = I - J:  T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ
        for (int d = 1; d < NB; ++d) {
            const int nblk = NB - d;
            for (int e = tid; e < nblk * 256; e += 256) {
                const int J = e / 256, I = J + d, r = (e % 256) / 16, c = e % 16;
                float acc = 0.f;
                for (int K = J; K < I; ++K)
#pragma unroll
                    for (int m = 0; m < 16; ++m) acc += sm.u.at.A[16 * I + r][16 * K + m] * sm.u.at.Tf[16 * K + m][16 * J + c];
                sm.P[e] = acc;
            }
            __syncthreads();
            for (int e = tid; e < nblk * 256; e += 256) {
                const int J = e / 256, I = J + d, r = (e % 256) / 16, c = e % 16;
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < 16; ++m) acc += sm.u.at.Tf[16 * I + r][16 * I + m] * sm.P[J * 256 + m * 16 + c];
                sm.u.at.Tf[16 * I + r][16 * J + c] = -acc;
            }
            __syncthreads();
        }
        for (int e = tid; e < C * C; e += 256) {
            const int r = e / C, c = e % C;
            sm.T[r][c] = (ST)(c <= r ? sm.u.at.Tf[r][c] : 0.f);
        }
        __syncthreads();

        // ================= X, Y; W = diag(b)(V - X) ==========================
        f32x4 Y[OTPW];
#pragma unroll
        for (int j = 0; j < OTPW; ++j) {
            const int tile = wave + 4 * j;
            Y[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (tile < NOT) {
                const int rb = tile / NCB, cb = tile % NCB;
                f32x4 X = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, &sm.Kt[16 * rb][0], LDK, &sm.S[16 * cb][0], LDK, 0, DK,
                                   lane);
                Y[j] = tile_mma(Y[j], &sm.Qt[16 * rb][0], LDK, &sm.S[16 * cb][0], LDK, 0, DK, lane);
                const int dv = 16 * cb + lr;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * rb + 4 * lg + i;
                    float x = X[i];
                    if constexpr (!KDA) { x *= sm.eg[r]; Y[j][i] *= sm.eg[r]; }
                    const float w = sm.beta[r] * ((float)sm.V[r][dv] - x);
                    ST hi, lo;
                    split2<ST>(w, hi, lo);
                    sm.Wh[dv][r] = hi;
                    if constexpr (SPLIT) sm.Wl[dv][r] = lo;
                }
            }
        }
        __syncthreads();

        // ================= U = T W (lower-triangular in tokens) ==============
#pragma unroll
        for (int j = 0; j < OTPW; ++j) {
            const int tile = wave + 4 * j;
            if (tile < NOT) {
                const int rb = tile / NCB, cb = tile % NCB;
                const int kend = min(C, ((16 * rb + 16 + MS::KSTEP - 1) / MS::KSTEP) * MS::KSTEP);
                f32x4 acc = tile_mma(f32x4{0.f, 0.f, 0.f, 0.f}, &sm.T[16 * rb][0], LDC, &sm.Wh[16 * cb][0], LDC, 0,
                                     kend, lane);
                if constexpr (SPLIT) acc = tile_mma(acc, &sm.T[16 * rb][0], LDC, &sm.Wl[16 * cb][0], LDC, 0, kend, lane);
                const int dv = 16 * cb + lr;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * rb + 4 * lg + i;
                    ST hi, lo;
                    split2<ST>(acc[i], hi, lo);
                    sm.Uh[dv][r] = hi;
                    if constexpr (SPLIT) sm.Ul[dv][r] = lo;
                }
            }
        }
        __syncthreads();

        // ================= O = Y + M U;  S <- S Diag(e^{g_C}) + U^T K_end =====
#pragma unroll
        for (int j = 0; j < OTPW; ++j) {
            const int tile = wave + 4 * j;
            if (tile < NOT) {
                const int rb = tile / NCB, cb = tile % NCB;
                const int kend = min(C, ((16 * rb + 16 + MS::KSTEP - 1) / MS::KSTEP) * MS::KSTEP);
                f32x4 acc = tile_mma(Y[j], &sm.M[16 * rb][0], LDC, &sm.Uh[16 * cb][0], LDC, 0, kend, lane);
                if constexpr (SPLIT) acc = tile_mma(acc, &sm.M[16 * rb][0], LDC, &sm.Ul[16 * cb][0], LDC, 0, kend, lane);
                const int dv = 16 * cb + lr;
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.u.O[16 * rb + 4 * lg + i][dv] = p.scale * acc[i];
            }
        }
#pragma unroll
        for (int j = 0; j < STPW; ++j) {
            const int tile = wave + 4 * j;
            if (tile < NST) {
                const int cb = tile / NKB, kb = tile % NKB;
                float dec;
                if constexpr (KDA) dec = sm.egC[16 * kb + lr];
                else dec = sm.egCs;
                f32x4 acc = Sreg[j];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] *= dec;
                acc = tile_mma(acc, &sm.Uh[16 * cb][0], LDC, &sm.KeT[16 * kb][0], LDC, 0, C, lane);
                if constexpr (SPLIT) acc = tile_mma(acc, &sm.Ul[16 * cb][0], LDC, &sm.KeT[16 * kb][0], LDC, 0, C, lane);
                Sreg[j] = acc;
            }
        }
        __syncthreads();

        // ================= write the output slice ============================
        for (int e = tid; e < C * (DVS / 4); e += 256) {
            const int t = e / (DVS / 4), c = (e % (DVS / 4)) * 4;
            if (t < nv) {
                const f32x4 o = *reinterpret_cast<const f32x4 *>(&sm.u.O[t][c]);
                const size_t off = ((size_t)(t0 + t) * H + h) * DV + v0 + c;
                if (p.out_bf16) {
                    bf16x4 b;
#pragma unroll
                    for (int x = 0; x < 4; ++x) b[x] = (__bf16)o[x];
                    *reinterpret_cast<bf16x4 *>(gob + off) = b;
                } else {
                    *reinterpret_cast<f32x4 *>(gof + off) = o;
                }
            }
        }
        __syncthreads();
    }

    if (p.final_state) {
#pragma unroll
        for (int j = 0; j < STPW; ++j) {
            const int tile = wave + 4 * j;
            if (tile < NST) {
                const int cb = tile / NKB, kb = tile % NKB;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    p.final_state[sbase + (size_t)(v0 + 16 * cb + 4 * lg + i) * DK + 16 * kb + lr] = Sreg[j][i];
            }
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
    hipLaunchKernelGGL((prefill_kernel<DK, DVS, C, KDA, IT>), dim3((unsigned)grid), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace gdr
