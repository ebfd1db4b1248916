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
//     W_n = -T diag(b) (K e^g)                                WY factor (negated)
//     U   = T diag(b) V + W_n S0^T
//     O   = (Q e^g) S0^T + M U,   M = tril((Q e^g)(K e^-g)^T)
//     S_C = S0 Diag(e^{g_C}) + U^T (K e^{g_C - g}).
// (U = T diag(b) (V - (K e^g) S0^T) regrouped so that W_n, which does not
// depend on the state, is formed once per chunk outside the serial chain.)
//
// Two kernels.  Everything that does not depend on the state (prefix sums of
// the gates, decayed operands, the Gram matrices, T) is independent across
// chunks (W_n included), so prep_kernel computes it for every (chunk, head)
// at once and writes one record per chunk to the workspace.  chain_kernel then walks the
// chunks of each (sequence, head) in order: loader waves stream the records
// (and the value slice) ahead into LDS slots (four at 16/32-token chunks; at
// 64-token chunks two slots, each split into the halves read before and after
// a mid-chunk barrier and refilled separately), and
// one chain wave per 16 value channels carries its part of the state
// transposed (S^T: key rows x value columns) as fp32 MFMA accumulators.  In
// that layout the state and U feed the next product straight from
// registers (each lane's accumulator rows are exactly the k-indices its MFMA
// operand fragment needs), so the serial chain U -> (O, S) reads LDS only for
// the record's shared operands.
//
// Precision (bf16 q/k/v).  Outputs reach ~15x their RMS, so an error bound of
// 2e-2 x RMS on the largest element needs ~1e-3 relative accuracy on the
// terms that carry v; one bf16 rounding (2^-8) of those terms is too coarse.
// The chain's products run on fp16 MFMA (11-bit operands) with the
// value-carrying operands W and U split into an fp16 hi + lo pair (two MFMAs
// each); the per-channel-decay Gram M is formed from bf16 hi + lo pairs
// (three MFMAs: hi.hi + hi.lo + lo.hi).  The Gram A that feeds T keeps single
// bf16 operands: the delta rule's erase step corrects what an error in T
// leaves behind.  fp32 q/k/v use fp32 MFMA throughout.
//
// Exponent range.  Gated DeltaNet: the decay is a per-row scalar; raw k/q
// (exact in fp16) feed the products and e^{g_r - g_i} <= 1 scales the fp32
// results.  Kimi Delta Attention: the decay sits inside the key-channel sum,
// so the Gram operands carry it around a per-channel reference
// m = (g_first + g_last)/2: k e^{g-m}, q e^{g-m}, k e^{m-g} stay within
// e^{+-half the chunk's decay} in bf16 (fp32 exponent range; a channel whose
// log-decay over one chunk falls below about -170 overflows it).  The
// state-side operands k e^g, q e^g, k e^{g_C-g} are all <= 1 in magnitude.
#pragma once

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace gdr {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

template <typename T, int N> struct VecT { typedef T type __attribute__((ext_vector_type(N))); };

// ---- operands held in registers in the accumulator layout ------------------
// MFMA 16x16 tiles: lane l holds row (l & 15) of each 16-row operand and a
// group of k-values selected by l >> 4; A and B share that k-assignment, so
// the k-order inside one instruction is irrelevant.  The result gives lane l
// rows 4*(l>>4)+i (i < 4) of column l&15.
//
// RegB: a k-dimension of NBLK 16-blocks held as fp32 accumulator tiles v[blk]
// (lane: k-indices 16*blk + 4*lg + i).  As an MFMA B operand it is consumed
// with the A operand read from LDS at the same k-indices (RowA).
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
    // split v = hi + lo: this object takes hi, `lo` takes the remainder.
    // hi keeps the top 11 significant bits (exact in fp16 over its normal
    // range), so lo = v - hi is exact in fp32 and |lo| < 2^-10 |v|.
    __device__ __forceinline__ void set_split(const f32x4 *v, RegB &lo) {
#pragma unroll
        for (int s = 0; s < NBLK / 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x0 = v[2 * s][i], x1 = v[2 * s + 1][i];
                const float h0 = __uint_as_float(__float_as_uint(x0) & 0xffffe000u);
                const float h1 = __uint_as_float(__float_as_uint(x1) & 0xffffe000u);
                f[s][i] = (_Float16)h0;
                f[s][4 + i] = (_Float16)h1;
                lo.f[s][i] = (_Float16)(x0 - h0);
                lo.f[s][4 + i] = (_Float16)(x1 - h1);
            }
    }
    static constexpr int STEPS = NBLK / 2;   // 32-wide k-steps
    // acc += A * B over k-step s only
    template <class RA>
    __device__ __forceinline__ f32x4 step(f32x4 acc, const RA &a, int s) const {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.f[s], f[s], acc, 0, 0, 0);
    }
    // acc += A * B, A given as preloaded fragments (RowA) of the same k-range
    template <class RA>
    __device__ __forceinline__ f32x4 mma(f32x4 acc, const RA &a, int nsteps = 1 << 20) const {
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
            if (s < nsteps) acc = step(acc, a, s);
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
    // k-steps are 32 wide (two 16-blocks), as for fp16 operands; a 16-row
    // chunk (NBLK = 1) has one half step
    static constexpr int STEPS = (NBLK + 1) / 2;
    template <class RA>
    __device__ __forceinline__ f32x4 step(f32x4 acc, const RA &a, int s) const {
#pragma unroll
        for (int b = 2 * s; b < 2 * s + 2 && b < NBLK; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[b][i], f[b][i], acc, 0, 0, 0);
        return acc;
    }
    template <class RA>
    __device__ __forceinline__ f32x4 mma(f32x4 acc, const RA &a, int nsteps = 1 << 20) const {
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
            if (s < nsteps) acc = step(acc, a, s);
        return acc;
    }
};

// Stored k-order of the A operands.  An fp16 k-step gives lane group lg the
// k-indices {4lg+i, 16+4lg+i} (i < 4) of its 32; the record stores each
// 32-wide k-block with those eight adjacent (position 8lg + 4h + i holds
// k = 16h + 4lg + i), so one 16-byte LDS read fetches a lane's operand.  The
// map keeps aligned groups of four together.  fp32 steps (16 wide, four
// adjacent k per lane) are stored in plain order.
template <typename ST> __host__ __device__ constexpr int kpos(int k) {
    if constexpr (sizeof(ST) == 2) return (k & ~31) | (((k & 15) >> 2) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
    else return k;
}

// A-operand fragments of one 16-row tile read from LDS at the k-indices a
// RegB of the same NBLK supplies (lane row = lr, k = 16*blk + 4*lg + i), the
// row stored in kpos order.
template <typename ST, int NBLK> struct RowA;
// The lane reads 16-byte group 4s + lg (s: k-step) of its row; `sw` XORs
// the group index for rows stored swizzled (row_swizzle).
template <int NBLK> struct RowA<_Float16, NBLK> {
    f16x8 f[NBLK / 2];
    __device__ __forceinline__ void load(const _Float16 *arow, int lg, int nsteps = 1 << 20, int sw = 0) {
#pragma unroll
        for (int s = 0; s < NBLK / 2; ++s)
            if (s < nsteps) f[s] = *reinterpret_cast<const f16x8 *>(arow + 8 * ((4 * s + lg) ^ sw));
    }
    // the inverse of load (plain rows, kpos order)
    __device__ __forceinline__ void store(_Float16 *arow, int lg) const {
#pragma unroll
        for (int s = 0; s < NBLK / 2; ++s) *reinterpret_cast<f16x8 *>(arow + 32 * s + 8 * lg) = f[s];
    }
};
template <int NBLK> struct RowA<float, NBLK> {
    f32x4 f[NBLK];
    __device__ __forceinline__ void load(const float *arow, int lg, int nsteps = 1 << 20, int sw = 0) {
        const int nblk = nsteps < NBLK ? 2 * nsteps : NBLK;
#pragma unroll
        for (int b = 0; b < NBLK; ++b)
            if (b < nblk) f[b] = *reinterpret_cast<const f32x4 *>(arow + 4 * ((4 * b + lg) ^ sw));
    }
    __device__ __forceinline__ void store(float *arow, int lg) const {
#pragma unroll
        for (int b = 0; b < NBLK; ++b) *reinterpret_cast<f32x4 *>(arow + 16 * b + 4 * lg) = f[b];
    }
};

// A lane's fragment of row `row` of T diag(b) (k = column), from the fp32 T
// row and b: T_row,s b_s for s <= row, else 0, rounded to ST.
template <typename ST, int NBLK>
__device__ __forceinline__ RowA<ST, NBLK> tbeta_fragment(const float *trow, const float *beta, int row, int lg);
template <int NBLK>
__device__ __forceinline__ RowA<_Float16, NBLK> tbeta_fragment_f16(const float *trow, const float *beta, int row, int lg) {
    RowA<_Float16, NBLK> r;
#pragma unroll
    for (int s = 0; s < NBLK / 2; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int s0 = 32 * s + 16 * h + 4 * lg;
            const f32x4 t = *reinterpret_cast<const f32x4 *>(trow + s0), b = *reinterpret_cast<const f32x4 *>(beta + s0);
#pragma unroll
            for (int i = 0; i < 4; ++i) r.f[s][4 * h + i] = (_Float16)(s0 + i <= row ? t[i] * b[i] : 0.f);
        }
    return r;
}
template <>
__device__ __forceinline__ RowA<_Float16, 2> tbeta_fragment<_Float16, 2>(const float *trow, const float *beta, int row, int lg) {
    return tbeta_fragment_f16<2>(trow, beta, row, lg);
}
template <>
__device__ __forceinline__ RowA<_Float16, 4> tbeta_fragment<_Float16, 4>(const float *trow, const float *beta, int row, int lg) {
    return tbeta_fragment_f16<4>(trow, beta, row, lg);
}
template <int NBLK>
__device__ __forceinline__ RowA<float, NBLK> tbeta_fragment_f32(const float *trow, const float *beta, int row, int lg) {
    RowA<float, NBLK> r;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
        const int s0 = 16 * blk + 4 * lg;
        const f32x4 t = *reinterpret_cast<const f32x4 *>(trow + s0), b = *reinterpret_cast<const f32x4 *>(beta + s0);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.f[blk][i] = s0 + i <= row ? t[i] * b[i] : 0.f;
    }
    return r;
}
template <>
__device__ __forceinline__ RowA<float, 1> tbeta_fragment<float, 1>(const float *trow, const float *beta, int row, int lg) {
    return tbeta_fragment_f32<1>(trow, beta, row, lg);
}
template <>
__device__ __forceinline__ RowA<float, 2> tbeta_fragment<float, 2>(const float *trow, const float *beta, int row, int lg) {
    return tbeta_fragment_f32<2>(trow, beta, row, lg);
}

// acc += A * B over k-step s, both operands read from LDS as RowA fragments
// (A rows and B columns at lane l & 15)
template <int NBLK>
__device__ __forceinline__ f32x4 rowa_mma(f32x4 acc, const RowA<_Float16, NBLK> &a, const RowA<_Float16, NBLK> &b, int s) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.f[s], b.f[s], acc, 0, 0, 0);
}
template <int NBLK>
__device__ __forceinline__ f32x4 rowa_mma(f32x4 acc, const RowA<float, NBLK> &a, const RowA<float, NBLK> &b, int s) {
#pragma unroll
    for (int blk = 2 * s; blk < 2 * s + 2 && blk < NBLK; ++blk)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[blk][i], b.f[blk][i], acc, 0, 0, 0);
    return acc;
}

// ---- Gram products of the prep kernel: one 32-wide k-step -------------------
// Each lane supplies 8 operand values for the k-indices {4lg+i, 16+4lg+i}
// (i < 4) of the step; A and B use the same assignment.
__device__ __forceinline__ f32x4 gram_mma(f32x4 acc, const bf16x8 &a, const bf16x8 &b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 gram_mma(f32x4 acc, const f16x8 &a, const f16x8 &b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 gram_mma(f32x4 acc, const f32x8 &a, const f32x8 &b) {
#pragma unroll
    for (int x = 0; x < 8; ++x) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[x], b[x], acc, 0, 0, 0);
    return acc;
}
template <typename T> struct Frag8;
template <> struct Frag8<__bf16> { using type = bf16x8; };
template <> struct Frag8<_Float16> { using type = f16x8; };
template <> struct Frag8<float> { using type = f32x8; };

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

template <typename ST, int N>
__device__ __forceinline__ void store_vec(ST *dst, const ST (&v)[N]) {
    typename VecT<ST, N>::type x;
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = v[i];
    *reinterpret_cast<typename VecT<ST, N>::type *>(dst) = x;
}

// LDS row pitch for rows read as MFMA A fragments (lane: row l & 15, 16
// bytes at column group l >> 4).  A wave's 16-byte reads are served 32 lanes
// at a time from 128 four-byte banks, i.e. 16 rows x 32 contiguous bytes per
// half wave; those meet every bank once exactly when the pitch is an odd
// multiple of 32 bytes (measured with the LDS bank-conflict counter on gfx950).
constexpr int lds_pitch(int bytes) { return bytes + ((32 - bytes % 64) + 64) % 64; }

// ---- buffer stores ----------------------------------------------------------
// Fourth descriptor word of a raw (unstructured) buffer on CDNA.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kCachePolicyNT = 2;   // non-temporal
__device__ __forceinline__ void buffer_store_nt(__amdgpu_buffer_rsrc_t r, int byte_ofs, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, byte_ofs, 0, kCachePolicyNT);
}
__device__ __forceinline__ void buffer_store_nt(__amdgpu_buffer_rsrc_t r, int byte_ofs, __bf16 v) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), r, byte_ofs, 0, kCachePolicyNT);
}

// ---- per-chunk record (workspace, unpadded rows; the k-index of the A
// operands Wn, Qt (key channel), KeT, Tm, Mm (token) stored in kpos order) ----
template <int DK, int C, bool KDA, typename IT>
struct ChunkRec {
    using ST = typename Prec<IT>::ST;
    float dec[KDA ? DK : 4];   // e^{g_C}: per key channel (KDA) or dec[0] (GDN)
    ST Wn[C][DK];              // -T diag(b) (k e^g) (negated: U accumulates from T diag(b) V)
    ST Qt[C][DK];              // q e^g
    ST KeT[DK][C];             // (k e^{g_C - g})^T
    ST Tm[C][C];               // T diag(b), zero above the diagonal
    ST Mm[C][C];               // M, zero above the diagonal
};

// ============================ prep kernel ====================================
template <int DK, int C, bool KDA, typename IT>
struct PrepSmem {
    static constexpr int NB = C / 16, NT = NB * (NB + 1) / 2;
    static constexpr int LDG = DK + 4;                 // fp32 rows
    static constexpr int LDI = DK + 16 / sizeof(IT);   // input rows
    static constexpr int LDA = C + 4;
    // 64-token chunks (WIDE): the four waves' partial Gram tiles are summed
    // in pairs into two copies, and (K e^g)^T is parked in the staged q's
    // columns once the Gram phase has read them (see the kernel), so that two
    // workgroups still share a CU.
    static constexpr bool WIDE = NB == 4;
    static constexpr int NCOPY = WIDE ? 2 : 4;
    using ST = typename Prec<IT>::ST;
    static constexpr int LDT = lds_pitch(C * (int)sizeof(ST)) / (int)sizeof(ST);
    static constexpr int TILEB = 16 * 20 * 4;                    // one fp32 tile, rows of 20
    static constexpr int OFF_TF = NT * TILEB;                    // WIDE: T after the A tiles
    static constexpr int OFF_TFT = OFF_TF + C * LDA * 4;         //   then T^T
    static constexpr int RAWB = WIDE ? OFF_TFT + C * LDA * 4 : 16;
    // WIDE: the staged q block is also where the Gram phase parks (K e^g)^T
    // for the W product, so it must lie past everything written in between
    // (the partial tiles, then A, T and T^T): padding before Ks where needed.
    static constexpr int GR = KDA ? C : 1;            // rows of G
    static constexpr int TILES_END = NCOPY * 2 * NT * TILEB > RAWB ? NCOPY * 2 * NT * TILEB : RAWB;
    static constexpr int QB = C * LDI * (int)sizeof(IT);
    static constexpr int PADB0 = TILES_END - GR * LDG * 4 - QB;
    static constexpr int PADB = WIDE && PADB0 > 0 ? (PADB0 + 15) / 16 * 16 : 0;
    struct InPlain {
        float G[GR][LDG];   // KDA: log-decay, then g - m
        IT Ks[C][LDI];
        IT Qs[C][LDI];
    };
    struct InPadded {
        float G[GR][LDG];
        char pad[PADB > 0 ? PADB : 16];
        IT Ks[C][LDI];
        IT Qs[C][LDI];
    };
    using In = typename std::conditional<(PADB > 0), InPadded, InPlain>::type;
    static_assert(!WIDE || GR * LDG * 4 + PADB + QB >= TILES_END, "staged q past the tiles");
    union alignas(16) {
        In in;
        float Pt[NCOPY][2 * NT][16][20];  // partial Gram tiles: A tiles, then M tiles
        char raw[RAWB];
    } u;
    alignas(16) float em[KDA ? DK : 4];  // KDA: e^m
    float g[C], egc[C], egt[C];          // GDN: g, e^{g_C - g}, e^g
    alignas(16) float beta[C];
    // Once the partial tiles are summed, their space holds the lower tiles
    // of A (in place of copy 0's partials: each thread overwrites only what
    // it has read), T = (I + A)^-1 and T's diagonal blocks transposed.
    __device__ float *a_tile(int tt) { return &u.Pt[0][tt][0][0]; }   // rows of 20
    __device__ float (*tf())[LDA] {
        if constexpr (WIDE) return reinterpret_cast<float (*)[LDA]>(u.raw + OFF_TF);
        else return reinterpret_cast<float (*)[LDA]>(&u.Pt[1][0][0][0]);
    }
    __device__ float (*tft())[LDA] {
        if constexpr (WIDE) return reinterpret_cast<float (*)[LDA]>(u.raw + OFF_TFT);
        else return reinterpret_cast<float (*)[LDA]>(&u.Pt[2][0][0][0]);
    }
    static_assert(WIDE || C * LDA <= 2 * NT * 16 * 20, "T fits in one wave's partial tiles");
    // operands of W = T diag(b) (K e^g), token index in kpos order
    alignas(16) ST ktT[WIDE ? 1 : DK][LDT];
};

struct PrepKArgs {
    int T, H, num_seqs;
    int HK, G;                   // q/k heads; value head h reads q/k head h / G
    long num_records;            // chunk slots x heads in this launch
    int j0, seg_chunks;          // dense: chunks [j0, j0 + seg_chunks) of every sequence
    float scale;                 // readout factor, folded into Q e^g and M
    const void *q, *k;
    const void *beta, *log_alpha;    // fp32 or bf16 (the kernel's GDT)
    const int32_t *cu, *choff;
    char *rec;
};

// Every (chunk, head) record is independent, so this kernel is bound by its
// HBM traffic, not by the latency of its serial steps: a few persistent
// workgroups (four waves each) per CU walk the records, each holding the next
// record's inputs in flight while it computes the current one.
// GRP: value heads share q/k heads (G > 1); compiled apart so that the
// ungrouped kernel carries none of the grouped record order's registers.
// GDT: storage type of beta and log alpha (float or __bf16; widened to fp32
// when they reach LDS).
template <int DK, int C, bool KDA, typename IT, bool GRP, typename GDT>
__global__ __launch_bounds__(256, C == 64 ? 2 : 3) void prep_kernel(PrepKArgs p) {
    using SM = PrepSmem<DK, C, KDA, IT>;
    using Rec = ChunkRec<DK, C, KDA, IT>;
    using ST = typename Prec<IT>::ST;
    using GT = typename Prec<IT>::GT;
    using FT = typename std::conditional<KDA, GT, ST>::type;   // Gram operand type
    using F8 = typename Frag8<FT>::type;
    constexpr bool SPLIT = Prec<IT>::SPLIT;
    constexpr int NB = SM::NB, NT = SM::NT;
    constexpr int EPV = 16 / sizeof(IT);
    using IV = typename VecT<IT, EPV>::type;
    constexpr int NSEG = 256 / DK;           // prefix-sum lanes per key channel
    constexpr int SEGL = C / NSEG;           //   tokens per lane
    constexpr int NSTEP = (DK + 31) / 32;    // 32-wide k-steps of the Gram
    constexpr bool WIDE = SM::WIDE;
    static_assert(NB <= 2 || (WIDE && sizeof(ST) == 2), "the inverse below handles two or four 16-token blocks (four: 16-bit operands)");
    static_assert(SEGL >= 1 && C <= 64, "prefix-sum thread mapping");
    static_assert(sizeof(Rec) == chunk_record_bytes(DK, C, KDA, sizeof(ST)), "record layout");
    static_assert(sizeof(SM) <= (sizeof(ST) == 2 ? (WIDE ? 80 : 64) : 160) * 1024, "LDS budget (fp16: two workgroups per CU)");
    static_assert(sizeof(ST) == 4 || (C % 32 == 0 && DK % 32 == 0), "fp16 operands are stored in 32-wide k-blocks");

    constexpr int KVPT = (C * DK / EPV + 255) / 256;        // 16-byte k (and q) vectors per thread
    constexpr int GVPT = KDA ? (C * DK / 4 + 255) / 256 : 1;  // 16-byte log-decay vectors per thread

    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int H = p.H;
    const IT *gq = static_cast<const IT *>(p.q);
    const IT *gk = static_cast<const IT *>(p.k);
    constexpr size_t RS = chunk_record_stride(DK, C, KDA, sizeof(ST));

    // Record L = (chunk slot x, head h), L = x * H + h; the G value heads
    // h = G j .. G j + G - 1 share q/k head j, so their records form group
    // L / G.  Workgroup b handles positions r = b, b + grid, ... (grid a
    // multiple of 8, so all on XCD b % 8).  Groups go round-robin over the 8
    // XCDs and a group's G records to positions r, r + 8, ..., so they run
    // side by side on one XCD and read their q/k once from HBM, then from
    // that XCD's L2 (with G = 1, position r holds record r).  locate gives the
    // record's index, first token and token count (0: no such chunk).
    // (Record counts stay below 2^31, which the host checks, so 32-bit
    // arithmetic suffices.)
    const int G = GRP ? p.G : 1;
    const long NP = GRP ? (p.num_records / G + 7) / 8 * 8 * G : p.num_records;
    auto record_at = [&](long r) -> long {       // num_records: no record
        if constexpr (!GRP) return r;
        if (r >= NP) return p.num_records;
        const unsigned slot = (unsigned)r / 8u;
        return (long)((slot / G * 8u + (unsigned)r % 8u) * G + slot % G);
    };
    auto locate = [&](long L, int &h, int &t0, int &nv) {
        h = (int)(L % H);
        const int x = (int)(L / H);
        nv = 0;
        t0 = 0;
        if (L >= p.num_records) return;
        int n, j;
        if (p.cu) {
            if (x >= p.choff[p.num_seqs]) return;
            int lo = 0, hi = p.num_seqs - 1;     // last n with choff[n] <= x
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (p.choff[mid] <= x) lo = mid;
                else hi = mid - 1;
            }
            n = lo;
            j = x - p.choff[n];
        } else {
            n = x / p.seg_chunks;
            j = p.j0 + x % p.seg_chunks;
        }
        const int bos = p.cu ? p.cu[n] : n * p.T;
        const int eos = p.cu ? p.cu[n + 1] : bos + p.T;
        t0 = bos + j * C;
        nv = min(C, eos - t0);
    };
    // the raw inputs of one record, held in registers while the previous
    // record is processed (zeros past the sequence end)
    IV kr[KVPT], qr[KVPT];
    using GV = typename std::conditional<std::is_same<GDT, float>::value, f32x4, bf16x4>::type;
    const GDT *gla = static_cast<const GDT *>(p.log_alpha);
    const GDT *gbeta = static_cast<const GDT *>(p.beta);
    GV gr[GVPT];
    float br = 0.f, gs = 0.f;
    auto fetch = [&](long r) {
        int h, t0, nv;
        locate(record_at(r), h, t0, nv);
#pragma unroll
        for (int x = 0; x < KVPT; ++x) {
            const int e = tid + 256 * x;
            const int t = e / (DK / EPV), c = (e % (DK / EPV)) * EPV;
            kr[x] = IV{};
            qr[x] = IV{};
            if (e < C * DK / EPV && t < nv) {
                const size_t off = ((size_t)(t0 + t) * p.HK + h / p.G) * DK + c;
                kr[x] = *reinterpret_cast<const IV *>(gk + off);
                qr[x] = *reinterpret_cast<const IV *>(gq + off);
            }
        }
        if constexpr (KDA) {
#pragma unroll
            for (int x = 0; x < GVPT; ++x) {
                const int e = tid + 256 * x;
                const int t = e / (DK / 4), c = (e % (DK / 4)) * 4;
                gr[x] = GV{};
                if (e < C * DK / 4 && t < nv)
                    gr[x] = *reinterpret_cast<const GV *>(gla + ((size_t)(t0 + t) * H + h) * DK + c);
            }
        } else {
            gs = tid < nv ? to_f32(gla[(size_t)(t0 + tid) * H + h]) : 0.f;
        }
        br = tid < nv ? to_f32(gbeta[(size_t)(t0 + tid) * H + h]) : 0.f;
    };

    // persistent workgroups: records blockIdx.x, + gridDim.x, ...; the next
    // record's inputs are requested as soon as this one's reach LDS
    long r = blockIdx.x;
    fetch(r);
    for (; r < NP; r += gridDim.x) {
    const long L = record_at(r);
    int h, t0, nv;
    locate(L, h, t0, nv);
    if (nv == 0) {                           // uniform: a chunk slot past the last sequence's end
        fetch(r + gridDim.x);
        continue;
    }
    Rec &rec = *reinterpret_cast<Rec *>(p.rec + (size_t)L * RS);

    // ---- A: inputs to LDS
#pragma unroll
    for (int x = 0; x < KVPT; ++x) {
        const int e = tid + 256 * x;
        if (e < C * DK / EPV) {
            const int t = e / (DK / EPV), c = (e % (DK / EPV)) * EPV;
            *reinterpret_cast<IV *>(&sm.u.in.Ks[t][c]) = kr[x];
            *reinterpret_cast<IV *>(&sm.u.in.Qs[t][c]) = qr[x];
        }
    }
    if constexpr (KDA) {
#pragma unroll
        for (int x = 0; x < GVPT; ++x) {
            const int e = tid + 256 * x;
            if (e < C * DK / 4) {
                const int t = e / (DK / 4), c = (e % (DK / 4)) * 4;
                f32x4 g4;
#pragma unroll
                for (int i = 0; i < 4; ++i) g4[i] = to_f32(gr[x][i]);
                *reinterpret_cast<f32x4 *>(&sm.u.in.G[t][c]) = g4;
            }
        }
    } else if (wave == 0) {
        float g = gs;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(g, off);
            if (lane >= off) g += y;
        }
        const float gC = __shfl(g, C - 1);
        if (lane < C) {
            sm.g[lane] = g;
            sm.egc[lane] = __expf(gC - g);
            sm.egt[lane] = __expf(g);
        }
        if (lane < 4) rec.dec[lane] = lane == 0 ? __expf(gC) : 0.f;
    }
    if (tid < C) sm.beta[tid] = br;
    // (64-token chunks: the next record's inputs are requested once
    // the Gram tiles have left registers, which then have room for them;
    // requesting its q and k here already spills and was measured slower)
    constexpr bool LATE_FETCH = WIDE;
    if constexpr (!LATE_FETCH) fetch(r + gridDim.x);
    __syncthreads();

    // ---- B: per-channel prefix sums (KDA), K_end^T to the record and
    // (K e^g)^T to LDS, one key channel per NSEG lanes, SEGL tokens each
    // (WIDE: (K e^g)^T is formed in C below instead)
    const int gc = tid / NSEG, gseg = tid % NSEG;
    {
        float ke[SEGL], kt[SEGL];
        if constexpr (KDA) {
            float gv[SEGL];
#pragma unroll
            for (int s = 0; s < SEGL; ++s) gv[s] = sm.u.in.G[gseg * SEGL + s][gc];
#pragma unroll
            for (int s = 1; s < SEGL; ++s) gv[s] += gv[s - 1];
            float incl = gv[SEGL - 1];
#pragma unroll
            for (int off = 1; off < NSEG; off <<= 1) {
                const float y = __shfl_up(incl, off, NSEG);
                if (gseg >= off) incl += y;
            }
            const float carry = incl - gv[SEGL - 1];
            const float gC = __shfl(incl, NSEG - 1, NSEG);
            const float g0 = __shfl(gv[0], 0, NSEG);
            const float m = 0.5f * (g0 + gC);
#pragma unroll
            for (int s = 0; s < SEGL; ++s) {
                const int t = gseg * SEGL + s;
                const float g = gv[s] + carry;
                sm.u.in.G[t][gc] = g - m;
                const float kv = (float)sm.u.in.Ks[t][gc];
                ke[s] = kv * __expf(gC - g);
                if constexpr (!WIDE) kt[s] = kv * __expf(g);
            }
            if (gseg == 0) {
                sm.em[gc] = __expf(m);
                rec.dec[gc] = __expf(gC);
            }
        } else {
#pragma unroll
            for (int s = 0; s < SEGL; ++s) {
                const int t = gseg * SEGL + s;
                const float kv = (float)sm.u.in.Ks[t][gc];
                ke[s] = kv * sm.egc[t];
                if constexpr (!WIDE) kt[s] = kv * sm.egt[t];
            }
        }
        if constexpr (SEGL % 4 == 0) {
#pragma unroll
            for (int s = 0; s < SEGL; s += 4) {
                const ST v4[4] = {(ST)ke[s], (ST)ke[s + 1], (ST)ke[s + 2], (ST)ke[s + 3]};
                store_vec<ST, 4>(&rec.KeT[gc][kpos<ST>(gseg * SEGL + s)], v4);
                if constexpr (!WIDE) {
                    const ST w4[4] = {(ST)kt[s], (ST)kt[s + 1], (ST)kt[s + 2], (ST)kt[s + 3]};
                    store_vec<ST, 4>(&sm.ktT[gc][kpos<ST>(gseg * SEGL + s)], w4);
                }
            }
        } else {
            static_assert(!WIDE, "64-token chunks take the vector path");
#pragma unroll
            for (int s = 0; s < SEGL; ++s) {
                rec.KeT[gc][kpos<ST>(gseg * SEGL + s)] = (ST)ke[s];
                sm.ktT[gc][kpos<ST>(gseg * SEGL + s)] = (ST)kt[s];
            }
        }
    }
    __syncthreads();

    // ---- C: decayed operands and partial Gram tiles; wave w takes k-steps w, w+4, ...
    f32x4 accA[NT], accM[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) accA[t] = accM[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // (16-bit operands: the two halves hh of a lane's eight channels are
    // adjacent in the stored k-order, so they leave as one 16-byte store)
    constexpr bool QT_MERGE = sizeof(ST) == 2 && DK >= 32;
    for (int s = wave; s < NSTEP; s += 4) {
        F8 fk[NB], fq[NB], fql[NB], fr[NB], frl[NB];
        // the Gram tile (I, J) of this k-step
        auto tile_mma = [&](int I, int J) {
            const int tt = I * (I + 1) / 2 + J;
            if constexpr (KDA) {
                accA[tt] = gram_mma(accA[tt], fk[I], fr[J]);
                accM[tt] = gram_mma(accM[tt], fq[I], fr[J]);
                if constexpr (SPLIT) {
                    accM[tt] = gram_mma(accM[tt], fq[I], frl[J]);
                    accM[tt] = gram_mma(accM[tt], fql[I], fr[J]);
                }
            } else {
                accA[tt] = gram_mma(accA[tt], fk[I], fk[J]);
                accM[tt] = gram_mma(accM[tt], fq[I], fk[J]);
            }
        };
        // WIDE: (K e^g)^T of this k-step's 32 channels, for the W product.
        // Only this wave reads these channels' columns of the staged q, so
        // once a pair of row blocks is done their q columns take the values:
        // piece (channel j, kpos group 4 s' + g) of (K e^g)^T goes to q row
        // 32 s' + j, columns 32 s + 8 g .. + 7 (the W product reads it back).
        ST ktp[2][8];
        ST *const qcols = reinterpret_cast<ST *>(&sm.u.in.Qs[0][0]) + 32 * s;
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
            const int t = 16 * rb + lr;
            ST qt8[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int ch = 32 * s + 16 * hh + 4 * lg;
                const bool valid = ch < DK;      // false only for DK = 16, second half
                float kf[4], qf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    kf[i] = valid ? (float)sm.u.in.Ks[t][ch + i] : 0.f;
                    qf[i] = valid ? (float)sm.u.in.Qs[t][ch + i] : 0.f;
                }
                ST qt[4];
                if constexpr (KDA) {
                    f32x4 xv{0.f, 0.f, 0.f, 0.f}, emv{0.f, 0.f, 0.f, 0.f};
                    if (valid) {
                        xv = *reinterpret_cast<const f32x4 *>(&sm.u.in.G[t][ch]);
                        emv = *reinterpret_cast<const f32x4 *>(&sm.em[ch]);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float e1 = __expf(xv[i]), e2 = __expf(-xv[i]);
                        const float lk = kf[i] * e1, lq = qf[i] * e1, rk = kf[i] * e2;
                        fk[rb][4 * hh + i] = (FT)lk;
                        const FT qh = (FT)lq, rh = (FT)rk;
                        fq[rb][4 * hh + i] = qh;
                        fr[rb][4 * hh + i] = rh;
                        fql[rb][4 * hh + i] = (FT)(lq - (float)qh);
                        frl[rb][4 * hh + i] = (FT)(rk - (float)rh);
                        qt[i] = (ST)(lq * emv[i] * p.scale);
                        if constexpr (WIDE) ktp[rb & 1][4 * hh + i] = (ST)(lk * emv[i]);
                    }
                } else {
                    // raw k, q for the Gram (the decay scales its fp32 result);
                    // k e^g, q e^g for the state-side products
                    const float e = sm.egt[t];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        fk[rb][4 * hh + i] = (ST)kf[i];
                        fq[rb][4 * hh + i] = (ST)qf[i];
                        qt[i] = (ST)(qf[i] * e * p.scale);
                        if constexpr (WIDE) ktp[rb & 1][4 * hh + i] = (ST)(kf[i] * e);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) qt8[4 * hh + i] = qt[i];
                if (!QT_MERGE && valid) store_vec<ST, 4>(&rec.Qt[t][kpos<ST>(ch)], qt);
            }
            if constexpr (QT_MERGE) store_vec<ST, 8>(&rec.Qt[t][kpos<ST>(32 * s + 4 * lg)], qt8);
            // WIDE: the tiles of row block rb as soon as its operands exist,
            // so only the column operands stay live across row blocks
            if constexpr (WIDE) {
#pragma unroll
                for (int J = 0; J <= rb; ++J) tile_mma(rb, J);
                if (rb & 1) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                qcols[(32 * (rb >> 1) + 16 * hh + 4 * lg + i) * SM::LDI + 8 * (lr >> 2) + 4 * h + (lr & 3)] =
                                    ktp[h][4 * hh + i];
                }
            }
        }
        if constexpr (!WIDE) {
#pragma unroll
            for (int I = 0; I < NB; ++I)
#pragma unroll
                for (int J = 0; J <= I; ++J) tile_mma(I, J);
        }
    }
    __syncthreads();   // the partial tiles overwrite the staged inputs
    if constexpr (WIDE) {
        // waves 2, 3 store their partial tiles as copies 0, 1; then waves
        // 0, 1 add theirs in place
        if (wave >= 2) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sm.u.Pt[wave - 2][t][4 * lg + i][lr] = accA[t][i];
                    sm.u.Pt[wave - 2][NT + t][4 * lg + i][lr] = accM[t][i];
                }
        }
        __syncthreads();
        if (wave < 2) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sm.u.Pt[wave][t][4 * lg + i][lr] += accA[t][i];
                    sm.u.Pt[wave][NT + t][4 * lg + i][lr] += accM[t][i];
                }
        }
        if constexpr (LATE_FETCH) fetch(r + gridDim.x);
    } else {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sm.u.Pt[wave][t][4 * lg + i][lr] = accA[t][i];
                sm.u.Pt[wave][NT + t][4 * lg + i][lr] = accM[t][i];
            }
    }
    __syncthreads();

    // ---- D: sum the partial tiles; masks, beta and (GDN) the decay factors.
    // (16-bit operands, C = 32: a thread takes columns c0 and c0 + 16, which
    // are adjacent in the stored k-order, and stores both at once.)
    constexpr int MH = (sizeof(ST) == 2 && C == 32) ? 2 : 1;   // column halves per thread
    for (int e = tid; e < C * C / (4 * MH); e += 256) {
        const int R = e / (C / (4 * MH)), cb0 = (e % (C / (4 * MH))) * 4;
        ST mv[4 * MH];
#pragma unroll
        for (int hf = 0; hf < MH; ++hf) {
            const int c0 = cb0 + 16 * hf;
            const int I = R >> 4, J = c0 >> 4, r = R & 15, cc = c0 & 15;
            f32x4 a{0.f, 0.f, 0.f, 0.f}, m{0.f, 0.f, 0.f, 0.f};
            if (J <= I) {
                const int tt = I * (I + 1) / 2 + J;
#pragma unroll
                for (int w = 0; w < SM::NCOPY; ++w) {
                    a += *reinterpret_cast<const f32x4 *>(&sm.u.Pt[w][tt][r][cc]);
                    m += *reinterpret_cast<const f32x4 *>(&sm.u.Pt[w][NT + tt][r][cc]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = c0 + i;
                float fa = c < R ? a[i] * sm.beta[R] : 0.f;
                float fm = c <= R ? m[i] : 0.f;
                if constexpr (!KDA) {
                    const float d = c <= R ? __expf(sm.g[R] - sm.g[c]) : 0.f;
                    fa *= d;
                    fm *= d;
                }
                if (J <= I) sm.a_tile(I * (I + 1) / 2 + J)[r * 20 + cc + i] = fa;
                mv[4 * hf + i] = (ST)(fm * p.scale);
            }
        }
        store_vec<ST, 4 * MH>(&rec.Mm[R][kpos<ST>(cb0)], mv);
    }
    __syncthreads();
    // T = (I + A)^-1.  On wave 0: the diagonal 16x16 blocks by forward
    // substitution, one column per lane (lanes 16 I .. 16 I + 15 block I; for
    // two blocks the upper half wave repeats the lower): t_i = delta_ij -
    // sum_{m<i} A_im t_m, with the block's strictly lower triangle read into
    // registers first (all lanes of a block read the same rows).  Then the
    // first subdiagonal block of each 32-token half, T_{I+1,I} =
    // -T_{I+1,I+1} (A_{I+1,I} T_II), as two fp32 MFMA products on the same
    // wave: A_{I+1,I} T_II lands in the accumulator layout that the second
    // product takes as its B operand.  Four blocks (64-token chunks) add the
    // lower-left 32x32 block, -T_hi (A_lo,hi T_lo) in 32-token blocks, one
    // 16x16 tile per wave.
    float (*const Tf)[SM::LDA] = sm.tf();
    float (*const TfT)[SM::LDA] = sm.tft();
    if (wave == 0) {
        const int I = (lane >> 4) % NB, jc = lane & 15;
        const float *adiag = sm.a_tile(I * (I + 1) / 2 + I);
        float tcol[16];
        if constexpr (WIDE) {
            // (rows read as they are needed: the next record's inputs are
            // in flight in registers here)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc0 = (i == jc) ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
                for (int m4 = 0; m4 < i; m4 += 4) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&adiag[i * 20 + m4]);
#pragma unroll
                    for (int mm = 0; mm < 4; ++mm) {
                        const int m = m4 + mm;
                        if (m < i) {
                            if (m & 1) acc1 -= a4[mm] * tcol[m];
                            else acc0 -= a4[mm] * tcol[m];
                        }
                    }
                }
                tcol[i] = acc0 + acc1;
            }
        } else {
            f32x4 arow[16][4];
#pragma unroll
            for (int i = 1; i < 16; ++i)
#pragma unroll
                for (int m4 = 0; m4 < i; m4 += 4) arow[i][m4 / 4] = *reinterpret_cast<const f32x4 *>(&adiag[i * 20 + m4]);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc0 = (i == jc) ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) {
                    if (m & 1) acc1 -= arow[i][m / 4][m % 4] * tcol[m];
                    else acc0 -= arow[i][m / 4][m % 4] * tcol[m];
                }
                tcol[i] = acc0 + acc1;
            }
        }
        if (lane < 16 * NB) {
#pragma unroll
            for (int i = 0; i < 16; ++i) Tf[16 * I + i][16 * I + jc] = tcol[i];
#pragma unroll
            for (int i4 = 0; i4 < 16; i4 += 4)
                *reinterpret_cast<f32x4 *>(&TfT[16 * I + jc][16 * I + i4]) =
                    f32x4{tcol[i4], tcol[i4 + 1], tcol[i4 + 2], tcol[i4 + 3]};
        }
        // (this wave's LDS writes above are visible to its reads below:
        // one wave's LDS operations execute in order)
#pragma unroll
        for (int I0 = 0; I0 + 1 < NB; I0 += 2) {
            const int I1 = I0 + 1;
            RowA<float, 1> a10, t00c, t11;
            a10.load(sm.a_tile(I1 * (I1 + 1) / 2 + I0) + lr * 20, lg);   // A_{I1,I0} rows
            t00c.load(&TfT[16 * I0 + lr][16 * I0], lg);                   // T_{I0,I0} columns
            const f32x4 P = rowa_mma(f32x4{0.f, 0.f, 0.f, 0.f}, a10, t00c, 0);
            RegB<float, 1> pb;
            pb.set(&P);
            t11.load(&Tf[16 * I1 + lr][16 * I1], lg);                     // T_{I1,I1} rows
            const f32x4 t10 = pb.mma(f32x4{0.f, 0.f, 0.f, 0.f}, t11);
#pragma unroll
            for (int i = 0; i < 4; ++i) Tf[16 * I1 + 4 * lg + i][16 * I0 + lr] = -t10[i];
        }
    }
    if constexpr (WIDE) {
        __syncthreads();
        // tile (i, j), i in {2, 3}, j in {0, 1}:  X_kj = sum_{m=j..1} A_km T_mj
        // for k = 2 .. i, then T_ij = -sum_{k=2..i} T_ik X_kj.  The
        // accumulator of X is the B operand of the second product (its rows
        // are that product's k-index).  The tiles read only T's diagonal
        // 32x32 blocks, which no wave writes here.
        const int i = 2 + (wave >> 1), j = wave & 1;
        auto mm_lds = [&](f32x4 acc, const float *A, int lda, const float *B, int ldb) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(A + lr * lda + 4 * lg);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], B[(4 * lg + r) * ldb + lr], acc, 0, 0, 0);
            return acc;
        };
        auto mm_reg = [&](f32x4 acc, const float *A, int lda, const f32x4 &X) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(A + lr * lda + 4 * lg);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], X[r], acc, 0, 0, 0);
            return acc;
        };
        auto xblk = [&](int k) {
            f32x4 x{0.f, 0.f, 0.f, 0.f};
            for (int m = j; m < 2; ++m) x = mm_lds(x, sm.a_tile(k * (k + 1) / 2 + m), 20, &Tf[16 * m][16 * j], SM::LDA);
            return x;
        };
        f32x4 t = mm_reg(f32x4{0.f, 0.f, 0.f, 0.f}, &Tf[16 * i][32], SM::LDA, xblk(2));
        if (i == 3) t = mm_reg(t, &Tf[48][48], SM::LDA, xblk(3));
#pragma unroll
        for (int r = 0; r < 4; ++r) Tf[16 * i + 4 * lg + r][16 * j + lr] = -t[r];
    }
    __syncthreads();
    // ---- E: T diag(b) and W = T diag(b) (K e^g), both to the record.  The
    // B operand of the W product is T diag(b) itself (rows: output token,
    // k: token), built per lane from T and b as the rounded values the
    // record stores; those lane fragments are 16-byte pieces of the record's
    // T diag(b) rows.  Each W tile is W^T for (16 keys, 16 tokens), so a
    // lane's four results are adjacent keys of one token.
    {
        RowA<ST, NB> tbf[NB];
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            const int row = 16 * tb + lr;
            tbf[tb] = tbeta_fragment<ST, NB>(&Tf[row][0], sm.beta, row, lg);
            if (wave == tb) tbf[tb].store(&rec.Tm[row][0], lg);
        }
        // Key blocks of every token block: 16-bit operands, the adjacent
        // pairs (2p, 2p + 1) for p = wave, wave + 4, ..., whose results are
        // adjacent in the stored k-order and leave as one 16-byte store;
        // fp32 operands, blocks kb = wave, wave + 4, ...
        constexpr int KP = sizeof(ST) == 2 ? 2 : 1;   // key blocks per store
        // WIDE: this wave's key-block pair is the k-step it took in C, whose
        // (K e^g)^T pieces sit in its columns of the staged q
        static_assert(!WIDE || DK / (16 * KP) <= 4, "at most one key-block pair per wave");
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
#pragma unroll
        for (int j = 0; j < (DK / (16 * KP) + 3) / 4; ++j) {
            const int pb = wave + 4 * j;
            if (pb < DK / (16 * KP)) {
                ST w[4 * KP];
#pragma unroll
                for (int x = 0; x < KP; ++x) {
                    const int kb = KP * pb + x;
                    RowA<ST, NB> a;
                    if constexpr (WIDE) {
                        const ST *qc = reinterpret_cast<const ST *>(&sm.u.in.Qs[0][0]) + 32 * wave + 8 * lg;
#pragma unroll
                        for (int st = 0; st < NB / 2; ++st)
                            a.f[st] = *reinterpret_cast<const f16x8 *>(qc + (32 * st + 16 * x + lr) * SM::LDI);
                    } else {
                        a.load(&sm.ktT[16 * kb + lr][0], lg);
                    }
                    f32x4 acc{0.f, 0.f, 0.f, 0.f};
                    // (k-steps past the diagonal of T's row block tb are zero)
#pragma unroll
                    for (int st = 0; st < RegB<ST, NB>::STEPS; ++st)
                        if (32 * st < 16 * tb + 16) acc = rowa_mma(acc, a, tbf[tb], st);
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[4 * x + i] = (ST)(-acc[i]);
                }
                store_vec<ST, 4 * KP>(&rec.Wn[16 * tb + lr][kpos<ST>(16 * KP * pb + 4 * lg)], w);
            }
        }
    }
    __syncthreads();   // the next record's inputs overwrite this one's scratch
    }
}

// ============================ chain kernel ===================================
// Swizzle of an unpadded LDS row of G 16-byte groups: row r stores logical
// group c at position c ^ row_swizzle(G, r).  Rows r and r + 32/G fall on the
// same banks; the XOR moves the two groups a lane pair reads onto distinct
// banks for 16 consecutive rows (the same rule as lds_pitch, for rows that
// cannot be padded because they are filled by whole-wave LDS-direct loads).
// Periodic in r with period 16.
__host__ __device__ constexpr int row_swizzle(int G, int r) { return G >= 4 ? 2 * ((r / (32 / G)) % (G / 2)) : 0; }

// Loader waves of the chain kernel: kRecordWaves copy records into LDS with
// LDS-direct loads, one more wave carries the value slice through registers.
constexpr int kRecordWaves = 3;
constexpr int kLoaderWaves = kRecordWaves + 1;

template <int DK, int DVS, int C, bool KDA, typename IT>
struct alignas(16) ChainSlot {
    using ST = typename Prec<IT>::ST;
    using Rec = ChunkRec<DK, C, KDA, IT>;
    static constexpr int NPIECE = (int)sizeof(Rec) / 16;
    // record bytes rounded up to whole rounds of the record waves' 1 KB loads
    static constexpr int RPIECES = (NPIECE + 64 * kRecordWaves - 1) / (64 * kRecordWaves) * (64 * kRecordWaves);
    static constexpr int LDVT = lds_pitch(C * (int)sizeof(ST)) / (int)sizeof(ST);
    union {
        Rec r;                          // the record, each row swizzled (row_swizzle)
        char raw[16 * RPIECES];
    } rec;
    ST Vt[DVS][LDVT];                   // value slice as an MFMA operand: value rows, tokens in kpos order
};

// 64-token chunks: a whole record per slot leaves room for only two slots,
// i.e. one chunk of lead for its fetch.  So a slot is split into the fields a
// chain wave reads before the chunk's mid-point barrier (part A: the decay row,
// T diag(b), W_n, Q e^g) and after it (part B: K_end^T, M), and each part is
// refilled as soon as the chain is done with it.  Rows are swizzled as in
// ChainSlot; each part is padded to whole rounds of the record waves' loads.
template <int DK, int DVS, int C, bool KDA, typename IT>
struct alignas(16) ChainSlot64 {
    using ST = typename Prec<IT>::ST;
    struct PartA {
        float dec[KDA ? DK : 4];
        ST Tm[C][C];
        ST Wn[C][DK];
        ST Qt[C][DK];
    };
    struct PartB {
        ST KeT[DK][C];
        ST Mm[C][C];
    };
    static constexpr int ROUND = 64 * kRecordWaves;
    static constexpr int APIECES = ((int)sizeof(PartA) / 16 + ROUND - 1) / ROUND * ROUND;
    static constexpr int BPIECES = ((int)sizeof(PartB) / 16 + ROUND - 1) / ROUND * ROUND;
    static constexpr int RPIECES = APIECES + BPIECES;
    static constexpr int LDVT = lds_pitch(C * (int)sizeof(ST)) / (int)sizeof(ST);
    union {
        PartA r;
        char raw[16 * APIECES];
    } a;
    union {
        PartB r;
        char raw[16 * BPIECES];
    } b;
    ST Vt[DVS][LDVT];
};

// Global record piece (plain ChunkRec layout) held by 16-byte position q of
// part A (PB = false) or part B of a ChainSlot64 (past the part: piece 0).
template <int DK, int C, bool KDA, typename IT>
__device__ __forceinline__ int rec64_piece_at(bool PB, int q) {
    using ST = typename Prec<IT>::ST;
    constexpr int PD = (KDA ? DK : 4) * 4 / 16;
    constexpr int GK = DK * (int)sizeof(ST) / 16, GC = C * (int)sizeof(ST) / 16;
    constexpr int WN = PD, QT = WN + C * GK, KE = QT + C * GK, TM = KE + DK * GC, MM = TM + C * GC;
    auto row = [](int base, int G, int x) {
        const int r = x / G, g = x % G;
        return base + r * G + (g ^ row_swizzle(G, r));
    };
    if (!PB) {
        if (q < PD) return q;
        q -= PD;
        if (q < C * GC) return row(TM, GC, q);
        q -= C * GC;
        if (q < C * GK) return row(WN, GK, q);
        q -= C * GK;
        if (q < C * GK) return row(QT, GK, q);
        return 0;
    }
    if (q < DK * GC) return row(KE, GC, q);
    q -= DK * GC;
    if (q < C * GC) return row(MM, GC, q);
    return 0;
}

// The record piece held by 16-byte position q of a slot's record area (past
// the record: any valid piece).  The decay row is stored plainly; the rows of
// Wn, Qt (G = DK groups) and KeT, Tm, Mm (G = C groups) are swizzled.
template <int DK, int C, bool KDA, typename IT>
__device__ __forceinline__ int rec_piece_at(int q) {
    using ST = typename Prec<IT>::ST;
    constexpr int PD = (KDA ? DK : 4) * 4 / 16;
    constexpr int GK = DK * (int)sizeof(ST) / 16, GC = C * (int)sizeof(ST) / 16;
    constexpr int NP = (int)sizeof(ChunkRec<DK, C, KDA, IT>) / 16;
    if (q >= NP) return NP - 1;
    if (q < PD) return q;
    q -= PD;
    if (q < 2 * C * GK) {
        const int r = q / GK, g = q % GK;
        return PD + r * GK + (g ^ row_swizzle(GK, r));
    }
    q -= 2 * C * GK;
    const int r = q / GC, g = q % GC;
    return PD + 2 * C * GK + r * GC + (g ^ row_swizzle(GC, r));
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds + 16 l (lds uniform across the wave).  Completion is counted by
// vmcnt like any load.  (The builtin exists only in the device pass; the host
// pass, which compiles just the kernel's launch stub, never runs it.)
__device__ __forceinline__ void lds_direct_load16(const void *src, void *lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
#else
    (void)src;
    (void)lds;
#endif
}


struct ChainKArgs {
    int T, H, DV, num_seqs;
    int j0, seg_chunks;          // dense: chunks [j0, j0 + seg_chunks) of every sequence
    const void *v;
    const float *state_in;       // state entering chunk j0 (NULL: zeros)
    const int32_t *cu, *order, *choff;
    const char *rec;
    void *out;
    float *state_out;            // state after the last chunk processed (NULL: not written)
};

template <int DK, int DVS, int C, bool KDA, typename IT, bool OUTB>
__global__ __launch_bounds__(64 * (kLoaderWaves + DVS / 16)) void chain_kernel(ChainKArgs p) {
    constexpr int NB = C / 16;                     // 16-token blocks per chunk
    using Slot = typename std::conditional<NB == 4, ChainSlot64<DK, DVS, C, KDA, IT>, ChainSlot<DK, DVS, C, KDA, IT>>::type;
    using Rec = ChunkRec<DK, C, KDA, IT>;
    using ST = typename Prec<IT>::ST;
    constexpr bool SPLIT = Prec<IT>::SPLIT;
    constexpr int NLW = kLoaderWaves;
    constexpr int NKB = DK / 16;                   // 16-channel key blocks
    constexpr int EPV = 16 / sizeof(IT);
    using IV = typename VecT<IT, EPV>::type;
    constexpr int NRW = kRecordWaves;
    constexpr int RX = Slot::RPIECES / (64 * NRW);  // LDS-direct loads per record-wave lane per chunk
    constexpr int VV = C * (DVS / EPV);            // 16-byte value vectors per chunk
    // LDS slots: the chain reads one while the loaders fill the next NSLOT - 1
    // (64-token chunks: two split slots, whatever fits; see ChainSlot64)
    constexpr int NSLOT = NB == 4 ? 2 : std::min<int>(4, (int)((160 * 1024) / sizeof(Slot)));
    constexpr int GK = DK * (int)sizeof(ST) / 16, GC = C * (int)sizeof(ST) / 16;
    constexpr size_t RS = chunk_record_stride(DK, C, KDA, sizeof(ST));
    static_assert(sizeof(Rec) % 16 == 0, "record pieces");
    static_assert(GK <= 32 && GC <= 32, "row swizzle covers rows of up to 32 groups");
    static_assert(VV % 64 == 0, "whole value vectors per lane of the value wave");
    static_assert(NSLOT >= 2, "LDS budget");
    static_assert(NB <= 2 || (NB == 4 && sizeof(ST) == 2), "16 or 32 tokens per chunk; 64 with 16-bit operands");
    // 32-wide k-steps of the lower-triangular T and M rows of row block rb
    auto tri_steps = [](int rb) { return (16 * rb + 16 + 31) / 32; };

    __shared__ Slot slot0, slot1, slot2, slot3;
    auto slot = [&](int i) -> Slot & {
        if constexpr (NSLOT > 3) if (i == 3) return slot3;
        if constexpr (NSLOT > 2) if (i == 2) return slot2;
        return i == 1 ? slot1 : slot0;
    };
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index in a scalar register: the chain / loader split below is a
    // uniform branch, so each wave executes only its own path's barriers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int H = p.H, DV = p.DV;

    // ---- block -> (sequence, head, value slice); the slices of one
    // (sequence, head) share blockIdx % 8, i.e. one XCD and its L2, where
    // their common records meet.
    const int NS = DV / DVS;
    const int xcd = blockIdx.x & 7, qd = blockIdx.x >> 3;
    const int urank = (qd / NS) * 8 + xcd, slice = qd % NS;
    if (urank >= p.num_seqs * H) return;
    const int srank = urank / H, h = urank % H;
    const int n = p.order ? p.order[srank] : srank;
    int bos, eos, rbase;
    if (p.cu) { bos = p.cu[n]; eos = p.cu[n + 1]; rbase = p.choff[n]; }
    else { bos = n * p.T; eos = bos + p.T; rbase = n * p.seg_chunks; }
    const int v0 = slice * DVS;
    const int nall = (eos - bos + C - 1) / C;
    const int nchunks = p.cu ? nall : max(0, min(nall - p.j0, p.seg_chunks));
    bos += p.j0 * C;                                         // first token of this launch's chunks
    const char *rec0 = p.rec + ((size_t)rbase * H + h) * RS;   // its chunk i at rec0 + i * H * RS

    if (wave >= NLW) {
        // =================== chain wave: 16 value channels ===================
        const int cb = wave - NLW;
        // the chain is the serial critical path: let it win issue arbitration
        // against loader waves and co-resident prep workgroups
        __builtin_amdgcn_s_setprio(2);
        // S^T of this wave's value block (lane: value column v0 + 16 cb + lr,
        // key rows 16 kb + 4 lg + i)
        f32x4 St[NKB];
        const size_t srow = ((size_t)n * H + h) * DV * DK + (size_t)(v0 + 16 * cb + lr) * DK + 4 * lg;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            St[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (p.state_in) St[kb] = *reinterpret_cast<const f32x4 *>(p.state_in + srow + 16 * kb);
        }
        using OT = typename std::conditional<OUTB, __bf16, float>::type;
        // outputs of a chunk: buffer stores from the chunk's first output
        // element (a uniform base) at fixed per-lane byte offsets (row
        // 16 rb + 4 lg + i, column lr); the buffer's size ends after the
        // chunk's last token, so rows past the sequence are dropped by the
        // range check.  Non-temporal, so they do not push the records the
        // value slices share out of L2.
        const int HDV = H * DV;
        int oofs[NB][4];
#pragma unroll
        for (int rb = 0; rb < NB; ++rb)
#pragma unroll
            for (int i = 0; i < 4; ++i) oofs[rb][i] = ((16 * rb + 4 * lg + i) * HDV + lr) * (int)sizeof(OT);
        const int swK = row_swizzle(GK, lr), swC = row_swizzle(GC, lr);
        lds_barrier();
        for (int jc = 0; jc < nchunks; ++jc) {
            const Slot &bs = slot(jc % NSLOT);
            const int t0 = bos + jc * C;
            const int nv = min(C, eos - t0);
            OT *ob = static_cast<OT *>(p.out) + ((size_t)t0 * H + h) * DV + v0 + 16 * cb;
            const __amdgpu_buffer_rsrc_t orsrc =
                __builtin_amdgcn_make_buffer_rsrc(ob, 0, ((nv - 1) * HDV + 16) * (int)sizeof(OT), kBufferWord3);
            f32x4 U[NB], Y[NB];
            if constexpr (NB == 4) {
            // 64-token chunks: too many operands to hold at once, so each
            // product's record rows are read just before it.  Part A of the
            // slot feeds U and Y, part B the state update and O; the barrier
            // between them lets the loaders refill part A.
            const auto &bc = bs.a.r;
            const auto &bcb = bs.b.r;
            {
                RowA<ST, NB> vb;
                vb.load(&bs.Vt[16 * cb + lr][0], lg);
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    RowA<ST, NB> ta;
                    ta.load(&bc.Tm[16 * rb + lr][0], lg, tri_steps(rb), swC);
                    U[rb] = Y[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < RegB<ST, NB>::STEPS; ++st)
                        if (st < tri_steps(rb)) U[rb] = rowa_mma(U[rb], ta, vb, st);
                }
            }
            RegB<ST, NKB> sop;
            sop.set(St);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                f32x4 d;
                if constexpr (KDA) d = *reinterpret_cast<const f32x4 *>(&bc.dec[16 * kb + 4 * lg]);
                else d = f32x4{bc.dec[0], bc.dec[0], bc.dec[0], bc.dec[0]};
#pragma unroll
                for (int i = 0; i < 4; ++i) St[kb][i] *= d[i];
            }
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                RowA<ST, NKB> wa;
                wa.load(&bc.Wn[16 * rb + lr][0], lg, 1 << 20, swK);
                U[rb] = sop.mma(U[rb], wa);
            }
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                RowA<ST, NKB> qa;
                qa.load(&bc.Qt[16 * rb + lr][0], lg, 1 << 20, swK);
                Y[rb] = sop.mma(Y[rb], qa);
            }
            RegB<ST, NB> uh, ul;
            uh.set_split(U, ul);
            lds_barrier();   // mid-chunk: part A is free
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                RowA<ST, NB> kea;
                kea.load(&bcb.KeT[16 * kb + lr][0], lg, 1 << 20, swC);
#pragma unroll
                for (int st = 0; st < RegB<ST, NB>::STEPS; ++st) St[kb] = uh.step(St[kb], kea, st);
#pragma unroll
                for (int st = 0; st < RegB<ST, NB>::STEPS; ++st) St[kb] = ul.step(St[kb], kea, st);
            }
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                RowA<ST, NB> ma;
                ma.load(&bcb.Mm[16 * rb + lr][0], lg, tri_steps(rb), swC);
#pragma unroll
                for (int st = 0; st < RegB<ST, NB>::STEPS; ++st)
                    if (st < tri_steps(rb)) Y[rb] = uh.step(Y[rb], ma, st);
#pragma unroll
                for (int st = 0; st < RegB<ST, NB>::STEPS; ++st)
                    if (st < tri_steps(rb)) Y[rb] = ul.step(Y[rb], ma, st);
            }
            } else {
            const Rec &bc = bs.rec.r;
            // every LDS operand of the chunk, issued up front in the order of use
            RowA<ST, NKB> wa[NB], qa[NB];
            RowA<ST, NB> ta[NB], vb;
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                ta[rb].load(&bc.Tm[16 * rb + lr][0], lg, tri_steps(rb), swC);
                wa[rb].load(&bc.Wn[16 * rb + lr][0], lg, 1 << 20, swK);
            }
            vb.load(&bs.Vt[16 * cb + lr][0], lg);
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) qa[rb].load(&bc.Qt[16 * rb + lr][0], lg, 1 << 20, swK);
            f32x4 dk[KDA ? NKB : 1];
            if constexpr (KDA) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) dk[kb] = *reinterpret_cast<const f32x4 *>(&bc.dec[16 * kb + 4 * lg]);
            } else {
                const float d = bc.dec[0];
                dk[0] = f32x4{d, d, d, d};
            }
            RowA<ST, NB> ma[NB], kea[NKB];
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) ma[rb].load(&bc.Mm[16 * rb + lr][0], lg, tri_steps(rb), swC);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) kea[kb].load(&bc.KeT[16 * kb + lr][0], lg, 1 << 20, swC);

            // U = T diag(b) V + W_neg S0^T: the state-independent part first
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                U[rb] = Y[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < RegB<ST, NB>::STEPS; ++st)
                    if (st < tri_steps(rb)) U[rb] = rowa_mma(U[rb], ta[rb], vb, st);
            }
            RegB<ST, NKB> sop;
            sop.set(St);
            // the decayed state S0 Diag(e^{g_C}), formed while the products run
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) St[kb][i] *= dk[KDA ? kb : 0][i];
            // the state-dependent part of U, then Y = (Q e^g) S0^T; NB
            // independent accumulations each, interleaved k-step by k-step
#pragma unroll
            for (int st = 0; st < RegB<ST, NKB>::STEPS; ++st)
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) U[rb] = sop.step(U[rb], wa[rb], st);
#pragma unroll
            for (int st = 0; st < RegB<ST, NKB>::STEPS; ++st)
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) Y[rb] = sop.step(Y[rb], qa[rb], st);
            RegB<ST, NB> uh, ul;
            uh.set_split(U, ul);
            // S^T <- Diag(e^{g_C}) S0^T + K_end^T U: hi products of every key
            // block, then lo
#pragma unroll
            for (int st = 0; st < RegB<ST, NB>::STEPS; ++st)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) St[kb] = uh.step(St[kb], kea[kb], st);
            if constexpr (SPLIT) {
#pragma unroll
                for (int st = 0; st < RegB<ST, NB>::STEPS; ++st)
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) St[kb] = ul.step(St[kb], kea[kb], st);
            }
            // O = Y + M U
#pragma unroll
            for (int st = 0; st < RegB<ST, NB>::STEPS; ++st)
#pragma unroll
                for (int rb = 0; rb < NB; ++rb)
                    if (st < tri_steps(rb)) Y[rb] = uh.step(Y[rb], ma[rb], st);
            if constexpr (SPLIT) {
#pragma unroll
                for (int st = 0; st < RegB<ST, NB>::STEPS; ++st)
#pragma unroll
                    for (int rb = 0; rb < NB; ++rb)
                        if (st < tri_steps(rb)) Y[rb] = ul.step(Y[rb], ma[rb], st);
            }
            }
#pragma unroll
            for (int rb = 0; rb < NB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) buffer_store_nt(orsrc, oofs[rb][i], (OT)Y[rb][i]);
            lds_barrier();
        }
        if (p.state_out) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                *reinterpret_cast<f32x4 *>(p.state_out + srow + 16 * kb) = St[kb];
        }
        return;
    }

    // ============================ loader waves ================================
    // Chunk c uses slot c % NSLOT; its loads are issued NSLOT - 1 chunks
    // ahead.  Every chunk issues the same loads, unconditionally (chunks past
    // the end reload the last one into a slot nobody reads; value rows past
    // the sequence are zeroed when written), so a wave's count of loads in
    // flight is fixed.  The two kinds of loader run on separate waves: a wave
    // whose code both writes LDS and has LDS-direct loads in flight would be
    // made to wait for all of them before each write.
    if (nchunks > 0 && wave < NRW && NB == 4) {
        if constexpr (NB == 4) {
        // ---- record waves, 64-token chunks: the slot's two parts are loaded
        // separately, in the order A(0) B(0) A(1) B(1) A(2) ...: part B of
        // chunk c + 1 once chunk c - 1 is done with that slot (its end
        // barrier), part A of chunk c + 2 once chunk c is done with part A
        // (its mid-point barrier).  Each barrier waits for the part the
        // chain reads next, with the two parts issued after it in flight.
        constexpr int XA = Slot::APIECES / (64 * NRW), XB = Slot::BPIECES / (64 * NRW);
        constexpr int PEND = XA + XB;
        static_assert(PEND < 64, "vmcnt range");
        int goa[XA], gob[XB];
#pragma unroll
        for (int x = 0; x < XA; ++x) goa[x] = 16 * rec64_piece_at<DK, C, KDA, IT>(false, 64 * (x * NRW + wave) + lane);
#pragma unroll
        for (int x = 0; x < XB; ++x) gob[x] = 16 * rec64_piece_at<DK, C, KDA, IT>(true, 64 * (x * NRW + wave) + lane);
        auto issue_a = [&](int c, int sl) {
            const char *src = rec0 + (size_t)min(c, nchunks - 1) * H * RS;
            char *dst = slot(sl).a.raw + 1024 * wave;
#pragma unroll
            for (int x = 0; x < XA; ++x) lds_direct_load16(src + goa[x], dst + 1024 * NRW * x);
        };
        auto issue_b = [&](int c, int sl) {
            const char *src = rec0 + (size_t)min(c, nchunks - 1) * H * RS;
            char *dst = slot(sl).b.raw + 1024 * wave;
#pragma unroll
            for (int x = 0; x < XB; ++x) lds_direct_load16(src + gob[x], dst + 1024 * NRW * x);
        };
        // every part but the two issued last has landed
        auto wait_pend = [&]() { __builtin_amdgcn_s_waitcnt((PEND & 15) | ((PEND >> 4) << 14) | (7 << 4) | (15 << 8)); };
        issue_a(0, 0);
        issue_b(0, 0);
        issue_a(1, 1);
        wait_pend();       // A(0)
        lds_barrier();
        for (int c = 0; c < nchunks; ++c) {
            const int sl = c & 1;
            issue_b(c + 1, sl ^ 1);
            wait_pend();   // B(c)
            lds_barrier();                 // chunk c: mid-point
            issue_a(c + 2, sl);
            wait_pend();   // A(c + 1)
            lds_barrier();                 // chunk c: end
        }
        // no LDS-direct write may land after the workgroup's LDS is released
        __builtin_amdgcn_s_waitcnt(0);
        }
    } else if (nchunks > 0 && wave < NRW) {
        if constexpr (NB != 4) {
        // ---- record waves: global -> LDS directly, no registers.  Load x of
        // wave w fills the slot's record bytes [1 KB (x NRW + w), +1 KB), lane
        // l the 16-byte position q = 64 (x NRW + w) + l, which holds the
        // record piece rec_piece_at(q).
        int goff[RX];
#pragma unroll
        for (int x = 0; x < RX; ++x) goff[x] = 16 * rec_piece_at<DK, C, KDA, IT>(64 * (x * NRW + wave) + lane);
        auto issue = [&](int c, int sl) {
            const char *src = rec0 + (size_t)min(c, nchunks - 1) * H * RS;
            char *dst = slot(sl).rec.raw + 1024 * wave;
#pragma unroll
            for (int x = 0; x < RX; ++x) lds_direct_load16(src + goff[x], dst + 1024 * NRW * x);
        };
        // chunk c + 1 has landed while the NSLOT - 2 chunks after it stay in
        // flight (loads complete in issue order)
        constexpr int AFTER = (NSLOT - 2) * RX;
        static_assert(AFTER < 64, "vmcnt range");
        auto wait_next = [&]() { __builtin_amdgcn_s_waitcnt((AFTER & 15) | ((AFTER >> 4) << 14) | (7 << 4) | (15 << 8)); };
#pragma unroll
        for (int c = 0; c < NSLOT - 1; ++c) issue(c, c);
        wait_next();   // chunk 0
        lds_barrier();
        for (int jb = 0; jb < nchunks; jb += NSLOT) {
#pragma unroll
            for (int u = 0; u < NSLOT; ++u) {
                if (jb + u < nchunks) {
                    issue(jb + u + NSLOT - 1, (u + NSLOT - 1) % NSLOT);   // the slot chunk jb + u - 1 used
                    wait_next();                                        // chunk jb + u + 1
                    lds_barrier();
                }
            }
        }
        // no LDS-direct write may land after the workgroup's LDS is released
        __builtin_amdgcn_s_waitcnt(0);
        }
    } else if (nchunks > 0) {
        // ---- value wave: the value slice through registers, written
        // transposed (value rows, tokens in kpos order) as the fp16 operand
        // VQ chunks in registers: the loads of chunk c + VQ - 1 are issued
        // while chunk c + 1 is written to its slot (with two slots, still
        // two chunks of lead)
        constexpr int VPL = VV / 64;
        constexpr int VQ = NSLOT < 3 ? 3 : NSLOT;
        constexpr int UNR = NSLOT % VQ == 0 ? NSLOT : VQ * NSLOT;   // a multiple of both
        static_assert(UNR % VQ == 0 && UNR % NSLOT == 0, "value ring unroll");
        const IT *gv = static_cast<const IT *>(p.v);
        IV vr[VQ][VPL];
        bool vok[VQ][VPL];
        auto issue = [&](int c, int sl) {
            const int cc = min(c, nchunks - 1);
#pragma unroll
            for (int y = 0; y < VPL; ++y) {
                const int e = lane + 64 * y, vt = e / (DVS / EPV), vc = (e % (DVS / EPV)) * EPV;
                const int t = bos + cc * C + vt;
                // (non-temporal: each slice reads its values once, and leaving
                // them out of L2 keeps the records the slices share there
                // longer: the chain's HBM fetch fell from 2.9-3.4 to 2.5 GB
                // per KDA 32K call)
                vr[sl][y] = __builtin_nontemporal_load(
                    reinterpret_cast<const IV *>(gv + ((size_t)min(t, eos - 1) * H + h) * DV + v0 + vc));
                vok[sl][y] = t < eos;
            }
        };
        using UT = typename std::conditional<sizeof(IT) == 2, unsigned short, unsigned>::type;
        auto commit = [&](int rq, int sl) {
#pragma unroll
            for (int y = 0; y < VPL; ++y) {
                const int e = lane + 64 * y, vt = e / (DVS / EPV), vc = (e % (DVS / EPV)) * EPV;
                const UT keep = vok[rq][y] ? UT(~UT(0)) : UT(0);   // rows past the sequence become +0
#pragma unroll
                for (int i = 0; i < EPV; ++i) {
                    // (element copied out first: a bit cast of a vector element
                    // in place reads element 0 with this compiler)
                    const IT el = vr[rq][y][i];
                    const IT x = __builtin_bit_cast(IT, UT(__builtin_bit_cast(UT, el) & keep));
                    slot(sl).Vt[vc + i][kpos<ST>(vt)] = (ST)(float)x;
                }
            }
        };
#pragma unroll
        for (int c = 0; c < VQ - 1; ++c) issue(c, c);
        commit(0, 0);
        lds_barrier();
        for (int jb = 0; jb < nchunks; jb += UNR) {
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int jc = jb + u;
                if (jc < nchunks) {
                    issue(jc + VQ - 1, (u + VQ - 1) % VQ);
                    if constexpr (NB == 4) lds_barrier();   // chunk jc: mid-point
                    if (jc + 1 < nchunks) commit((u + 1) % VQ, (u + 1) % NSLOT);
                    lds_barrier();
                }
            }
        }
    } else {
        lds_barrier();   // the chain waves' first barrier
    }
}

template <int DK, int C, bool KDA, typename IT>
hipError_t launch_prep(const PrefillArgs &a, int j0, int seg_chunks, char *rec, long record_chunks, hipStream_t st) {
    if (record_chunks <= 0) return hipSuccess;
    PrepKArgs pk;
    pk.T = a.seqlen;
    pk.H = a.num_heads;
    pk.HK = a.num_qk_heads;
    pk.G = a.num_heads / a.num_qk_heads;
    pk.num_seqs = a.num_seqs;
    pk.j0 = j0;
    pk.seg_chunks = seg_chunks;
    pk.scale = a.scale;
    pk.q = a.q; pk.k = a.k;
    pk.beta = a.beta; pk.log_alpha = a.log_alpha;
    pk.cu = a.cu_seqlens;
    pk.choff = a.chunk_offset;
    pk.rec = rec;
    pk.num_records = record_chunks * a.num_heads;
    // workgroups of this kernel that fit on the device at once (computed on
    // the first call; concurrent first calls compute the same value)
    static std::atomic<int> resident_cache{0};
    int resident = resident_cache.load(std::memory_order_relaxed);
    if (!resident) {
        int dev = 0, cus = 0, per_cu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e == hipSuccess)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, prep_kernel<DK, C, KDA, IT, false, float>, 256, 0);
        if (e != hipSuccess) return e;
        resident = std::max(1, cus * per_cu);
        resident_cache.store(resident, std::memory_order_relaxed);
    }
    // grouped: a multiple of 8 workgroups (8 XCDs) unless the device holds fewer
    const bool grp = pk.G > 1;
    const long grid = grp ? std::min<long>((pk.num_records / pk.G + 7) / 8 * 8 * pk.G, resident)
                          : std::min<long>(pk.num_records, resident);
#define GDR_PREP(GRP_, GT_) hipLaunchKernelGGL((prep_kernel<DK, C, KDA, IT, GRP_, GT_>), dim3((unsigned)grid), dim3(256), 0, st, pk)
    if (a.gate_bf16) {
        if (grp) GDR_PREP(true, __bf16);
        else GDR_PREP(false, __bf16);
    } else {
        if (grp) GDR_PREP(true, float);
        else GDR_PREP(false, float);
    }
#undef GDR_PREP
    return hipGetLastError();
}

template <int DK, int DVS, int C, bool KDA, typename IT>
hipError_t launch_chain(const PrefillArgs &a, int j0, int seg_chunks, const char *rec, const float *state_in,
                        float *state_out, hipStream_t st) {
    constexpr int threads = 64 * (kLoaderWaves + DVS / 16);
    ChainKArgs p;
    p.T = a.seqlen;
    p.H = a.num_heads;
    p.DV = a.dv;
    p.num_seqs = a.num_seqs;
    p.j0 = j0;
    p.seg_chunks = seg_chunks;
    p.v = a.v;
    p.state_in = state_in;
    p.cu = a.cu_seqlens;
    p.order = a.cu_seqlens ? a.order : nullptr;
    p.choff = a.chunk_offset;
    p.rec = rec;
    p.out = a.out;
    p.state_out = state_out;
    const long units = (long)a.num_seqs * a.num_heads;
    const long grid = ((units + 7) / 8) * 8 * (a.dv / DVS);
    if (a.out_bf16)
        hipLaunchKernelGGL((chain_kernel<DK, DVS, C, KDA, IT, true>), dim3((unsigned)grid), dim3(threads), 0, st, p);
    else
        hipLaunchKernelGGL((chain_kernel<DK, DVS, C, KDA, IT, false>), dim3((unsigned)grid), dim3(threads), 0, st, p);
    return hipGetLastError();
}

// One segment (the default): every record, then every chain.  When the
// caller's workspace holds fewer records, dense batches run in segments of
// chunks: records of one segment at a time, the state carried between
// segments in the workspace.  (Running a segment's records on a second stream
// beside the previous segment's chains was measured slower: the two kernels
// then compete for HBM and evict each other's records from L2.)
template <int DK, int DVS, int C, bool KDA, typename IT>
hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t st) {
    const int ncps = (a.seqlen + C - 1) / C;
    if (a.num_segments <= 1) {
        hipError_t e = launch_prep<DK, C, KDA, IT>(a, 0, ncps, a.records, a.record_chunks, st);
        if (e != hipSuccess) return e;
        return launch_chain<DK, DVS, C, KDA, IT>(a, 0, ncps, a.records, a.initial_state, a.final_state, st);
    }
    const int S = a.segment_chunks;
    for (int sgi = 0; sgi < a.num_segments; ++sgi) {
        const int j0 = sgi * S, cnt = min(S, ncps - j0);
        hipError_t e = launch_prep<DK, C, KDA, IT>(a, j0, cnt, a.records, (long)a.batch * cnt, st);
        if (e != hipSuccess) return e;
        const bool last = sgi == a.num_segments - 1;
        e = launch_chain<DK, DVS, C, KDA, IT>(a, j0, cnt, a.records, sgi == 0 ? a.initial_state : a.carry,
                                             last ? a.final_state : a.carry, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gdr
