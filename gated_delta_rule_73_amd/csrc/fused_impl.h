// fused_impl.h -- single-kernel chunked prefill of the gated delta rule for
// gfx950 (bf16 q/k/v, fp32 state, 64-token chunks).
//
// The recurrence (page "How the New Flash Models Work: Inside GLM-5.3-Flash
// and Qwen3.8-Flash-Next", section "Linear attention: a fixed-size memory in
// place of the cache"):  S_t = S_{t-1} Diag(a_t)(I - b_t k_t k_t^T) + b_t v_t k_t^T,
// o_t = S_t q_t, a scalar decay per head (Gated DeltaNet) or one per key
// channel (Kimi Delta Attention).  Chunked form, derived from that equation
// (the pages give no algorithm): for a chunk of C tokens entering with state
// S0 and in-chunk cumulative log decay g (per key channel),
//     A   = strict_tril(diag(b) (K e^g)(K e^-g)^T),   T = (I + A)^-1
//     W_n = -T diag(b) (K e^g)
//     U   = T diag(b) V + W_n S0^T
//     O   = (Q e^g) S0^T + M U,    M = tril((Q e^g)(K e^-g)^T)
//     S_C = S0 Diag(e^{g_C}) + U^T (K e^{g_C - g}).
// The scalar factor `scale` is folded into Q e^g and M.
//
// Work split.  Everything except U, O and S_C is independent of the state
// (a per-chunk "record": W_n, Q e^g, K_end^T = (K e^{g_C-g})^T, T diag(b), M,
// e^{g_C}), and every value slice of a (sequence, head) needs the same
// record.  One workgroup runs per (sequence, head, slice of DVS value
// channels); the NS slices of a unit form a group placed on one XCD
// (workgroups are dispatched round-robin over the 8 XCDs, so blockIdx % 8
// selects the XCD; the kernel checks this at start-up).  Slice s of a group
// builds the records of the chunks r with r % NS == s and publishes them in
// a ring of D record slots in global memory, small enough to stay in that
// XCD's L2; every slice copies each record into LDS and advances its state
// slice.  The record therefore never travels to HBM, and HBM carries only
// q, k, v, the gates, the outputs and the states.
//
// Roles inside a workgroup (no role ever waits on a barrier shared with
// another role, so a role blocked on another workgroup cannot stall the
// roles that other workgroups wait for):
//   * NCW = DVS / 16 chain waves: 16 value channels each, the state slice
//     held transposed (key rows x value columns) in fp32 MFMA accumulators.
//   * one loader wave: waits for record r in the ring, copies its LDS part
//     (e^{g_C}, W_n, K_end^T, T diag(b), M) into one of two LDS slots with
//     LDS-direct loads, and the value slice (transposed, fp16) beside it.
//   * NB = C / 16 prep waves, wave p owning the 16 tokens of row tile p for
//     every key channel: gate prefix sums (DPP scans across lanes), decayed
//     operands, the Gram products on MFMA, the inverse, W_n.
// Handshakes: loader -> chain: LDS word full[slot] = r + 1; chain -> loader:
// LDS counter done[slot]; prep waves among themselves: an LDS counter
// barrier; across workgroups: flag[ring slot] = r + 1 (producer -> every
// slice) and progress[slice] = records consumed (slice -> producers, who
// reuse a ring slot only once every slice has consumed its previous record).
// Cross-workgroup flags use agent-scope atomics; the ring data itself is
// written with plain stores and read with loads that miss in the CU's L1
// (sc1) and are served by the XCD's L2 the producer wrote to (when the
// start-up check finds a group spread over XCDs, the kernel adds agent-scope
// release/acquire fences around the flags, which write the L2 back to memory
// and invalidate the readers' L2 lines).
// Every wait is bounded: on a time-out the kernel raises an abort word that
// every wait polls, all roles leave their loops, and the affected final
// states are written as NaN.
//
// Precision: as the two-kernel prefill (prefill_impl.h): chain products on
// fp16 MFMA with U split into fp16 hi + lo; the per-channel-decay Gram M from
// bf16 hi + lo operands, A from single bf16 operands (Kimi Delta Attention);
// raw bf16 q/k with an exact fp32 decay mask (Gated DeltaNet); T in fp32.
// Kimi Delta Attention operands carry the decay around the per-channel
// midpoint m = (g_first + g_C) / 2 of the chunk.
#pragma once

#include <type_traits>

#include "prefill_impl.h"

namespace gdr {

constexpr int kFusedChunk = 64;
constexpr int kFusedSpin = 1 << 22;     // polls before a wait gives up (each poll sleeps ~64 cycles)

// ---- ring record: the LDS part first, then Q e^g (read from the ring) -----
template <int DK, int C, bool KDA>
struct FusedRecLds {
    float dec[KDA ? DK : 4];   // e^{g_C} per key channel (GDN: dec[0])
    _Float16 Wn[C][DK];        // key channel in kpos order
    _Float16 KeT[DK][C];       // token in kpos order
    _Float16 Tm[C][C];         // T diag(b), token (column) in kpos order, zero above the diagonal
    _Float16 Mm[C][C];         // M, zero above the diagonal
};
template <int DK, int C, bool KDA>
struct FusedRec : FusedRecLds<DK, C, KDA> {
    _Float16 Qt[C][DK];        // Q e^g scale, key channel in kpos order
};
template <int DK, int C, bool KDA>
constexpr int fused_lds_part() {
    return (int)sizeof(FusedRecLds<DK, C, KDA>);
}
template <int DK, int C, bool KDA>
constexpr size_t fused_rec_stride() { return (sizeof(FusedRec<DK, C, KDA>) + 255) & ~size_t(255); }

// per-workgroup global scratch of the prep waves: the right Gram operands of
// every row tile (two bf16 planes for KDA, raw k for GDN) and (K e^g)^T
template <int DK, int C, bool KDA>
struct FusedScratch {
    __bf16 rk[C / 16][KDA ? 2 : 1][16][DK];       // [tile][plane][token][key channel in kpos order]
    _Float16 KtT[DK][C];                          // token in kpos order
};
template <int DK, int C, bool KDA>
constexpr size_t fused_scratch_stride() { return (sizeof(FusedScratch<DK, C, KDA>) + 255) & ~size_t(255); }

// ---- LDS ------------------------------------------------------------------
template <int DK, int DVS, int C, bool KDA>
struct alignas(16) FusedSlot {
    static constexpr int LDSB = fused_lds_part<DK, C, KDA>();
    static constexpr int RAW = (LDSB + 1023) / 1024 * 1024;   // whole 1 KB rounds of the loader's copies
    static constexpr int LDVT = lds_pitch(C * 2) / 2;
    union {
        FusedRecLds<DK, C, KDA> r;
        char raw[RAW];
    } rec;
    _Float16 Vt[DVS][LDVT];       // value slice: value rows, tokens in kpos order
};

template <int DK, int DVS, int C, bool KDA>
struct FusedSmem {
    static constexpr int NB = C / 16, LDT = C + 4;
    FusedSlot<DK, DVS, C, KDA> slot[2];
    // prep scratch
    alignas(16) float At[C][LDT];    // A (strictly lower part)
    alignas(16) float Tt[C][LDT];    // T: lower part incl. diagonal; T^T mirrored into the upper part
    alignas(16) float tot[NB][KDA ? DK : 4];   // per-tile totals of the log-decay
    alignas(16) float gfirst[KDA ? DK : 4];    // log-decay of the chunk's first token
    alignas(16) float carry[NB][KDA ? DK : 4]; // KDA: log-decay before each tile
    alignas(16) float mid[KDA ? DK : 4], em[KDA ? DK : 4], ecm[KDA ? DK : 4];
    alignas(16) float beta[C], g[C];           // g: GDN cumulative log-decay per token
    // handshakes
    int full[2], done[2], pbar, local, abort;
};

struct FusedArgs {
    int T, H, HK, G, DV, num_seqs;
    int NS, D, ngroups, gpx;        // slices per group, ring depth, groups, groups per XCD
    float scale;
    bool gate_bf16, out_bf16;
    const void *q, *k, *v, *beta, *log_alpha;
    const float *state_in;
    float *state_out;
    const int32_t *cu, *order;
    char *ring, *scratch;
    int *ctl;                       // flags [ngroups][D], progress [ngroups][NS], xcc [ngroups][NS], abort
    void *out;
};

__device__ __forceinline__ int ld_agent(const int *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_agent(int *p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// A handshake word for readers on this XCD (local) or anywhere on the device.
// An agent-scope store writes through to memory (about a microsecond before
// it completes and before readers see it); within one XCD a plain store
// reaches the shared L2, where the readers' agent-scope loads (which miss in
// their CUs' L1) find it.
__device__ __forceinline__ void st_flag(int *p, int v, bool local) {
    if (local) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    else st_agent(p, v);
}
__device__ __forceinline__ int ld_lds(const int *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }
__device__ __forceinline__ void st_lds(int *p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }

// inclusive prefix sum across each row of 16 lanes (DPP row shifts; lanes
// shifted in from outside the row contribute 0)
template <int N>
__device__ __forceinline__ float dpp_row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 | N, 0xf, 0xf, false));
}
// sum over each row of 16 lanes, every lane of the row receiving it (DPP row rotations)
template <int N>
__device__ __forceinline__ float dpp_row_ror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 | N, 0xf, 0xf, false));
}
__device__ __forceinline__ float sum_row16(float x) {
    x += dpp_row_ror<8>(x);
    x += dpp_row_ror<4>(x);
    x += dpp_row_ror<2>(x);
    x += dpp_row_ror<1>(x);
    return x;
}
__device__ __forceinline__ float scan_row16(float x) {
    x += dpp_row_shr<1>(x);
    x += dpp_row_shr<2>(x);
    x += dpp_row_shr<4>(x);
    x += dpp_row_shr<8>(x);
    return x;
}

// Loads of data another workgroup wrote: the sc1 policy misses in the CU's
// L1 (a plain or sc0 load can return a line the L1 still holds from the
// slot's previous record; measured on gfx950: sc0 loads hit L1 like plain
// ones) and is served by the XCD's L2.
constexpr int kCoherentLoad = 16;   // sc1
__device__ __forceinline__ i32x4 ring_load16(__amdgpu_buffer_rsrc_t r, int ofs) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, ofs, 0, kCoherentLoad);
}
__device__ __forceinline__ void lds_direct_load16_coherent(const void *src, void *lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, kCoherentLoad);
#else
    (void)src;
    (void)lds;
#endif
}

// The unit (sequence n, value head h, token range) a group processes at its
// i-th turn; false once the group has none left.  Units are ranked by
// (sequence in `order`, q/k head, value head in its group); the value heads
// that share a q/k head go to one XCD, round-robin over the XCD's groups.
struct FusedUnit {
    int n, h, bos, eos, nch;
};
template <int CH = kFusedChunk>
__device__ __forceinline__ bool fused_unit(const FusedArgs &p, int g, int i, FusedUnit &u) {
    const int x = g & 7, gl = g >> 3;
    const int lam = i * p.gpx + gl;
    const int P = (lam / p.G) * 8 + x, j = lam % p.G;
    if (P >= p.num_seqs * p.HK) return false;
    const int sr = P / p.HK, hq = P % p.HK;
    u.n = p.order ? p.order[sr] : sr;
    u.h = hq * p.G + j;
    if (p.cu) {
        u.bos = p.cu[u.n];
        u.eos = p.cu[u.n + 1];
    } else {
        u.bos = u.n * p.T;
        u.eos = u.bos + p.T;
    }
    u.nch = (u.eos - u.bos + CH - 1) / CH;
    return true;
}

// the record piece held by 16-byte position q of a slot (rows swizzled with
// row_swizzle so the chain's A-fragment reads meet distinct banks); past the
// LDS part: any valid piece
template <int DK, int C, bool KDA>
__device__ __forceinline__ int fused_piece_at(int q) {
    constexpr int PD = (KDA ? DK : 4) * 4 / 16;
    constexpr int GK = DK * 2 / 16, GC = C * 2 / 16;
    constexpr int NP = fused_lds_part<DK, C, KDA>() / 16;
    if (q >= NP) return NP - 1;
    if (q < PD) return q;
    q -= PD;
    if (q < C * GK) {   // Wn rows
        const int r = q / GK, gg = q % GK;
        return PD + r * GK + (gg ^ row_swizzle(GK, r));
    }
    q -= C * GK;
    const int r = q / GC, gg = q % GC;   // KeT, Tm, Mm rows (GC groups each)
    return PD + C * GK + r * GC + (gg ^ row_swizzle(GC, r));
}

// bounded waits: true once `cond` holds; false on a time-out or an abort
// raised elsewhere (a time-out raises it)
template <class F>
__device__ __forceinline__ bool wait_until(F cond, int *abort_word) {
    for (int it = 0; it < kFusedSpin; ++it) {
        if (cond()) return true;
        if ((it & 63) == 63 && ld_agent(abort_word)) return false;
        __builtin_amdgcn_s_sleep(1);
    }
    st_agent(abort_word, 1);
    return false;
}

template <int DK, int DVS, int C, bool KDA>
__global__ __launch_bounds__(64 * (DVS / 16 + 1 + C / 16)) void fused_prefill_kernel(FusedArgs p) {
    using SM = FusedSmem<DK, DVS, C, KDA>;
    using Rec = FusedRec<DK, C, KDA>;
    using RecL = FusedRecLds<DK, C, KDA>;
    using Slot = FusedSlot<DK, DVS, C, KDA>;
    using Scr = FusedScratch<DK, C, KDA>;
    using ST = _Float16;
    constexpr int NCW = DVS / 16, NB = C / 16, NPW = NB;
    constexpr int NKB = DK / 16, NKS = DK / 32;
    constexpr int GK = DK * 2 / 16, GC = C * 2 / 16;
    constexpr size_t RS = fused_rec_stride<DK, C, KDA>();
    constexpr int LDSB = fused_lds_part<DK, C, KDA>();
    constexpr int RX = Slot::RAW / 1024;        // loader rounds per record
    static_assert(C == 64 && DK % 32 == 0 && DK <= 128, "shapes");
    static_assert(sizeof(SM) <= 160 * 1024, "LDS budget");
    static_assert(LDSB % 16 == 0, "record pieces");
    static_assert(GK <= 32 && GC <= 32, "row swizzle");
    static_assert(RS == fused_record_bytes(DK, KDA) && fused_scratch_stride<DK, C, KDA>() == fused_scratch_bytes(DK, KDA),
                  "the host's workspace layout (launch.h) matches the kernel's");

    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int H = p.H, DV = p.DV, NS = p.NS, D = p.D;

    // ---- block -> (group, slice); every slice of a group on XCD blockIdx % 8
    const int xcd = blockIdx.x & 7, qd = blockIdx.x >> 3;
    const int g = (qd / NS) * 8 + xcd, slice = qd % NS;
    int *flags = p.ctl + (size_t)g * D;
    int *progress = p.ctl + (size_t)p.ngroups * D + (size_t)g * NS;
    int *xccw = p.ctl + (size_t)p.ngroups * (D + NS) + (size_t)g * NS;
    int *abort_word = p.ctl + (size_t)p.ngroups * (D + 2 * NS);
    char *ring = p.ring + (size_t)g * D * RS;
    Scr &scr = *reinterpret_cast<Scr *>(p.scratch + (size_t)blockIdx.x * fused_scratch_stride<DK, C, KDA>());

    if (tid == 0) {
        sm.full[0] = sm.full[1] = 0;
        sm.done[0] = sm.done[1] = 0;
        sm.pbar = 0;
        sm.abort = 0;
        // group locality: every member records its XCD, then compares
        const int me = (int)__builtin_amdgcn_s_getreg((3 << 11) | 20);   // HW_REG_XCC_ID[3:0]
        st_agent(&xccw[slice], me);
        int local = 1;
        for (int s = 0; s < NS; ++s) {
            int v = -1;
            if (!wait_until([&] { v = ld_agent(&xccw[s]); return v >= 0; }, abort_word)) { sm.abort = 1; break; }
            local &= v == me;
        }
        sm.local = local;
    }
    __syncthreads();
    const bool local = sm.local;
    if (sm.abort) return;

    // total records of the group and a walker over (unit, chunk) pairs
    // ================================ chain waves ================================
    if (wave < NCW) {
        const int cw = wave;
        __builtin_amdgcn_s_setprio(2);
        using OT_F = float;
        const int HDV = H * DV;
        const int v0 = slice * DVS + 16 * cw;
        int r = 0;
        bool failed = false;
        FusedUnit u;
        for (int ui = 0; fused_unit(p, g, ui, u); ++ui) {
            const size_t srow = ((size_t)u.n * H + u.h) * DV * DK + (size_t)(v0 + lr) * DK + 4 * lg;
            f32x4 St[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                St[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (p.state_in) St[kb] = *reinterpret_cast<const f32x4 *>(p.state_in + srow + 16 * kb);
            }
            for (int c = 0; c < u.nch && !failed; ++c, ++r) {
                const int sl = r & 1;
                if (!wait_until([&] { return ld_lds(&sm.full[sl]) == r + 1; }, abort_word)) { failed = true; break; }
                const Slot &bs = sm.slot[sl];
                const RecL &bc = bs.rec.r;
                const int t0 = u.bos + c * C;
                const int nv = min(C, u.eos - t0);
                // Q e^g rows from the ring (A operand of Y), requested first
                const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
                    ring + (size_t)(r % D) * RS + fused_lds_part<DK, C, KDA>(), 0, C * DK * 2, kBufferWord3);
                RowA<ST, NKB> qa[NB];
#pragma unroll
                for (int rb = 0; rb < NB; ++rb)
#pragma unroll
                    for (int s = 0; s < NKS; ++s) {
                        const i32x4 x = ring_load16(qrs, ((16 * rb + lr) * DK + 8 * (4 * s + lg)) * 2);
                        qa[rb].f[s] = __builtin_bit_cast(f16x8, x);
                    }
                const int swK = row_swizzle(GK, lr), swC = row_swizzle(GC, lr);
                auto tri = [](int rb) { return (16 * rb + 16 + 31) / 32; };
                // U = T diag(b) V (state-independent part)
                RowA<ST, NB> vb;
                vb.load(&bs.Vt[16 * cw + lr][0], lg);
                f32x4 U[NB], Y[NB];
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    RowA<ST, NB> ta;
                    ta.load(&bc.Tm[16 * rb + lr][0], lg, tri(rb), swC);
                    U[rb] = Y[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < NB / 2; ++st)
                        if (st < tri(rb)) U[rb] = rowa_mma(U[rb], ta, vb, st);
                }
                RegB<ST, NKB> sop;
                sop.set(St);
                f32x4 dk[KDA ? NKB : 1];
                if constexpr (KDA) {
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) dk[kb] = *reinterpret_cast<const f32x4 *>(&bc.dec[16 * kb + 4 * lg]);
                } else {
                    const float d = bc.dec[0];
                    dk[0] = f32x4{d, d, d, d};
                }
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) St[kb][i] *= dk[KDA ? kb : 0][i];
                // U += W_n S0^T, Y = (Q e^g) S0^T
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    RowA<ST, NKB> wa;
                    wa.load(&bc.Wn[16 * rb + lr][0], lg, 1 << 20, swK);
#pragma unroll
                    for (int s = 0; s < NKS; ++s) U[rb] = sop.step(U[rb], wa, s);
                }
#pragma unroll
                for (int rb = 0; rb < NB; ++rb)
#pragma unroll
                    for (int s = 0; s < NKS; ++s) Y[rb] = sop.step(Y[rb], qa[rb], s);
                RegB<ST, NB> uh, ul;
                uh.set_split(U, ul);
                // S^T <- Diag(e^{g_C}) S0^T + K_end^T U (hi, then lo)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    RowA<ST, NB> kea;
                    kea.load(&bc.KeT[16 * kb + lr][0], lg, 1 << 20, swC);
#pragma unroll
                    for (int st = 0; st < NB / 2; ++st) St[kb] = uh.step(St[kb], kea, st);
#pragma unroll
                    for (int st = 0; st < NB / 2; ++st) St[kb] = ul.step(St[kb], kea, st);
                }
                // O = Y + M U
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    RowA<ST, NB> ma;
                    ma.load(&bc.Mm[16 * rb + lr][0], lg, tri(rb), swC);
#pragma unroll
                    for (int st = 0; st < NB / 2; ++st)
                        if (st < tri(rb)) {
                            Y[rb] = uh.step(Y[rb], ma, st);
                            Y[rb] = ul.step(Y[rb], ma, st);
                        }
                }
                // this slot's LDS reads are done
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
                if (lane == 0) __hip_atomic_fetch_add(&sm.done[sl], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                // outputs: rows 16 rb + 4 lg + i, column v0 + lr; rows past the
                // sequence fall outside the buffer range and are dropped
                if (p.out_bf16) {
                    __bf16 *ob = static_cast<__bf16 *>(p.out) + ((size_t)t0 * H + u.h) * DV + v0;
                    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(ob, 0, ((nv - 1) * HDV + 16) * 2, kBufferWord3);
#pragma unroll
                    for (int rb = 0; rb < NB; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            buffer_store_nt(ors, ((16 * rb + 4 * lg + i) * HDV + lr) * 2, (__bf16)Y[rb][i]);
                } else {
                    OT_F *ob = static_cast<OT_F *>(p.out) + ((size_t)t0 * H + u.h) * DV + v0;
                    const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(ob, 0, ((nv - 1) * HDV + 16) * 4, kBufferWord3);
#pragma unroll
                    for (int rb = 0; rb < NB; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) buffer_store_nt(ors, ((16 * rb + 4 * lg + i) * HDV + lr) * 4, Y[rb][i]);
                }
            }
            if (p.state_out) {
                const float nanv = __builtin_nanf("");
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    f32x4 o = St[kb];
                    if (failed) o = f32x4{nanv, nanv, nanv, nanv};
                    *reinterpret_cast<f32x4 *>(p.state_out + srow + 16 * kb) = o;
                }
            }
            if (failed) {   // the remaining units of the group: NaN final states
                FusedUnit w;
                for (int uj = ui + 1; fused_unit(p, g, uj, w); ++uj)
                    if (p.state_out) {
                        const size_t wrow = ((size_t)w.n * H + w.h) * DV * DK + (size_t)(v0 + lr) * DK + 4 * lg;
                        const float nanv = __builtin_nanf("");
#pragma unroll
                        for (int kb = 0; kb < NKB; ++kb)
                            *reinterpret_cast<f32x4 *>(p.state_out + wrow + 16 * kb) = f32x4{nanv, nanv, nanv, nanv};
                    }
                break;
            }
        }
        return;
    }

    // ================================ loader wave ================================
    if (wave == NCW) {
        int goff[RX];
#pragma unroll
        for (int x = 0; x < RX; ++x) goff[x] = 16 * fused_piece_at<DK, C, KDA>(64 * x + lane);
        constexpr int EPV = 8;                      // bf16 values per 16-byte vector
        constexpr int VPL = C * DVS / EPV / 64;     // value vectors per lane per chunk
        static_assert(VPL >= 1 && (C * DVS / EPV) % 64 == 0, "value vectors");
        const __bf16 *gv = static_cast<const __bf16 *>(p.v);
        int r = 0;
        FusedUnit u;
        for (int ui = 0; fused_unit(p, g, ui, u); ++ui) {
            bool failed = false;
            for (int c = 0; c < u.nch; ++c, ++r) {
                const int sl = r & 1;
                // the chain waves are done with record r - 2 (this slot's last use)
                if (r >= 2) {
                    const int want = NCW * (r >> 1);
                    if (!wait_until([&] { return ld_lds(&sm.done[sl]) >= want; }, abort_word)) { failed = true; break; }
                    if (lane == 0) st_flag(&progress[slice], r - 1, local);
                }
                // record r published?
                if (!wait_until([&] { return ld_agent(&flags[r % D]) == r + 1; }, abort_word)) { failed = true; break; }
                if (!local) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                const char *src = ring + (size_t)(r % D) * RS;
                char *dst = sm.slot[sl].rec.raw;
#pragma unroll
                for (int x = 0; x < RX; ++x) lds_direct_load16_coherent(src + goff[x], dst + 1024 * x);
                // the value slice, transposed into fp16 (rows past the sequence: 0)
                const int t0 = u.bos + c * C;
                i32x4 vr[VPL];
                bool vok[VPL];
#pragma unroll
                for (int y = 0; y < VPL; ++y) {
                    const int e = lane + 64 * y, vt = e / (DVS / EPV), vc = (e % (DVS / EPV)) * EPV;
                    const int t = t0 + vt;
                    vok[y] = t < u.eos;
                    vr[y] = *reinterpret_cast<const i32x4 *>(gv + ((size_t)min(t, u.eos - 1) * H + u.h) * DV + slice * DVS + vc);
                }
                __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): LDS-direct copies and value loads landed
#pragma unroll
                for (int y = 0; y < VPL; ++y) {
                    const int e = lane + 64 * y, vt = e / (DVS / EPV), vc = (e % (DVS / EPV)) * EPV;
                    const bf16x8 b = __builtin_bit_cast(bf16x8, vr[y]);
#pragma unroll
                    for (int i = 0; i < EPV; ++i) sm.slot[sl].Vt[vc + i][kpos<ST>(vt)] = vok[y] ? (ST)(float)b[i] : (ST)0.f;
                }
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
                if (lane == 0) st_lds(&sm.full[sl], r + 1);
            }
            if (failed) break;
        }
        return;
    }

    // ================================= prep waves =================================
    const int pw = wave - NCW - 1;     // row tile of this wave
    int bar_epoch = 0;
    auto prep_barrier = [&]() -> bool {
        __builtin_amdgcn_s_waitcnt(0xc07f);   // this wave's LDS writes are complete
        bar_epoch += NPW;
        if (lane == 0) __hip_atomic_fetch_add(&sm.pbar, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int want = bar_epoch;
        return wait_until([&] { return ld_lds(&sm.pbar) >= want; }, abort_word);
    };
    const __bf16 *gq = static_cast<const __bf16 *>(p.q);
    const __bf16 *gk = static_cast<const __bf16 *>(p.k);

    // inputs of one owned record, held in registers: k and q fragments (kpos
    // layout: lane (lr, lg), k-step s holds channels 32 s + {4 lg + i, 16 + 4 lg + i}),
    // the log-decay (per channel or per token) and beta of token 16 pw + lr
    bf16x8 kin[NKS], qin[NKS];
    f32x4 lain[KDA ? 2 * NKS : 1];
    float bin = 0.f, lain_h = 0.f;
    auto fetch = [&](const FusedUnit &uu, int c) {
        const int t = uu.bos + c * C + 16 * pw + lr;
        const bool ok = t < uu.eos;
        const int hq = uu.h / p.G;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            kin[s] = bf16x8{};
            qin[s] = bf16x8{};
        }
        if (ok) {
#pragma unroll
            for (int s = 0; s < NKS; ++s)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const size_t off = ((size_t)t * p.HK + hq) * DK + 32 * s + 16 * hh + 4 * lg;
                    const bf16x4 kv = *reinterpret_cast<const bf16x4 *>(gk + off);
                    const bf16x4 qv = *reinterpret_cast<const bf16x4 *>(gq + off);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        kin[s][4 * hh + i] = kv[i];
                        qin[s][4 * hh + i] = qv[i];
                    }
                }
        }
        if constexpr (KDA) {
#pragma unroll
            for (int x = 0; x < 2 * NKS; ++x) {
                lain[x] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (ok) {
                    const size_t off = ((size_t)t * H + uu.h) * DK + 32 * (x >> 1) + 16 * (x & 1) + 4 * lg;
                    if (p.gate_bf16) {
                        const bf16x4 b4 = *reinterpret_cast<const bf16x4 *>(static_cast<const __bf16 *>(p.log_alpha) + off);
#pragma unroll
                        for (int i = 0; i < 4; ++i) lain[x][i] = (float)b4[i];
                    } else {
                        lain[x] = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(p.log_alpha) + off);
                    }
                }
            }
        } else {
            lain_h = 0.f;
            if (ok)
                lain_h = p.gate_bf16 ? (float)static_cast<const __bf16 *>(p.log_alpha)[(size_t)t * H + uu.h]
                                     : static_cast<const float *>(p.log_alpha)[(size_t)t * H + uu.h];
        }
        bin = 0.f;
        if (ok)
            bin = p.gate_bf16 ? (float)static_cast<const __bf16 *>(p.beta)[(size_t)t * H + uu.h]
                              : static_cast<const float *>(p.beta)[(size_t)t * H + uu.h];
    };

    // walker over the group's records, positioned at the next one this slice owns
    struct Cursor { int ui, c, r; FusedUnit u; bool valid; };
    auto advance = [&](Cursor &cu_) {   // to the next owned record after the current position
        while (cu_.valid) {
            ++cu_.c;
            ++cu_.r;
            while (cu_.c >= cu_.u.nch) {
                ++cu_.ui;
                cu_.c = 0;
                if (!fused_unit(p, g, cu_.ui, cu_.u)) { cu_.valid = false; return; }
            }
            if (cu_.r % NS == slice) return;
        }
    };
    Cursor cur;
    cur.ui = 0;
    cur.c = -1;
    cur.r = -1;
    cur.valid = fused_unit(p, g, 0, cur.u);
    advance(cur);
    if (cur.valid) fetch(cur.u, cur.c);

    // constant B fragments that transpose a 16 x 32 A fragment through the
    // MFMA (D = A I_h: lane l gets channel 16 h + (l & 15) of tokens 4 lg + i)
    f16x8 eye[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 8; ++j) eye[hf][j] = (lg == (lr >> 2) && j == 4 * hf + (lr & 3)) ? (ST)1.f : (ST)0.f;

    constexpr float L2E = 1.4426950408889634f;
    while (cur.valid) {
        const FusedUnit u = cur.u;
        const int c = cur.c, r = cur.r;
        const int t0 = u.bos + c * C;
        Rec &rec = *reinterpret_cast<Rec *>(ring + (size_t)(r % D) * RS);
        // the ring slot is free once every slice has consumed record r - D
        if (pw == 0 && r >= D) {
            const int want = r - D + 1;
            bool ok = true;
            for (int s = 0; s < NS && ok; ++s)
                ok = wait_until([&] { return ld_agent(&progress[s]) >= want; }, abort_word);
            if (!ok) break;
        }
        // ---- P2: in-tile prefix sums of the log-decay; beta
        f32x4 gsc[KDA ? 2 * NKS : 1];
        float gsh = 0.f;
        if constexpr (KDA) {
#pragma unroll
            for (int x = 0; x < 2 * NKS; ++x)
#pragma unroll
                for (int i = 0; i < 4; ++i) gsc[x][i] = scan_row16(lain[x][i]);
            if (lr == 15) {
#pragma unroll
                for (int x = 0; x < 2 * NKS; ++x) *reinterpret_cast<f32x4 *>(&sm.tot[pw][32 * (x >> 1) + 16 * (x & 1) + 4 * lg]) = gsc[x];
            }
            if (pw == 0 && lr == 0) {
#pragma unroll
                for (int x = 0; x < 2 * NKS; ++x) *reinterpret_cast<f32x4 *>(&sm.gfirst[32 * (x >> 1) + 16 * (x & 1) + 4 * lg]) = gsc[x];
            }
        } else {
            gsh = scan_row16(lain_h);
            if (lr == 15 && lg == 0) sm.tot[pw][0] = gsh;
        }
        if (lg == 0) sm.beta[16 * pw + lr] = bin;
        if (!prep_barrier()) break;

        // ---- P2b (KDA): per-channel constants on prep wave 0; e^{g_C} to the ring
        if constexpr (KDA) {
            if (pw == 0) {
#pragma unroll
                for (int cc = 0; cc < DK / 64 + (DK < 64); ++cc) {
                    const int ch = lane + 64 * cc;
                    if (ch < DK) {
                        float run = 0.f;
#pragma unroll
                        for (int tb = 0; tb < NB; ++tb) {
                            sm.carry[tb][ch] = run;
                            run += sm.tot[tb][ch];
                        }
                        const float m = 0.5f * (sm.gfirst[ch] + run);
                        sm.mid[ch] = m;
                        sm.em[ch] = __builtin_amdgcn_exp2f(m * L2E);
                        sm.ecm[ch] = __builtin_amdgcn_exp2f((run - m) * L2E);
                        rec.dec[ch] = __builtin_amdgcn_exp2f(run * L2E);
                    }
                }
            }
            if (!prep_barrier()) break;
        }

        // ---- P3: decayed operands; Q e^g and K_end^T to the ring; (K e^g)^T and
        // the right Gram operands to the scratch
        bf16x8 fl[NKS], fqh[NKS], fql[NKS];   // left Gram operands (GDN: fl = k, fqh = q)
        float gt_row = 0.f;   // GDN: cumulative log-decay of this lane's token
        if constexpr (!KDA) {
            float carry = 0.f, gC = 0.f;
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                const float tt = sm.tot[tb][0];
                if (tb < pw) carry += tt;
                gC += tt;
            }
            gt_row = gsh + carry;
            if (lg == 0) sm.g[16 * pw + lr] = gt_row;
            if (pw == 0 && lane == 0) rec.dec[0] = __builtin_amdgcn_exp2f(gC * L2E);
            const float eg = __builtin_amdgcn_exp2f(gt_row * L2E) , egc = __builtin_amdgcn_exp2f((gC - gt_row) * L2E);
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                f16x8 qt, kt, ke;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float kf = (float)kin[s][j], qf = (float)qin[s][j];
                    qt[j] = (ST)(qf * eg * p.scale);
                    kt[j] = (ST)(kf * eg);
                    ke[j] = (ST)(kf * egc);
                }
                fl[s] = kin[s];
                fqh[s] = qin[s];
                *reinterpret_cast<f16x8 *>(&rec.Qt[16 * pw + lr][32 * s + 8 * lg]) = qt;
                // transposes: K_end^T to the ring, (K e^g)^T to the scratch
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const f32x4 te = __builtin_amdgcn_mfma_f32_16x16x32_f16(ke, eye[hf], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    const f32x4 tk = __builtin_amdgcn_mfma_f32_16x16x32_f16(kt, eye[hf], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    const int ch = 32 * s + 16 * hf + lr;
                    const int tp = 32 * (pw >> 1) + 8 * lg + 4 * (pw & 1);
                    const ST e4[4] = {(ST)te[0], (ST)te[1], (ST)te[2], (ST)te[3]};
                    const ST k4[4] = {(ST)tk[0], (ST)tk[1], (ST)tk[2], (ST)tk[3]};
                    store_vec<ST, 4>(&rec.KeT[ch][tp], e4);
                    store_vec<ST, 4>(&scr.KtT[ch][tp], k4);
                }
                *reinterpret_cast<bf16x8 *>(&scr.rk[pw][0][lr][32 * s + 8 * lg]) = kin[s];
            }
        } else {
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                f16x8 qt, kt, ke;
                bf16x8 frh, frl;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int cb = 32 * s + 16 * hh + 4 * lg;
                    const f32x4 cr = *reinterpret_cast<const f32x4 *>(&sm.carry[pw][cb]);
                    const f32x4 md = *reinterpret_cast<const f32x4 *>(&sm.mid[cb]);
                    const f32x4 emv = *reinterpret_cast<const f32x4 *>(&sm.em[cb]);
                    const f32x4 ecv = *reinterpret_cast<const f32x4 *>(&sm.ecm[cb]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = 4 * hh + i;
                        const float d2 = (gsc[2 * s + hh][i] + cr[i] - md[i]) * L2E;
                        const float E = __builtin_amdgcn_exp2f(d2), Ei = __builtin_amdgcn_exp2f(-d2);
                        const float kf = (float)kin[s][j], qf = (float)qin[s][j];
                        const float lk = kf * E, lq = qf * E, rk = kf * Ei;
                        fl[s][j] = (__bf16)lk;
                        const __bf16 qh = (__bf16)lq, rh = (__bf16)rk;
                        fqh[s][j] = qh;
                        fql[s][j] = (__bf16)(lq - (float)qh);
                        frh[j] = rh;
                        frl[j] = (__bf16)(rk - (float)rh);
                        qt[j] = (ST)(lq * emv[i] * p.scale);
                        kt[j] = (ST)(lk * emv[i]);
                        ke[j] = (ST)(rk * ecv[i]);
                    }
                }
                *reinterpret_cast<f16x8 *>(&rec.Qt[16 * pw + lr][32 * s + 8 * lg]) = qt;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const f32x4 te = __builtin_amdgcn_mfma_f32_16x16x32_f16(ke, eye[hf], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    const f32x4 tk = __builtin_amdgcn_mfma_f32_16x16x32_f16(kt, eye[hf], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    const int ch = 32 * s + 16 * hf + lr;
                    const int tp = 32 * (pw >> 1) + 8 * lg + 4 * (pw & 1);
                    const ST e4[4] = {(ST)te[0], (ST)te[1], (ST)te[2], (ST)te[3]};
                    const ST k4[4] = {(ST)tk[0], (ST)tk[1], (ST)tk[2], (ST)tk[3]};
                    store_vec<ST, 4>(&rec.KeT[ch][tp], e4);
                    store_vec<ST, 4>(&scr.KtT[ch][tp], k4);
                }
                *reinterpret_cast<bf16x8 *>(&scr.rk[pw][0][lr][32 * s + 8 * lg]) = frh;
                *reinterpret_cast<bf16x8 *>(&scr.rk[pw][KDA ? 1 : 0][lr][32 * s + 8 * lg]) = frl;
                // one key block at a time: keeps the scheduler from hoisting every
                // block's constants (register pressure)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): scratch stores complete
        if (!prep_barrier()) break;

        // ---- P4: Gram tiles (pw, J), J <= pw: A to LDS, M to the ring
        const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(&scr, 0, (int)sizeof(Scr), kBufferWord3);
        const f32x4 brow = *reinterpret_cast<const f32x4 *>(&sm.beta[16 * pw + 4 * lg]);
#pragma unroll 1
        for (int J = 0; J <= (pw | 1) && J < NB; ++J) {
            const int mrow = 16 * pw + lr;                                  // M row of this lane
            const int mcol = 32 * (J >> 1) + 8 * lg + 4 * (J & 1);          // its 4 columns (kpos)
            if (J > pw) {   // above the diagonal inside the same 32-wide block: zeros
                const ST z4[4] = {(ST)0.f, (ST)0.f, (ST)0.f, (ST)0.f};
                store_vec<ST, 4>(&rec.Mm[mrow][mcol], z4);
                continue;
            }
            bf16x8 rh[NKS], rl[NKS];
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                rh[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                    srs, (int)offsetof(Scr, rk) + (((J * (KDA ? 2 : 1) + 0) * 16 + lr) * DK + 32 * s + 8 * lg) * 2, 0, kCoherentLoad));
                if constexpr (KDA)
                    rl[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                        srs, (int)offsetof(Scr, rk) + (((J * 2 + 1) * 16 + lr) * DK + 32 * s + 8 * lg) * 2, 0, kCoherentLoad));
            }
            f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f}, mt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NKS; ++s) {
                a = gram_mma(a, fl[s], rh[s]);          // A[r = 16 pw + 4 lg + i][i' = 16 J + lr]
                mt = gram_mma(mt, rh[s], fqh[s]);       // M^T[i' = 16 J + 4 lg + i][r = 16 pw + lr]
                if constexpr (KDA) {
                    mt = gram_mma(mt, rl[s], fqh[s]);
                    mt = gram_mma(mt, rh[s], fql[s]);
                }
            }
            // A (strictly lower) -> LDS
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * pw + 4 * lg + i, cc = 16 * J + lr;
                float v = cc < rr ? a[i] * brow[i] : 0.f;
                if constexpr (!KDA) v *= cc < rr ? __builtin_amdgcn_exp2f((sm.g[rr] - sm.g[cc]) * L2E) : 0.f;
                sm.At[rr][cc] = v;
            }
            // M (lower incl. diagonal) -> ring
            ST m4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int cc = 16 * J + 4 * lg + i;
                float v = cc <= mrow ? mt[i] * p.scale : 0.f;
                if constexpr (!KDA) v *= cc <= mrow ? __builtin_amdgcn_exp2f((sm.g[mrow] - sm.g[cc]) * L2E) : 0.f;
                m4[i] = (ST)v;
            }
            store_vec<ST, 4>(&rec.Mm[mrow][mcol], m4);
        }
        // the next owned record's inputs (this one's operands are consumed)
        Cursor nxt = cur;
        advance(nxt);
        if (nxt.valid) fetch(nxt.u, nxt.c);
        if (!prep_barrier()) break;

        // ---- P5: T = (I + A)^-1.  Diagonal blocks: wave p inverts block p,
        // unit lower triangular I + N with N nilpotent (N^16 = 0), as
        // (I - N)(I + N^2)(I + N^4)(I + N^8) on the fp32 MFMA.  A product X Y
        // takes X as rows (A operand) and Y in the accumulator layout (B
        // operand); a result goes through its own LDS tile when it is next
        // needed as rows.
        {
            const int I = pw;
            float(*tile)[SM::LDT] = reinterpret_cast<float(*)[SM::LDT]>(&sm.Tt[16 * I][16 * I]);
            auto rows_of = [&](const f32x4 &acc) {   // acc (col lr, rows 4 lg + i) -> rows (row lr, k 4 lg + i)
#pragma unroll
                for (int i = 0; i < 4; ++i) tile[4 * lg + i][lr] = acc[i];
                RowA<float, 1> a;
                a.load(&tile[lr][0], lg);
                return a;
            };
            auto plus_eye = [&](f32x4 acc) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += 4 * lg + i == lr ? 1.f : 0.f;
                return acc;
            };
            RowA<float, 1> nrow;
            nrow.load(&sm.At[16 * I + lr][16 * I], lg);   // N rows (zero on and above the diagonal)
            RegB<float, 1> ncol;
#pragma unroll
            for (int i = 0; i < 4; ++i) ncol.f[0][i] = sm.At[16 * I + 4 * lg + i][16 * I + lr];
            const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
            RegB<float, 1> b2, b4, b8;
            const f32x4 n2 = ncol.mma(z, nrow);
            b2.set(&n2);
            const f32x4 n4 = b2.mma(z, rows_of(n2));
            b4.set(&n4);
            const f32x4 n8 = b4.mma(z, rows_of(n4));
            // (I - N) rows
            RowA<float, 1> imn;
#pragma unroll
            for (int i = 0; i < 4; ++i) imn.f[0][i] = (4 * lg + i == lr ? 1.f : 0.f) - nrow.f[0][i];
            f32x4 q = plus_eye(n2);
            RegB<float, 1> bq;
            bq.set(&q);
            f32x4 r1 = bq.mma(z, imn);             // (I - N)(I + N^2)
            q = plus_eye(n4);
            bq.set(&q);
            const f32x4 r2 = bq.mma(z, rows_of(r1));   // ... (I + N^4)
            q = plus_eye(n8);
            bq.set(&q);
            const f32x4 tii = bq.mma(z, rows_of(r2));  // ... (I + N^8) = T_II
            // lower part (rows >= column) and its mirror (upper part)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * lg + i >= lr) tile[4 * lg + i][lr] = tii[i];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * lg + i > lr) tile[lr][4 * lg + i] = tii[i];
        }
        if (!prep_barrier()) break;
        // Off-diagonal blocks, column J on wave J, top to bottom:
        // T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ; the blocks T_KJ of this column
        // stay in registers in the accumulator layout (the B operand).
        {
            const int J = pw;
            f32x4 tcolb[NB];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                tcolb[0][i] = (4 * lg + i >= lr) ? sm.Tt[16 * J + 4 * lg + i][16 * J + lr] : 0.f;
#pragma unroll
            for (int dI = 1; dI < NB; ++dI) {
                const int I = J + dI;
                if (I >= NB) break;
                f32x4 P = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dK = 0; dK < dI; ++dK) {
                    RowA<float, 1> aik;
                    aik.load(&sm.At[16 * I + lr][16 * (J + dK)], lg);
                    RegB<float, 1> tk;
                    tk.set(&tcolb[dK]);
                    P = tk.mma(P, aik);
                }
                RegB<float, 1> pb;
                pb.set(&P);
                RowA<float, 1> tii;
                tii.load(&sm.Tt[16 * I + lr][16 * I], lg);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (4 * lg + i > lr) tii.f[0][i] = 0.f;
                const f32x4 tij = pb.mma(f32x4{0.f, 0.f, 0.f, 0.f}, tii);
                f32x4 ntij;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ntij[i] = -tij[i];
                    sm.Tt[16 * I + 4 * lg + i][16 * J + lr] = ntij[i];
                }
                *reinterpret_cast<f32x4 *>(&sm.Tt[16 * J + lr][16 * I + 4 * lg]) = ntij;
                tcolb[dI] = ntij;
            }
        }
        if (!prep_barrier()) break;

        // ---- P6: T diag(b) rows to the ring; W_n = -T diag(b) (K e^g) for
        // this wave's key-block pairs
        auto tbeta_row = [&](int row, RowA<ST, NB> &f) {
#pragma unroll
            for (int st = 0; st < NB / 2; ++st)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int s0 = 32 * st + 16 * hh + 4 * lg;
                    f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f}, b = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (s0 <= row) {
                        t = *reinterpret_cast<const f32x4 *>(&sm.Tt[row][s0]);
                        b = *reinterpret_cast<const f32x4 *>(&sm.beta[s0]);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) f.f[st][4 * hh + i] = (ST)(s0 + i <= row ? t[i] * b[i] : 0.f);
                }
        };
        {
            RowA<ST, NB> own;
            tbeta_row(16 * pw + lr, own);
            own.store(&rec.Tm[16 * pw + lr][0], lg);
        }
        for (int pp = pw; pp < NKB / 2; pp += NPW) {
            RowA<ST, NB> kta[2];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int st = 0; st < NB / 2; ++st)
                    kta[x].f[st] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                        srs, (int)offsetof(Scr, KtT) + ((32 * pp + 16 * x + lr) * C + 32 * st + 8 * lg) * 2, 0, kCoherentLoad));
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) {
                RowA<ST, NB> tb;
                tbeta_row(16 * rb + lr, tb);
                const int nst = (16 * rb + 16 + 31) / 32;
                ST w[8];
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int st = 0; st < NB / 2; ++st)
                        if (st < nst) acc = rowa_mma(acc, kta[x], tb, st);
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[4 * x + i] = (ST)(-acc[i]);
                }
                store_vec<ST, 8>(&rec.Wn[16 * rb + lr][32 * pp + 8 * lg], w);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): every ring store of this wave is complete (and the fetch landed)
        if (!prep_barrier()) break;
        // ---- P7: publish
        if (pw == 0 && lane == 0) {
            if (!local) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            st_flag(&flags[r % D], r + 1, local);
        }
        cur = nxt;
    }
}

// Zero the handshake words of one call: flags and progress, member XCDs -1,
// the abort word.
static __global__ __launch_bounds__(256) void fused_ctl_init(int *ctl, int nflags, int nxcc) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < nflags) ctl[i] = 0;
    else if (i < nflags + nxcc) ctl[i] = -1;
    else if (i == nflags + nxcc) ctl[i] = 0;
}

template <int DK, int DVS, bool KDA>
int fused_blocks_per_cu() {
    int n = 0;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fused_prefill_kernel<DK, DVS, kFusedChunk, KDA>,
                                                        64 * (DVS / 16 + 1 + kFusedChunk / 16), 0) == hipSuccess
               ? n
               : 0;
}

template <int DK, int DVS, bool KDA>
hipError_t launch_fused_t(const FusedArgs &fa, int grid, hipStream_t st) {
    const int nflags = fa.ngroups * (fa.D + fa.NS), nxcc = fa.ngroups * fa.NS;
    hipLaunchKernelGGL(fused_ctl_init, dim3((unsigned)((nflags + nxcc + 1 + 255) / 256)), dim3(256), 0, st, fa.ctl,
                       nflags, nxcc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fused_prefill_kernel<DK, DVS, kFusedChunk, KDA>), dim3((unsigned)grid),
                       dim3(64 * (DVS / 16 + 1 + kFusedChunk / 16)), 0, st, fa);
    return hipGetLastError();
}

}  // namespace gdr
