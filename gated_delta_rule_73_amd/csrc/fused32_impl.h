// fused32_impl.h -- single-kernel chunked prefill with 32-token chunks, one
// prep wave per record (gfx950, bf16 q/k/v, fp32 state).
//
// Same recurrence, chunk algebra, ring protocol and roles as fused_impl.h
// (the 64-token kernel); what differs is how records are built.  A 32-token
// record fits one wave: lane (l & 15) owns tokens l & 15 and 16 + (l & 15) of
// the chunk, and for each 32-wide block of key channels the lane group l >> 4
// owns channels {4 lg + i, 16 + 4 lg + i}.  So a single prep wave scans the
// log-decay of all 32 tokens (DPP across lanes, the second row tile carried
// from the first), forms the decayed operands, accumulates the three lower
// Gram tiles on MFMA block by block, inverts I + A and forms W_n, all in
// registers plus a small LDS scratch of its own -- no barrier with any other
// wave.  Two prep waves per workgroup build different records at once; with
// NS slices per (sequence, head), 2 NS records are in flight per unit, slice
// s wave p building the records r with r % NS == s and (r / NS) % 2 == p.
// A record is 29 KB (d_k = 128), so the ring of D = 2 NS + 4 records stays in
// the XCD's L2.  The loader keeps one record's copies in flight while it
// finishes the previous one, over three LDS slots.
#pragma once

#include "fused_impl.h"

namespace gdr {

constexpr int kFusedChunk32 = 32;

template <int DK, bool KDA>
struct Fused32Rec {
    float dec[KDA ? DK : 4];   // e^{g_C} per key channel (GDN: dec[0])
    _Float16 Wn[32][DK];       // key channel in kpos order
    _Float16 Qt[32][DK];       // Q e^g scale, key channel in kpos order
    _Float16 KeT[DK][32];      // token in kpos order
    _Float16 Tm[32][32];       // T diag(b), token in kpos order, zero above the diagonal
    _Float16 Mm[32][32];       // M, zero above the diagonal
};
template <int DK, bool KDA>
constexpr size_t fused32_rec_stride() { return (sizeof(Fused32Rec<DK, KDA>) + 255) & ~size_t(255); }

template <int DK, int DVS, bool KDA>
struct alignas(16) Fused32Slot {
    static constexpr int RB = (int)sizeof(Fused32Rec<DK, KDA>);
    static constexpr int RAW = (RB + 1023) / 1024 * 1024;   // whole 1 KB rounds of the loader's copies
    static constexpr int LDVT = lds_pitch(32 * 2) / 2;
    union {
        Fused32Rec<DK, KDA> r;
        char raw[RAW];
    } rec;
    _Float16 Vt[DVS][LDVT];   // value slice: value rows, tokens in kpos order
};

template <int DK>
struct alignas(16) Prep32Scratch {
    float At[32][36];    // A (strictly lower part)
    float Tt[32][36];    // T (lower part incl. diagonal); diagonal blocks double as product scratch
    float beta[32], g[32];
    _Float16 KtT[DK][40];   // (K e^g)^T: key rows, tokens in kpos order (80-byte rows: conflict-free 16-byte reads)
};

template <int DK, int DVS, bool KDA>
struct Fused32Smem {
    static constexpr int NSLOT = 3;
    Fused32Slot<DK, DVS, KDA> slot[NSLOT];
    Prep32Scratch<DK> ps[2];
    int full[NSLOT], done[NSLOT], local, abort;
};

// the piece of a record held by 16-byte position q of a slot (rows swizzled
// with row_swizzle); past the record: any valid piece
template <int DK, bool KDA>
__device__ __forceinline__ int fused32_piece_at(int q) {
    constexpr int PD = (KDA ? DK : 4) * 4 / 16;
    constexpr int GK = DK * 2 / 16, GC = 32 * 2 / 16;
    constexpr int NP = (int)sizeof(Fused32Rec<DK, KDA>) / 16;
    if (q >= NP) return NP - 1;
    if (q < PD) return q;
    q -= PD;
    if (q < 2 * 32 * GK) {   // Wn, Qt rows
        const int r = q / GK, gg = q % GK;
        return PD + r * GK + (gg ^ row_swizzle(GK, r));
    }
    q -= 2 * 32 * GK;
    const int r = q / GC, gg = q % GC;   // KeT, Tm, Mm rows
    return PD + 2 * 32 * GK + r * GC + (gg ^ row_swizzle(GC, r));
}

template <int DK, int DVS, bool KDA>
__global__ __launch_bounds__(64 * (DVS / 16 + 3)) void fused32_prefill_kernel(FusedArgs p) {
    constexpr int C = 32, NB = 2, NSLOT = 3;
    using SM = Fused32Smem<DK, DVS, KDA>;
    using Rec = Fused32Rec<DK, KDA>;
    using Slot = Fused32Slot<DK, DVS, KDA>;
    using ST = _Float16;
    constexpr int NCW = DVS / 16;
    constexpr int NKB = DK / 16, NKS = DK / 32;
    constexpr int GK = DK * 2 / 16, GC = C * 2 / 16;
    constexpr size_t RS = fused32_rec_stride<DK, KDA>();
    constexpr int RX = Slot::RAW / 1024;        // loader rounds per record
    static_assert(DK % 32 == 0 && DK <= 128, "shapes");
    static_assert(sizeof(SM) <= 160 * 1024, "LDS budget");
    static_assert(sizeof(Rec) % 16 == 0, "record pieces");
    static_assert(RS == fused32_record_bytes(DK, KDA), "the host's workspace layout (launch.h) matches the kernel's");

    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int H = p.H, DV = p.DV, NS = p.NS, D = p.D;

    const int xcd = blockIdx.x & 7, qd = blockIdx.x >> 3;
    const int g = (qd / NS) * 8 + xcd, slice = qd % NS;
    int *flags = p.ctl + (size_t)g * D;
    int *progress = p.ctl + (size_t)p.ngroups * D + (size_t)g * NS;
    int *xccw = p.ctl + (size_t)p.ngroups * (D + NS) + (size_t)g * NS;
    int *abort_word = p.ctl + (size_t)p.ngroups * (D + 2 * NS);
    char *ring = p.ring + (size_t)g * D * RS;

    if (tid == 0) {
        for (int i = 0; i < NSLOT; ++i) sm.full[i] = sm.done[i] = 0;
        sm.abort = 0;
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

    // ================================ chain waves ================================
    if (wave < NCW) {
        const int cw = wave;
        __builtin_amdgcn_s_setprio(2);
        const int HDV = H * DV;
        const int v0 = slice * DVS + 16 * cw;
        const int swK = row_swizzle(GK, lr), swC = row_swizzle(GC, lr);
        int r = 0;
        bool failed = false;
        FusedUnit u;
        for (int ui = 0; fused_unit<C>(p, g, ui, u); ++ui) {
            const size_t srow = ((size_t)u.n * H + u.h) * DV * DK + (size_t)(v0 + lr) * DK + 4 * lg;
            f32x4 St[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                St[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (p.state_in && !failed) St[kb] = *reinterpret_cast<const f32x4 *>(p.state_in + srow + 16 * kb);
            }
            for (int c = 0; c < u.nch && !failed; ++c, ++r) {
                const int sl = r % NSLOT;
                if (!wait_until([&] { return ld_lds(&sm.full[sl]) == r + 1; }, abort_word)) { failed = true; break; }
                const Slot &bs = sm.slot[sl];
                const Rec &bc = bs.rec.r;
                const int t0 = u.bos + c * C;
                const int nv = min(C, u.eos - t0);
                // U = T diag(b) V, the state-independent part
                RowA<ST, NB> vb, ta[NB];
                vb.load(&bs.Vt[16 * cw + lr][0], lg);
                f32x4 U[NB], Y[NB];
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    ta[rb].load(&bc.Tm[16 * rb + lr][0], lg, 1 << 20, swC);
                    U[rb] = rowa_mma(f32x4{0.f, 0.f, 0.f, 0.f}, ta[rb], vb, 0);
                    Y[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                RegB<ST, NKB> sop;
                sop.set(St);
                if constexpr (KDA) {
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        const f32x4 dk = *reinterpret_cast<const f32x4 *>(&bc.dec[16 * kb + 4 * lg]);
#pragma unroll
                        for (int i = 0; i < 4; ++i) St[kb][i] *= dk[i];
                    }
                } else {
                    const float d = bc.dec[0];
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) St[kb][i] *= d;
                }
                // U += W_n S0^T and Y = (Q e^g) S0^T, k-step by k-step
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    RowA<ST, NKB> wa, qa;
                    wa.load(&bc.Wn[16 * rb + lr][0], lg, 1 << 20, swK);
                    qa.load(&bc.Qt[16 * rb + lr][0], lg, 1 << 20, swK);
#pragma unroll
                    for (int s = 0; s < NKS; ++s) {
                        U[rb] = sop.step(U[rb], wa, s);
                        Y[rb] = sop.step(Y[rb], qa, s);
                    }
                }
                RegB<ST, NB> uh, ul;
                uh.set_split(U, ul);
                // S^T <- Diag(e^{g_C}) S0^T + K_end^T U (hi and lo)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    RowA<ST, NB> kea;
                    kea.load(&bc.KeT[16 * kb + lr][0], lg, 1 << 20, swC);
                    St[kb] = uh.step(St[kb], kea, 0);
                    St[kb] = ul.step(St[kb], kea, 0);
                }
                // O = Y + M U
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    RowA<ST, NB> ma;
                    ma.load(&bc.Mm[16 * rb + lr][0], lg, 1 << 20, swC);
                    Y[rb] = uh.step(Y[rb], ma, 0);
                    Y[rb] = ul.step(Y[rb], ma, 0);
                }
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this slot's LDS reads are done
                if (lane == 0) __hip_atomic_fetch_add(&sm.done[sl], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (p.out_bf16) {
                    __bf16 *ob = static_cast<__bf16 *>(p.out) + ((size_t)t0 * H + u.h) * DV + v0;
                    const __amdgpu_buffer_rsrc_t ors =
                        __builtin_amdgcn_make_buffer_rsrc(ob, 0, ((nv - 1) * HDV + 16) * 2, kBufferWord3);
#pragma unroll
                    for (int rb = 0; rb < NB; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            buffer_store_nt(ors, ((16 * rb + 4 * lg + i) * HDV + lr) * 2, (__bf16)Y[rb][i]);
                } else {
                    float *ob = static_cast<float *>(p.out) + ((size_t)t0 * H + u.h) * DV + v0;
                    const __amdgpu_buffer_rsrc_t ors =
                        __builtin_amdgcn_make_buffer_rsrc(ob, 0, ((nv - 1) * HDV + 16) * 4, kBufferWord3);
#pragma unroll
                    for (int rb = 0; rb < NB; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) buffer_store_nt(ors, ((16 * rb + 4 * lg + i) * HDV + lr) * 4, Y[rb][i]);
                }
            }
            if (p.state_out) {   // (a failed call leaves NaN final states)
                const float nanv = __builtin_nanf("");
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    *reinterpret_cast<f32x4 *>(p.state_out + srow + 16 * kb) =
                        failed ? f32x4{nanv, nanv, nanv, nanv} : St[kb];
            }
        }
        return;
    }

    // ================================ loader wave ================================
    if (wave == NCW) {
        constexpr int EPV = 8;                      // bf16 values per 16-byte vector
        constexpr int VPL = C * DVS / EPV / 64;     // value vectors per lane per chunk
        static_assert(VPL >= 1 && (C * DVS / EPV) % 64 == 0, "value vectors");
        // value slices travel VA records ahead of the record copies (they come
        // from HBM; the copies come from the L2).  Buffers in use at once: the
        // record awaiting its commit, this record, and VA more.  The record loop
        // is unrolled by VB so that every buffer index is a constant (a register
        // array indexed at run time would live in scratch memory).
        constexpr int VA = 3, VB = VA + 2;
        static_assert(RX + 2 * VPL + 2 < 63, "vmcnt range");
        const __bf16 *gv = static_cast<const __bf16 *>(p.v);
        i32x4 vr[VB][VPL];
        bool vok[VB][VPL];
        // walkers over the group's (unit, chunk) records
        struct Walk {
            int ui, c;
            FusedUnit u;
            bool have;
        };
        auto walk_skip = [&](Walk &w) {
            while (w.have && w.c >= w.u.nch) {
                ++w.ui;
                w.c = 0;
                w.have = fused_unit<C>(p, g, w.ui, w.u);
            }
        };
        auto walk_init = [&](Walk &w) {
            w.ui = 0;
            w.c = 0;
            w.have = fused_unit<C>(p, g, 0, w.u);
            walk_skip(w);
        };
        auto walk_next = [&](Walk &w) {
            ++w.c;
            walk_skip(w);
        };
        Walk wr, wv;
        walk_init(wr);
        walk_init(wv);
        // value loads of wv's record into buffer b (past the group's last record:
        // a harmless reload of the first value row, so every call issues VPL loads)
        auto issue_values = [&](i32x4 (&vb)[VPL], bool (&ok)[VPL]) {
            const int t0 = wv.have ? wv.u.bos + wv.c * C : 0;
#pragma unroll
            for (int y = 0; y < VPL; ++y) {
                const int e = lane + 64 * y, vt = e / (DVS / EPV), vc = (e % (DVS / EPV)) * EPV;
                const int t = t0 + vt;
                ok[y] = wv.have && t < wv.u.eos;
                const size_t row = wv.have ? (size_t)min(t, wv.u.eos - 1) * H + wv.u.h : 0;
                vb[y] = __builtin_nontemporal_load(reinterpret_cast<const i32x4 *>(gv + row * DV + slice * DVS + vc));
            }
            if (wv.have) walk_next(wv);
        };
        // the value slice of record rr into its slot, transposed to fp16 (rows past
        // the sequence: 0); then the slot is marked full
        auto commit = [&](int rr, const i32x4 (&vb)[VPL], const bool (&ok)[VPL]) {
            const int sl = rr % NSLOT;
#pragma unroll
            for (int y = 0; y < VPL; ++y) {
                const int e = lane + 64 * y, vt = e / (DVS / EPV), vc = (e % (DVS / EPV)) * EPV;
                const bf16x8 b = __builtin_bit_cast(bf16x8, vb[y]);
#pragma unroll
                for (int i = 0; i < EPV; ++i) sm.slot[sl].Vt[vc + i][kpos<ST>(vt)] = ok[y] ? (ST)(float)b[i] : (ST)0.f;
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
            if (lane == 0) st_lds(&sm.full[sl], rr + 1);
        };
#pragma unroll
        for (int i = 0; i < VA; ++i) issue_values(vr[i], vok[i]);
        bool done = !wr.have;
        for (int rb = 0; !done; rb += VB) {
#pragma unroll
            for (int j = 0; j < VB; ++j) {
                if (done) continue;
                const int r = rb + j, sl = r % NSLOT;
                if (r >= NSLOT) {   // the chain waves are done with record r - NSLOT (this slot's last use)
                    const int want = NCW * (r / NSLOT);
                    if (!wait_until([&] { return ld_lds(&sm.done[sl]) >= want; }, abort_word)) { done = true; continue; }
                }
                if (!wait_until([&] { return ld_agent(&flags[r % D]) == r + 1; }, abort_word)) { done = true; continue; }
                if (!local) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                const char *src = ring + (size_t)(r % D) * RS;
                char *dst = sm.slot[sl].rec.raw;
#pragma unroll
                for (int x = 0; x < RX; ++x)
                    lds_direct_load16_coherent(src + 16 * fused32_piece_at<DK, KDA>(64 * x + lane), dst + 1024 * x);
                issue_values(vr[(j + VA) % VB], vok[(j + VA) % VB]);   // record r + VA
                // records up to r - NSLOT are consumed: their ring slots may be rebuilt.
                // Stored every iteration (so every iteration issues the same memory
                // operations) and after this record's copies (so the wait below
                // never covers it).
                if (lane == 0) st_flag(&progress[slice], max(0, r - NSLOT + 1), local);
                if (r > 0) {
                    // the previous record's copies (and its values, issued earlier) have
                    // landed: loads complete in order, and after its copies came one
                    // value batch and a progress store, then this record's copies,
                    // another value batch and a progress store
                    constexpr int AFTER = RX + 2 * VPL + 2;
                    __builtin_amdgcn_s_waitcnt((AFTER & 15) | ((AFTER >> 4) << 14) | (7 << 4) | (15 << 8));
                    commit(r - 1, vr[(j + VB - 1) % VB], vok[(j + VB - 1) % VB]);
                }
                walk_next(wr);
                if (!wr.have) {   // r was the group's last record
                    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
                    commit(r, vr[j], vok[j]);
                    done = true;
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0);   // no LDS-direct write lands after the workgroup ends
        return;
    }

    // ================================= prep waves =================================
    const int pw = wave - NCW - 1;
    Prep32Scratch<DK> &ps = sm.ps[pw];
    const __bf16 *gq = static_cast<const __bf16 *>(p.q);
    const __bf16 *gk = static_cast<const __bf16 *>(p.k);
    constexpr float L2E = 1.4426950408889634f;
    // record r of the group: unit (in the group's order) and chunk
    auto locate = [&](int r, FusedUnit &uu, int &c) -> bool {
        for (int ui = 0; fused_unit<C>(p, g, ui, uu); ++ui) {
            if (r < uu.nch) {
                c = r;
                return true;
            }
            r -= uu.nch;
        }
        return false;
    };
    // inputs of one 32-wide block of key channels: k, q fragments of the two
    // row tiles and (per-channel decay) their log-decays
    struct KIn {
        bf16x8 k[2], q[2];
        f32x4 la[2][KDA ? 2 : 1];
    };
    auto load_block = [&](const FusedUnit &uu, int c, int s, KIn &in) {
        const int hq = uu.h / p.G;
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            const int t = uu.bos + c * C + 16 * T + lr;
            const bool ok = t < uu.eos;
            in.k[T] = bf16x8{};
            in.q[T] = bf16x8{};
#pragma unroll
            for (int hh = 0; hh < (KDA ? 2 : 1); ++hh) in.la[T][hh] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (ok) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const size_t off = ((size_t)t * p.HK + hq) * DK + 32 * s + 16 * hh + 4 * lg;
                    const bf16x4 kv = __builtin_nontemporal_load(reinterpret_cast<const bf16x4 *>(gk + off));
                    const bf16x4 qv = __builtin_nontemporal_load(reinterpret_cast<const bf16x4 *>(gq + off));
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        in.k[T][4 * hh + i] = kv[i];
                        in.q[T][4 * hh + i] = qv[i];
                    }
                    if constexpr (KDA) {
                        const size_t lo = ((size_t)t * H + uu.h) * DK + 32 * s + 16 * hh + 4 * lg;
                        if (p.gate_bf16) {
                            const bf16x4 b4 = __builtin_nontemporal_load(reinterpret_cast<const bf16x4 *>(static_cast<const __bf16 *>(p.log_alpha) + lo));
#pragma unroll
                            for (int i = 0; i < 4; ++i) in.la[T][hh][i] = (float)b4[i];
                        } else {
                            in.la[T][hh] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(static_cast<const float *>(p.log_alpha) + lo));
                        }
                    }
                }
            }
        }
    };
    auto token_scalar = [&](const void *base, const FusedUnit &uu, int c, int T) -> float {
        const int t = uu.bos + c * C + 16 * T + lr;
        if (t >= uu.eos) return 0.f;
        const size_t i = (size_t)t * H + uu.h;
        return p.gate_bf16 ? (float)static_cast<const __bf16 *>(base)[i] : static_cast<const float *>(base)[i];
    };
    // constant B fragments that transpose a 16 x 32 A fragment through the
    // MFMA (D = A I_h: lane l gets channel 16 h + (l & 15) of tokens 4 lg + i)
    f16x8 eye[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int j = 0; j < 8; ++j) eye[hf][j] = (lg == (lr >> 2) && j == 4 * hf + (lr & 3)) ? (ST)1.f : (ST)0.f;

    int r = slice + NS * pw;
    FusedUnit u;
    int c = 0;
    bool have = locate(r, u, c);
    // inputs in flight: blk[s % 2] holds key block s.  Blocks 0 and 1 of a
    // record are requested during the previous record's tail (the inverse and
    // W), the later ones one block ahead.
    KIn blk[2];
    if (have) {
        load_block(u, c, 0, blk[0]);
        if (NKS > 1) load_block(u, c, 1, blk[1]);
    }
    while (have) {
        Rec &rec = *reinterpret_cast<Rec *>(ring + (size_t)(r % D) * RS);
        const int t0 = u.bos + c * C;
        (void)t0;
        // the ring slot is free once every slice has consumed record r - D
        if (r >= D) {
            const int want = r - D + 1;
            bool ok = true;
            for (int s = 0; s < NS && ok; ++s) ok = wait_until([&] { return ld_agent(&progress[s]) >= want; }, abort_word);
            if (!ok) break;
        }
        const float b0 = token_scalar(p.beta, u, c, 0), b1 = token_scalar(p.beta, u, c, 1);
        if (lg == 0) {
            ps.beta[lr] = b0;
            ps.beta[16 + lr] = b1;
        }
        // GDN: the per-token decay, scanned once per record
        float eg[2] = {1.f, 1.f}, egc[2] = {1.f, 1.f};
        if constexpr (!KDA) {
            const float l0 = token_scalar(p.log_alpha, u, c, 0), l1 = token_scalar(p.log_alpha, u, c, 1);
            const float s0 = sum_row16(l0);
            const float x0 = scan_row16(l0), x1 = scan_row16(l1) + s0;
            const float gC = s0 + sum_row16(l1);
            eg[0] = __builtin_amdgcn_exp2f(x0 * L2E);
            eg[1] = __builtin_amdgcn_exp2f(x1 * L2E);
            egc[0] = __builtin_amdgcn_exp2f((gC - x0) * L2E);
            egc[1] = __builtin_amdgcn_exp2f((gC - x1) * L2E);
            if (lg == 0) {
                ps.g[lr] = x0;
                ps.g[16 + lr] = x1;
            }
            if (lane == 0) rec.dec[0] = __builtin_amdgcn_exp2f(gC * L2E);
        }
        // Gram accumulators: A tiles (0,0), (1,0), (1,1); M^T tiles likewise
        f32x4 a00{}, a10{}, a11{}, m00{}, m10{}, m11{};
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            const KIn &cur = blk[s % 2];
            bf16x8 lk[2], lqh[2], lql[2], rkh[2], rkl[2];
            f16x8 qt[2], kt[2], ke[2];
            if constexpr (KDA) {
                f32x4 dec4[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = 4 * hh + i;
                        // g of the two row tiles (the second carries the first's total),
                        // the chunk total g_C and the reference m = g_C / 2: every g of the
                        // chunk lies in [g_C, 0] for log-decays <= 0, so |g - m| <= |g_C| / 2,
                        // and e^m = e^{g_C - m}
                        const float l0 = cur.la[0][hh][i], l1 = cur.la[1][hh][i];
                        const float s0 = sum_row16(l0);
                        const float x0 = scan_row16(l0), x1 = scan_row16(l1) + s0;
                        const float gC = s0 + sum_row16(l1), m = 0.5f * gC;
                        const float em = __builtin_amdgcn_exp2f(m * L2E), ecm = em;
                        dec4[hh][i] = em * em;
                        const float xs[2] = {x0, x1};
#pragma unroll
                        for (int T = 0; T < 2; ++T) {
                            const float d2 = (xs[T] - m) * L2E;
                            const float E = __builtin_amdgcn_exp2f(d2), Ei = __builtin_amdgcn_exp2f(-d2);
                            const float kf = (float)cur.k[T][j], qf = (float)cur.q[T][j];
                            const float lkv = kf * E, lqv = qf * E, rkv = kf * Ei;
                            lk[T][j] = (__bf16)lkv;
                            const __bf16 qh = (__bf16)lqv, rh = (__bf16)rkv;
                            lqh[T][j] = qh;
                            lql[T][j] = (__bf16)(lqv - (float)qh);
                            rkh[T][j] = rh;
                            rkl[T][j] = (__bf16)(rkv - (float)rh);
                            qt[T][j] = (ST)(lqv * em * p.scale);
                            kt[T][j] = (ST)(lkv * em);
                            ke[T][j] = (ST)(rkv * ecm);
                        }
                    }
                if (lr == 0) {
                    *reinterpret_cast<f32x4 *>(&rec.dec[32 * s + 4 * lg]) = dec4[0];
                    *reinterpret_cast<f32x4 *>(&rec.dec[32 * s + 16 + 4 * lg]) = dec4[1];
                }
                a00 = gram_mma(a00, lk[0], rkh[0]);
                a10 = gram_mma(a10, lk[1], rkh[0]);
                a11 = gram_mma(a11, lk[1], rkh[1]);
                m00 = gram_mma(m00, rkh[0], lqh[0]);
                m00 = gram_mma(m00, rkl[0], lqh[0]);
                m00 = gram_mma(m00, rkh[0], lql[0]);
                m10 = gram_mma(m10, rkh[0], lqh[1]);
                m10 = gram_mma(m10, rkl[0], lqh[1]);
                m10 = gram_mma(m10, rkh[0], lql[1]);
                m11 = gram_mma(m11, rkh[1], lqh[1]);
                m11 = gram_mma(m11, rkl[1], lqh[1]);
                m11 = gram_mma(m11, rkh[1], lql[1]);
            } else {
#pragma unroll
                for (int T = 0; T < 2; ++T)
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float kf = (float)cur.k[T][j], qf = (float)cur.q[T][j];
                        qt[T][j] = (ST)(qf * eg[T] * p.scale);
                        kt[T][j] = (ST)(kf * eg[T]);
                        ke[T][j] = (ST)(kf * egc[T]);
                    }
                // raw k, q: the decay scales the fp32 Gram entries
                a00 = gram_mma(a00, cur.k[0], cur.k[0]);
                a10 = gram_mma(a10, cur.k[1], cur.k[0]);
                a11 = gram_mma(a11, cur.k[1], cur.k[1]);
                m00 = gram_mma(m00, cur.k[0], cur.q[0]);
                m10 = gram_mma(m10, cur.k[0], cur.q[1]);
                m11 = gram_mma(m11, cur.k[1], cur.q[1]);
            }
            // Q e^g rows; K_end^T and (K e^g)^T through the MFMA transpose
#pragma unroll
            for (int T = 0; T < 2; ++T) *reinterpret_cast<f16x8 *>(&rec.Qt[16 * T + lr][32 * s + 8 * lg]) = qt[T];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f16x8 ke8, kt8;
#pragma unroll
                for (int T = 0; T < 2; ++T) {
                    const f32x4 te = __builtin_amdgcn_mfma_f32_16x16x32_f16(ke[T], eye[hf], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    const f32x4 tk = __builtin_amdgcn_mfma_f32_16x16x32_f16(kt[T], eye[hf], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        ke8[4 * T + i] = (ST)te[i];
                        kt8[4 * T + i] = (ST)tk[i];
                    }
                }
                *reinterpret_cast<f16x8 *>(&rec.KeT[32 * s + 16 * hf + lr][8 * lg]) = ke8;
                *reinterpret_cast<f16x8 *>(&ps.KtT[32 * s + 16 * hf + lr][8 * lg]) = kt8;
            }
            // block s's inputs are consumed: its buffer takes block s + 2
            if (s + 2 < NKS) load_block(u, c, s + 2, blk[s % 2]);
        }
        // the next owned record: its first two blocks of inputs are requested now
        FusedUnit un;
        int cn = 0;
        const int rn = r + 2 * NS;
        const bool haven = locate(rn, un, cn);
        if (haven) {
            load_block(un, cn, 0, blk[0]);
            if (NKS > 1) load_block(un, cn, 1, blk[1]);
        }

        // ---- A -> LDS (strictly lower, times beta of the row); M -> ring
        {
            const f32x4 brow0 = *reinterpret_cast<const f32x4 *>(&ps.beta[4 * lg]);
            const f32x4 brow1 = *reinterpret_cast<const f32x4 *>(&ps.beta[16 + 4 * lg]);
            auto put_a = [&](const f32x4 &a, int I, int J, const f32x4 &brow) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 16 * I + 4 * lg + i, cc = 16 * J + lr;
                    float v = cc < rr ? a[i] * brow[i] : 0.f;
                    if constexpr (!KDA) v *= cc < rr ? __builtin_amdgcn_exp2f((ps.g[rr] - ps.g[cc]) * L2E) : 0.f;
                    ps.At[rr][cc] = v;
                }
            };
            put_a(a00, 0, 0, brow0);
            put_a(a10, 1, 0, brow1);
            put_a(a11, 1, 1, brow1);
            auto mval = [&](const f32x4 &m, int I, int J, int i) {
                const int rr = 16 * I + lr, cc = 16 * J + 4 * lg + i;
                float v = cc <= rr ? m[i] * p.scale : 0.f;
                if constexpr (!KDA) v *= cc <= rr ? __builtin_amdgcn_exp2f((ps.g[rr] - ps.g[cc]) * L2E) : 0.f;
                return (ST)v;
            };
            f16x8 mr0, mr1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mr0[i] = mval(m00, 0, 0, i);
                mr0[4 + i] = (ST)0.f;
                mr1[i] = mval(m10, 1, 0, i);
                mr1[4 + i] = mval(m11, 1, 1, i);
            }
            *reinterpret_cast<f16x8 *>(&rec.Mm[lr][8 * lg]) = mr0;
            *reinterpret_cast<f16x8 *>(&rec.Mm[16 + lr][8 * lg]) = mr1;
        }
        // ---- T = (I + A)^-1: diagonal blocks as (I - N)(I + N^2)(I + N^4)(I + N^8),
        // then T_10 = -T_11 A_10 T_00 (fp32 MFMA; X Y takes X as rows, Y in the
        // accumulator layout)
        f32x4 tdiag[2];
        {
            const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
            auto rows_of = [&](int I, const f32x4 &acc) {   // acc (col lr, rows 4 lg + i) -> rows
#pragma unroll
                for (int i = 0; i < 4; ++i) ps.Tt[16 * I + 4 * lg + i][16 * I + lr] = acc[i];
                RowA<float, 1> a;
                a.load(&ps.Tt[16 * I + lr][16 * I], lg);
                return a;
            };
            auto plus_eye = [&](f32x4 acc) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] += 4 * lg + i == lr ? 1.f : 0.f;
                return acc;
            };
            RowA<float, 1> nrow[2], imn[2];
            RegB<float, 1> ncol[2], b2[2], b4[2], bq;
            f32x4 n2[2], n4[2], n8[2];
#pragma unroll
            for (int I = 0; I < 2; ++I) {
                nrow[I].load(&ps.At[16 * I + lr][16 * I], lg);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    ncol[I].f[0][i] = ps.At[16 * I + 4 * lg + i][16 * I + lr];
                    imn[I].f[0][i] = (4 * lg + i == lr ? 1.f : 0.f) - nrow[I].f[0][i];
                }
                n2[I] = ncol[I].mma(z, nrow[I]);
                b2[I].set(&n2[I]);
            }
#pragma unroll
            for (int I = 0; I < 2; ++I) {
                n4[I] = b2[I].mma(z, rows_of(I, n2[I]));
                b4[I].set(&n4[I]);
            }
#pragma unroll
            for (int I = 0; I < 2; ++I) n8[I] = b4[I].mma(z, rows_of(I, n4[I]));
            f32x4 r1[2], r2[2];
#pragma unroll
            for (int I = 0; I < 2; ++I) {
                const f32x4 q = plus_eye(n2[I]);
                bq.set(&q);
                r1[I] = bq.mma(z, imn[I]);
            }
#pragma unroll
            for (int I = 0; I < 2; ++I) {
                const f32x4 q = plus_eye(n4[I]);
                bq.set(&q);
                r2[I] = bq.mma(z, rows_of(I, r1[I]));
            }
#pragma unroll
            for (int I = 0; I < 2; ++I) {
                const f32x4 q = plus_eye(n8[I]);
                bq.set(&q);
                tdiag[I] = bq.mma(z, rows_of(I, r2[I]));
            }
            // T's lower part: diagonal blocks, then T_10
#pragma unroll
            for (int I = 0; I < 2; ++I)
#pragma unroll
                for (int i = 0; i < 4; ++i) ps.Tt[16 * I + 4 * lg + i][16 * I + lr] = tdiag[I][i];
            RowA<float, 1> a10, t11;
            a10.load(&ps.At[16 + lr][0], lg);
            RegB<float, 1> t00b;
            t00b.set(&tdiag[0]);
            const f32x4 P = t00b.mma(z, a10);   // A_10 T_00
            RegB<float, 1> pb;
            pb.set(&P);
            t11.load(&ps.Tt[16 + lr][16], lg);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * lg + i > lr) t11.f[0][i] = 0.f;
            const f32x4 t10 = pb.mma(z, t11);
#pragma unroll
            for (int i = 0; i < 4; ++i) ps.Tt[16 + 4 * lg + i][lr] = -t10[i];
        }
        // ---- T diag(b) rows (also the B operand of W): token r = 16 I + lr,
        // columns {4 lg + i, 16 + 4 lg + i}
        RowA<ST, NB> tb[2];
#pragma unroll
        for (int I = 0; I < 2; ++I) {
            const int row = 16 * I + lr;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int s0 = 16 * hh + 4 * lg;
                f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f}, b = f32x4{0.f, 0.f, 0.f, 0.f};
                if (s0 <= row) {
                    t = *reinterpret_cast<const f32x4 *>(&ps.Tt[row][s0]);
                    b = *reinterpret_cast<const f32x4 *>(&ps.beta[s0]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) tb[I].f[0][4 * hh + i] = (ST)(s0 + i <= row ? t[i] * b[i] : 0.f);
            }
            tb[I].store(&rec.Tm[row][0], lg);
        }
        // ---- W_n = -T diag(b) (K e^g): W^T tiles (16 keys x 16 tokens)
#pragma unroll
        for (int s = 0; s < NKS; ++s)
#pragma unroll
            for (int I = 0; I < 2; ++I) {
                f16x8 w;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const f16x8 kta = *reinterpret_cast<const f16x8 *>(&ps.KtT[32 * s + 16 * hf + lr][8 * lg]);
                    const f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kta, tb[I].f[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[4 * hf + i] = (ST)(-acc[i]);
                }
                *reinterpret_cast<f16x8 *>(&rec.Wn[16 * I + lr][32 * s + 8 * lg]) = w;
            }
        // ---- publish: every ring store of this wave has completed
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0) (the next record's first loads land too)
        if (lane == 0) {
            if (!local) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            st_flag(&flags[r % D], r + 1, local);
        }
        r = rn;
        u = un;
        c = cn;
        have = haven;
    }
}

template <int DK, int DVS, bool KDA>
hipError_t launch_fused32_t(const FusedArgs &fa, int grid, hipStream_t st) {
    const int nflags = fa.ngroups * (fa.D + fa.NS), nxcc = fa.ngroups * fa.NS;
    hipLaunchKernelGGL(fused_ctl_init, dim3((unsigned)((nflags + nxcc + 1 + 255) / 256)), dim3(256), 0, st, fa.ctl,
                       nflags, nxcc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fused32_prefill_kernel<DK, DVS, KDA>), dim3((unsigned)grid), dim3(64 * (DVS / 16 + 3)), 0, st,
                       fa);
    return hipGetLastError();
}

}  // namespace gdr
