// gdr_api.cpp -- the C ABI of libgdr (declared in include/gdr.h): argument
// validation on the host, launch-shape selection, error reporting.  Every
// check runs before the first HIP call, so a rejected call enqueues nothing
// and needs no GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "gdr.h"
#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

gdr_status fail(gdr_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

gdr_status ok() {
    g_last_error[0] = '\0';
    return GDR_SUCCESS;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Range {
    const char *name;
    uintptr_t lo, hi;  // [lo, hi), empty when lo == hi
};

Range range(const char *name, const void *p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{name, lo, p ? lo + bytes : lo};
}

bool overlaps(const Range &a, const Range &b) {
    return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

size_t dsize(gdr_dtype t) { return t == GDR_BF16 ? 2 : 4; }

bool valid_dtype(int t) { return t == GDR_F32 || t == GDR_BF16; }
bool valid_gate(int g) { return g == GDR_GATE_HEAD || g == GDR_GATE_CHANNEL; }

gdr_status launch_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(GDR_ERROR_LAUNCH_FAILED, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

// Workspace of one prefill call: [order][chunk offsets] (packed batches only),
// the per-chunk records, and (segmented runs) the state carried between
// segments.  seg = 0: one record per chunk of every sequence (the size
// gdr_prefill_workspace_bytes reports); seg > 0 (dense batches): records of
// one segment of seg chunks at a time.
struct PrefillWorkspace {
    size_t order_off = 0, choff_off = 0, rec_off = 0, carry_off = 0, total = 0;
    long record_chunks = 0;
    int num_segments = 1, segment_chunks = 0;
};

constexpr int kMinSegmentChunks = 16;

PrefillWorkspace prefill_workspace(const gdr_prefill_shape &s, bool kda, bool bf16, int chunk, bool packed,
                                   long seg = 0) {
    PrefillWorkspace w;
    size_t off = 0;
    if (packed) {
        w.order_off = 0;
        off = round256(sizeof(int32_t) * (size_t)s.num_seqs);
        w.choff_off = off;
        off += round256(sizeof(int32_t) * ((size_t)s.num_seqs + 1));
    }
    const long ncps = ((long)s.seqlen + chunk - 1) / chunk;
    w.segment_chunks = (int)ncps;
    if (!packed && seg > 0 && seg < ncps) {
        w.segment_chunks = (int)seg;
        w.num_segments = (int)((ncps + seg - 1) / seg);
    }
    w.rec_off = off;
    w.record_chunks = packed ? ncps + s.num_seqs : (long)s.batch * w.segment_chunks;
    off += round256((size_t)w.record_chunks * (size_t)s.num_heads *
                    gdr::chunk_record_stride(s.head_dim_k, chunk, kda, bf16 ? 2 : 4));
    w.carry_off = off;
    if (w.num_segments > 1)
        off += round256((size_t)s.num_seqs * s.num_heads * s.head_dim_k * s.head_dim_v * sizeof(float));
    w.total = off;
    return w;
}

// The layout for a workspace of `bytes`: unsegmented if it fits, else (dense
// batches) the longest segment that fits; total > bytes if none does.
PrefillWorkspace fit_workspace(const gdr_prefill_shape &s, bool kda, bool bf16, int chunk, bool packed, size_t bytes) {
    PrefillWorkspace w = prefill_workspace(s, kda, bf16, chunk, packed);
    if (w.total <= bytes || packed) return w;
    long lo = kMinSegmentChunks, hi = w.segment_chunks - 1;
    PrefillWorkspace best = prefill_workspace(s, kda, bf16, chunk, packed, lo);
    if (best.total > bytes) return w;
    while (lo < hi) {   // largest segment whose layout fits
        const long mid = (lo + hi + 1) / 2;
        const PrefillWorkspace m = prefill_workspace(s, kda, bf16, chunk, packed, mid);
        if (m.total <= bytes) { lo = mid; best = m; }
        else hi = mid - 1;
    }
    return best;
}

// automatic chunk size: 32 tokens where compiled (the fastest schedule
// measured on every workload), else 16
int auto_chunk(bool bf16, bool kda, int dk) { return gdr::prefill_supported(bf16, kda, dk, 16, 32) ? 32 : 16; }


constexpr int kMaxDecodeTokens = 64;

// num_qk_heads: 0 means num_heads; else it must divide num_heads.
gdr_status resolve_qk_heads(int32_t num_heads, int32_t num_qk_heads, int &hk) {
    hk = num_qk_heads ? num_qk_heads : num_heads;
    if (hk < 1 || hk > num_heads || num_heads % hk != 0)
        return fail(GDR_ERROR_INVALID_VALUE, "num_qk_heads %d does not divide num_heads %d", num_qk_heads, num_heads);
    return GDR_SUCCESS;
}

// Validation shared by the one-token and the multi-token decode: K tokens
// per sequence, `state` holding num_slots (sequence or slot) states.  Fills
// `a` on success.
gdr_status check_decode(int32_t num_seqs, int32_t K, int32_t num_heads, int32_t num_qk_heads, int32_t dk, int32_t dv,
                        gdr_gate gate, gdr_dtype qkv_dtype, gdr_dtype gate_dtype, gdr_dtype out_dtype, const void *q,
                        const void *k, const void *v, const void *beta, const void *log_alpha,
                        const int32_t *num_tokens, const int32_t *num_commit, const int32_t *slots, float *state,
                        int32_t num_slots, float scale, void *out, gdr::DecodeArgs &a) {
    if (num_seqs < 0 || num_heads < 1 || dk < 1 || dv < 1)
        return fail(GDR_ERROR_INVALID_VALUE, "bad shape (num_seqs=%d heads=%d dk=%d dv=%d)", num_seqs, num_heads, dk,
                    dv);
    int hk = 0;
    if (resolve_qk_heads(num_heads, num_qk_heads, hk) != GDR_SUCCESS) return GDR_ERROR_INVALID_VALUE;
    if (!valid_gate(gate)) return fail(GDR_ERROR_INVALID_VALUE, "unknown gate kind %d", (int)gate);
    if (!valid_dtype(qkv_dtype) || !valid_dtype(gate_dtype) || !valid_dtype(out_dtype))
        return fail(GDR_ERROR_INVALID_VALUE, "unknown dtype (qkv=%d gate=%d out=%d)", (int)qkv_dtype,
                    (int)gate_dtype, (int)out_dtype);
    if (!(dk == 16 || dk == 32 || dk == 64 || dk == 128))
        return fail(GDR_ERROR_NOT_SUPPORTED, "head_dim_k %d not in {16, 32, 64, 128}", dk);
    if (dv % 4 != 0 || dv > 256) return fail(GDR_ERROR_NOT_SUPPORTED, "head_dim_v %d not a multiple of 4 <= 256", dv);
    if ((int64_t)num_seqs * K * num_heads > INT32_MAX || (int64_t)num_slots * num_heads > INT32_MAX)
        return fail(GDR_ERROR_INVALID_VALUE, "too many heads");
    if (num_seqs == 0) return ok();
    if (!q || !k || !v || !beta || !log_alpha || !state || !out)
        return fail(GDR_ERROR_INVALID_VALUE, "q, k, v, beta, log_alpha, state and out must be non-NULL");
    const bool kda = gate == GDR_GATE_CHANNEL;
    const size_t es = dsize(qkv_dtype), gs = dsize(gate_dtype);
    const size_t rows = (size_t)num_seqs * K;   // token rows
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(state, 16) || !aligned(log_alpha, kda ? 4 * gs : gs) ||
        !aligned(v, es) || !aligned(out, dsize(out_dtype)) || !aligned(beta, gs) || !aligned(num_tokens, 4) ||
        !aligned(num_commit, 4) || !aligned(slots, 4))
        return fail(GDR_ERROR_INVALID_VALUE, "misaligned pointer (q/k/state need 16 bytes, per-channel "
                                             "log_alpha 4 elements)");
    const Range in[] = {range("q", q, rows * hk * dk * es), range("k", k, rows * hk * dk * es),
                        range("v", v, rows * num_heads * dv * es), range("beta", beta, rows * num_heads * gs),
                        range("log_alpha", log_alpha, rows * num_heads * (kda ? dk : 1) * gs),
                        range("num_tokens", num_tokens, num_tokens ? 4 * (size_t)num_seqs : 0),
                        range("num_commit", num_commit, num_commit ? 4 * (size_t)num_seqs : 0),
                        range("state_slots", slots, slots ? 4 * (size_t)num_seqs : 0)};
    const Range rs = range("state", state, (size_t)num_slots * num_heads * dv * dk * 4);
    const Range ro = range("out", out, rows * num_heads * dv * dsize(out_dtype));
    for (const Range &r : in) {
        if (overlaps(rs, r)) return fail(GDR_ERROR_INVALID_VALUE, "state overlaps %s", r.name);
        if (overlaps(ro, r)) return fail(GDR_ERROR_INVALID_VALUE, "out overlaps %s", r.name);
    }
    if (overlaps(rs, ro)) return fail(GDR_ERROR_INVALID_VALUE, "out overlaps state");
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_qk_heads = hk;
    a.dk = dk;
    a.dv = dv;
    a.kda = kda;
    a.bf16 = qkv_dtype == GDR_BF16;
    a.out_bf16 = out_dtype == GDR_BF16;
    a.q = q; a.k = k; a.v = v;
    a.beta = beta;
    a.log_alpha = log_alpha;
    a.gate_bf16 = gate_dtype == GDR_BF16;
    a.state = state;
    a.scale = scale;
    a.out = out;
    a.max_tokens = K;
    a.num_slots = num_slots;
    a.num_tokens = num_tokens;
    a.num_commit = num_commit;
    a.slots = slots;
    return ok();
}
// Workspace of one backward call: [order][chunk offsets] (packed batches),
// the per-chunk records, the chunks' incoming states and their outgoing
// state gradients.  Packed batches size the chunk slots by the bound
// ceil(seqlen / C) + num_seqs, since the lengths live on the device.
struct BackwardWorkspace {
    size_t order_off = 0, choff_off = 0, rec_off = 0, st_off = 0, dst_off = 0, dqh_off = 0, dkh_off = 0;
    size_t bnd_off = 0, carry_off = 0, total = 0;
    long record_chunks = 0;
    int num_segments = 1;
    long segment_chunks = 0;
    bool fits = true;            // backward_workspace_within: false when nothing fits
};

// Dense batches may run the backward in time segments of at least this many
// chunks when the workspace holds less than one pass needs.
constexpr long kMinBackwardSegment = 16;

// Workspace of one pass (segment_chunks = 0 or >= the chunks per sequence),
// or of segments of segment_chunks chunks (dense batches only).
BackwardWorkspace backward_workspace(const gdr_prefill_shape &s, bool packed, long segment_chunks = 0) {
    BackwardWorkspace w;
    size_t off = 0;
    if (packed) {
        off = round256(sizeof(int32_t) * (size_t)s.num_seqs);
        w.choff_off = off;
        off += round256(sizeof(int32_t) * ((size_t)s.num_seqs + 1));
    }
    const long ncps = ((long)s.seqlen + gdr::kBackwardChunk - 1) / gdr::kBackwardChunk;
    long per_seq = ncps;
    if (!packed && segment_chunks > 0 && segment_chunks < ncps) {
        w.segment_chunks = segment_chunks;
        w.num_segments = (int)((ncps + segment_chunks - 1) / segment_chunks);
        per_seq = segment_chunks;
    }
    w.record_chunks = packed ? ncps + s.num_seqs : (long)s.batch * per_seq;
    const size_t slots = (size_t)w.record_chunks * (size_t)s.num_heads;
    const size_t state_bytes = (size_t)s.head_dim_k * s.head_dim_v * sizeof(float);
    w.rec_off = off;
    off += round256(slots * gdr::backward_record_bytes(s.head_dim_k));
    w.st_off = off;
    off += round256(slots * state_bytes);
    w.dst_off = off;
    off += round256(slots * state_bytes);
    if (w.num_segments > 1) {
        // the states entering segments 1 .. NS - 1, and two carried gradient sets
        const size_t set = (size_t)s.num_seqs * s.num_heads * state_bytes;
        w.bnd_off = off;
        off += round256((size_t)(w.num_segments - 1) * set);
        w.carry_off = off;
        off += round256(2 * set);
    }
    // grouped q/k heads: per-value-head dq and dk before the sum over each group
    const int hk = s.num_qk_heads > 0 ? s.num_qk_heads : s.num_heads;
    if (hk != s.num_heads) {
        const size_t per = round256((size_t)s.batch * s.seqlen * s.num_heads * s.head_dim_k * sizeof(float));
        w.dqh_off = off;
        w.dkh_off = off + per;
        off += 2 * per;
    }
    w.total = off;
    return w;
}

// Segment length for NS segments of (nearly) equal length, at least the
// minimum: ceil(ncps / NS) chunks, the last segment taking what remains.
long backward_segment_length(long ncps, long NS) {
    return std::max(kMinBackwardSegment, (ncps + NS - 1) / NS);
}

// The one-pass workspace when it fits, else (dense batches) the fewest time
// segments that fit, of equal length: every segment but the last is built
// twice, so fewer and shorter segments cost less; fits = false when none do.
BackwardWorkspace backward_workspace_within(const gdr_prefill_shape &s, bool packed, size_t bytes) {
    BackwardWorkspace one = backward_workspace(s, packed);
    one.fits = one.total <= bytes;
    if (one.fits || packed) return one;
    const long ncps = ((long)s.seqlen + gdr::kBackwardChunk - 1) / gdr::kBackwardChunk;
    for (long NS = 2; ncps > kMinBackwardSegment; ++NS) {
        const long S = backward_segment_length(ncps, NS);
        if ((ncps + S - 1) / S == NS) {          // (else a longer NS repeats a shorter one's S)
            const BackwardWorkspace w = backward_workspace(s, packed, S);
            if (w.total <= bytes) return w;
        }
        if (S == kMinBackwardSegment) break;     // more segments would not be shorter
    }
    one.fits = false;
    return one;
}

}  // namespace

extern "C" {

size_t gdr_prefill_backward_workspace_bytes(const gdr_prefill_shape *shape, gdr_gate gate, int32_t packed) {
    if (!shape || !valid_gate(gate)) return 0;
    const gdr_prefill_shape &s = *shape;
    if (s.batch < 1 || s.seqlen < 0 || s.num_heads < 1 || s.head_dim_k < 1 || s.head_dim_v < 1 || s.num_seqs < 0)
        return 0;
    return backward_workspace(s, packed != 0).total;
}

size_t gdr_prefill_backward_segment_workspace_bytes(const gdr_prefill_shape *shape, gdr_gate gate,
                                                    int32_t segment_chunks) {
    if (!shape || !valid_gate(gate)) return 0;
    const gdr_prefill_shape &s = *shape;
    if (s.batch < 1 || s.seqlen < 0 || s.num_heads < 1 || s.head_dim_k < 1 || s.head_dim_v < 1 || s.num_seqs < 0)
        return 0;
    if (segment_chunks < kMinBackwardSegment) return 0;
    return backward_workspace(s, false, segment_chunks).total;
}

gdr_status gdr_prefill_backward(const gdr_prefill_shape *shape, gdr_gate gate, gdr_dtype qkv_dtype,
                                gdr_dtype gate_dtype, const void *q, const void *k, const void *v, const void *beta,
                                const void *log_alpha, const float *initial_state, const int32_t *cu_seqlens,
                                float scale, const float *d_out, const float *d_final_state, float *dq,
                                float *dk_out, float *dv_out, float *dbeta, float *dlog_alpha,
                                float *d_initial_state, void *workspace, size_t workspace_bytes,
                                void *hip_stream) {
    if (!shape) return fail(GDR_ERROR_INVALID_VALUE, "shape is NULL");
    const gdr_prefill_shape s = *shape;
    if (s.batch < 1 || s.seqlen < 0 || s.num_heads < 1 || s.head_dim_k < 1 || s.head_dim_v < 1 || s.num_seqs < 0)
        return fail(GDR_ERROR_INVALID_VALUE,
                    "bad shape (batch=%d seqlen=%d heads=%d dk=%d dv=%d num_seqs=%d)", s.batch, s.seqlen,
                    s.num_heads, s.head_dim_k, s.head_dim_v, s.num_seqs);
    int hk = 0;
    if (resolve_qk_heads(s.num_heads, s.num_qk_heads, hk) != GDR_SUCCESS) return GDR_ERROR_INVALID_VALUE;
    if (!valid_gate(gate)) return fail(GDR_ERROR_INVALID_VALUE, "unknown gate kind %d", (int)gate);
    if (!valid_dtype(qkv_dtype) || !valid_dtype(gate_dtype))
        return fail(GDR_ERROR_INVALID_VALUE, "unknown dtype (qkv=%d gate=%d)", (int)qkv_dtype, (int)gate_dtype);
    const bool packed = cu_seqlens != nullptr;
    if (packed && s.batch != 1) return fail(GDR_ERROR_INVALID_VALUE, "cu_seqlens requires batch == 1");
    if (!packed && s.num_seqs != s.batch)
        return fail(GDR_ERROR_INVALID_VALUE, "dense batch needs num_seqs == batch (%d != %d)", s.num_seqs, s.batch);
    if (packed && s.num_seqs == 0 && s.seqlen > 0)
        return fail(GDR_ERROR_INVALID_VALUE, "packed tokens need at least one sequence");
    const int64_t tokens = (int64_t)s.batch * s.seqlen;
    if (tokens > INT32_MAX) return fail(GDR_ERROR_INVALID_VALUE, "more than 2^31-1 tokens");
    if ((int64_t)s.num_seqs * s.num_heads * (s.head_dim_v / 16) > INT32_MAX)
        return fail(GDR_ERROR_INVALID_VALUE, "too many (sequence, head) units");
    if (s.num_heads > 65535) return fail(GDR_ERROR_NOT_SUPPORTED, "more than 65535 heads");
    const int dk = s.head_dim_k, dv = s.head_dim_v;
    const bool bf16 = qkv_dtype == GDR_BF16, kda = gate == GDR_GATE_CHANNEL;
    if (!gdr::backward_supported(dk, dv))
        return fail(GDR_ERROR_NOT_SUPPORTED, "backward needs head_dim_k in {32, 64, 128} and head_dim_v in {32, 64, "
                    "96, 128} (got %d, %d)", dk, dv);

    const size_t es = dsize(qkv_dtype);
    const size_t nq = (size_t)tokens * hk * dk, nv = (size_t)tokens * s.num_heads * dv;
    const size_t ng = (size_t)tokens * s.num_heads, nla = kda ? ng * dk : ng;
    const size_t nstate = (size_t)s.num_seqs * s.num_heads * dv * dk;
    if (tokens > 0 && (!q || !k || !v || !beta || !log_alpha || !d_out || !dq || !dk_out || !dv_out || !dbeta ||
                       !dlog_alpha))
        return fail(GDR_ERROR_INVALID_VALUE, "q, k, v, beta, log_alpha, d_out and the five gradients must be non-NULL");
    const void *aligned16[] = {q, k, v, d_out, initial_state, d_final_state, d_initial_state, dq, dk_out};
    const char *names16[] = {"q", "k", "v", "d_out", "initial_state", "d_final_state", "d_initial_state", "dq", "dk"};
    for (int i = 0; i < 9; ++i)
        if (!aligned(aligned16[i], 16)) return fail(GDR_ERROR_INVALID_VALUE, "%s is not 16-byte aligned", names16[i]);
    const size_t gs = dsize(gate_dtype);
    const void *aligned4[] = {dv_out, dbeta, dlog_alpha, cu_seqlens};
    for (const void *p : aligned4)
        if (!aligned(p, 4)) return fail(GDR_ERROR_INVALID_VALUE, "gradients and cu_seqlens must be 4-byte aligned");
    if (!aligned(beta, gs)) return fail(GDR_ERROR_INVALID_VALUE, "beta must be %zu-byte aligned", gs);
    if (!aligned(log_alpha, kda ? 4 * gs : gs))
        return fail(GDR_ERROR_INVALID_VALUE, "log_alpha must be %zu-byte aligned", kda ? 4 * gs : gs);

    const BackwardWorkspace full = backward_workspace(s, packed);
    const BackwardWorkspace ws = backward_workspace_within(s, packed, workspace_bytes);
    if ((full.record_chunks + 8) * s.num_heads >= INT32_MAX)
        return fail(GDR_ERROR_NOT_SUPPORTED, "more than 2^31 (chunk, head) records");
    if (!ws.fits) {
        const long ncps = ((long)s.seqlen + gdr::kBackwardChunk - 1) / gdr::kBackwardChunk;
        if (packed || ncps <= kMinBackwardSegment)
            return fail(GDR_ERROR_INSUFFICIENT_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes,
                        full.total);
        return fail(GDR_ERROR_INSUFFICIENT_WORKSPACE,
                    "workspace %zu bytes < %zu needed (one pass), or %zu for segments of %ld chunks",
                    workspace_bytes, full.total, backward_workspace(s, packed, kMinBackwardSegment).total,
                    kMinBackwardSegment);
    }
    if (ws.total && !workspace) return fail(GDR_ERROR_INVALID_VALUE, "workspace is NULL");
    if (ws.total && !aligned(workspace, 256)) return fail(GDR_ERROR_INVALID_VALUE, "workspace is not 256-byte aligned");

    const Range in[] = {range("q", q, nq * es), range("k", k, nq * es), range("v", v, nv * es),
                        range("beta", beta, ng * gs), range("log_alpha", log_alpha, nla * gs),
                        range("initial_state", initial_state, nstate * 4),
                        range("cu_seqlens", cu_seqlens, packed ? 4 * ((size_t)s.num_seqs + 1) : 0),
                        range("d_out", d_out, nv * 4), range("d_final_state", d_final_state, nstate * 4)};
    const Range outs[] = {range("dq", dq, nq * 4), range("dk", dk_out, nq * 4), range("dv", dv_out, nv * 4),
                          range("dbeta", dbeta, ng * 4), range("dlog_alpha", dlog_alpha, nla * 4),
                          range("d_initial_state", d_initial_state, nstate * 4),
                          range("workspace", workspace, ws.total)};
    for (const Range &o : outs) {
        for (const Range &r : in)
            if (overlaps(o, r)) return fail(GDR_ERROR_INVALID_VALUE, "%s overlaps %s", o.name, r.name);
        for (const Range &o2 : outs)
            if (&o2 != &o && overlaps(o, o2)) return fail(GDR_ERROR_INVALID_VALUE, "%s overlaps %s", o.name, o2.name);
    }
    if (tokens == 0 && !d_initial_state) return ok();

    gdr::BackwardArgs a{};
    a.batch = s.batch;
    a.seqlen = s.seqlen;
    a.num_heads = s.num_heads;
    a.num_qk_heads = hk;
    a.dk = dk;
    a.dv = dv;
    a.num_seqs = s.num_seqs;
    a.kda = kda;
    a.bf16 = bf16;
    a.gate_bf16 = gate_dtype == GDR_BF16;
    a.q = q; a.k = k; a.v = v;
    a.beta = beta;
    a.log_alpha = log_alpha;
    a.initial_state = initial_state;
    a.cu_seqlens = cu_seqlens;
    a.scale = scale;
    a.d_out = d_out;
    a.d_final_state = d_final_state;
    a.dq = dq; a.dk_out = dk_out; a.dv_out = dv_out;
    a.dbeta = dbeta;
    a.dlog_alpha = dlog_alpha;
    a.d_initial_state = d_initial_state;
    char *wsb = static_cast<char *>(workspace);
    a.order = packed ? reinterpret_cast<int32_t *>(wsb + ws.order_off) : nullptr;
    a.chunk_offset = packed ? reinterpret_cast<int32_t *>(wsb + ws.choff_off) : nullptr;
    a.records = wsb ? reinterpret_cast<float *>(wsb + ws.rec_off) : nullptr;
    a.states = wsb ? reinterpret_cast<float *>(wsb + ws.st_off) : nullptr;
    a.dstates = wsb ? reinterpret_cast<float *>(wsb + ws.dst_off) : nullptr;
    a.dq_heads = hk != s.num_heads ? reinterpret_cast<float *>(wsb + ws.dqh_off) : nullptr;
    a.dk_heads = hk != s.num_heads ? reinterpret_cast<float *>(wsb + ws.dkh_off) : nullptr;
    a.record_chunks = ws.record_chunks;
    a.num_segments = ws.num_segments;
    a.segment_chunks = ws.segment_chunks;
    a.boundary_states = ws.num_segments > 1 ? reinterpret_cast<float *>(wsb + ws.bnd_off) : nullptr;
    a.carry = ws.num_segments > 1 ? reinterpret_cast<float *>(wsb + ws.carry_off) : nullptr;
    return launch_status(gdr::launch_backward(a, static_cast<hipStream_t>(hip_stream)), "gdr_prefill_backward");
}

const char *gdr_status_string(gdr_status s) {
    switch (s) {
        case GDR_SUCCESS: return "success";
        case GDR_ERROR_INVALID_VALUE: return "invalid value";
        case GDR_ERROR_NOT_SUPPORTED: return "not supported";
        case GDR_ERROR_INSUFFICIENT_WORKSPACE: return "insufficient workspace";
        case GDR_ERROR_LAUNCH_FAILED: return "launch failed";
    }
    return "unknown status";
}

const char *gdr_last_error(void) { return g_last_error; }

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

uint64_t gdr_state_bytes(int64_t num_seqs, int64_t num_heads, int64_t head_dim_k, int64_t head_dim_v) {
    if (num_seqs < 0 || num_heads < 0 || head_dim_k < 0 || head_dim_v < 0) return 0;
    return (uint64_t)num_seqs * (uint64_t)num_heads * (uint64_t)head_dim_k * (uint64_t)head_dim_v * sizeof(float);
}

size_t gdr_prefill_workspace_bytes(const gdr_prefill_shape *shape, gdr_gate gate, gdr_dtype qkv_dtype,
                                   int32_t chunk_size, int32_t packed) {
    if (!shape || !valid_gate(gate) || !valid_dtype(qkv_dtype)) return 0;
    const gdr_prefill_shape &s = *shape;
    if (s.batch < 1 || s.seqlen < 0 || s.num_heads < 1 || s.head_dim_k < 1 || s.num_seqs < 0) return 0;
    if (chunk_size != 0 && chunk_size != 16 && chunk_size != 32 && chunk_size != 64) return 0;
    const bool bf16 = qkv_dtype == GDR_BF16, kda = gate == GDR_GATE_CHANNEL;
    const int C = chunk_size ? chunk_size : auto_chunk(bf16, kda, s.head_dim_k);
    return prefill_workspace(s, kda, bf16, C, packed != 0).total;
}

gdr_status gdr_prefill_chunked(const gdr_prefill_shape *shape, gdr_gate gate, gdr_dtype qkv_dtype,
                               gdr_dtype gate_dtype, gdr_dtype out_dtype, const void *q, const void *k, const void *v,
                               const void *beta, const void *log_alpha, const float *initial_state,
                               const int32_t *cu_seqlens, int32_t chunk_size, int32_t dv_slice, float scale,
                               void *out, float *final_state, void *workspace, size_t workspace_bytes,
                               void *hip_stream) {
    if (!shape) return fail(GDR_ERROR_INVALID_VALUE, "shape is NULL");
    const gdr_prefill_shape s = *shape;
    if (s.batch < 1 || s.seqlen < 0 || s.num_heads < 1 || s.head_dim_k < 1 || s.head_dim_v < 1 || s.num_seqs < 0)
        return fail(GDR_ERROR_INVALID_VALUE,
                    "bad shape (batch=%d seqlen=%d heads=%d dk=%d dv=%d num_seqs=%d)", s.batch, s.seqlen,
                    s.num_heads, s.head_dim_k, s.head_dim_v, s.num_seqs);
    int hk = 0;
    if (resolve_qk_heads(s.num_heads, s.num_qk_heads, hk) != GDR_SUCCESS) return GDR_ERROR_INVALID_VALUE;
    if (!valid_gate(gate)) return fail(GDR_ERROR_INVALID_VALUE, "unknown gate kind %d", (int)gate);
    if (!valid_dtype(qkv_dtype) || !valid_dtype(gate_dtype) || !valid_dtype(out_dtype))
        return fail(GDR_ERROR_INVALID_VALUE, "unknown dtype (qkv=%d gate=%d out=%d)", (int)qkv_dtype,
                    (int)gate_dtype, (int)out_dtype);
    const bool packed = cu_seqlens != nullptr;
    if (packed && s.batch != 1) return fail(GDR_ERROR_INVALID_VALUE, "cu_seqlens requires batch == 1");
    if (!packed && s.num_seqs != s.batch)
        return fail(GDR_ERROR_INVALID_VALUE, "dense batch needs num_seqs == batch (%d != %d)", s.num_seqs, s.batch);
    if (packed && s.num_seqs == 0 && s.seqlen > 0)
        return fail(GDR_ERROR_INVALID_VALUE, "packed tokens need at least one sequence");
    const int64_t tokens = (int64_t)s.batch * s.seqlen;
    if (tokens > INT32_MAX) return fail(GDR_ERROR_INVALID_VALUE, "more than 2^31-1 tokens");
    if ((int64_t)s.num_seqs * s.num_heads > INT32_MAX / 8)
        return fail(GDR_ERROR_INVALID_VALUE, "too many (sequence, head) units");
    const int dk = s.head_dim_k, dv = s.head_dim_v;
    const bool bf16 = qkv_dtype == GDR_BF16;
    const bool kda = gate == GDR_GATE_CHANNEL;
    if (!(dk == 16 || dk == 32 || dk == 64 || dk == 128))
        return fail(GDR_ERROR_NOT_SUPPORTED, "head_dim_k %d not in {16, 32, 64, 128}", dk);
    if (dv % 16 != 0 || dv > 256) return fail(GDR_ERROR_NOT_SUPPORTED, "head_dim_v %d not a multiple of 16 <= 256", dv);
    if (chunk_size != 0 && chunk_size != 16 && chunk_size != 32 && chunk_size != 64)
        return fail(GDR_ERROR_INVALID_VALUE, "chunk_size %d not in {0, 16, 32, 64}", chunk_size);
    if (dv_slice != 0 && dv_slice != 16 && dv_slice != 32 && dv_slice != 64)
        return fail(GDR_ERROR_INVALID_VALUE, "dv_slice %d not in {0, 16, 32, 64}", dv_slice);
    if (dv_slice != 0 && dv % dv_slice != 0)
        return fail(GDR_ERROR_INVALID_VALUE, "dv_slice %d does not divide head_dim_v %d", dv_slice, dv);
    // automatic choices: 32-token chunks (16 where 32 is not compiled); the
    // value-slice width that needs the fewest rounds of chain workgroups
    int C = chunk_size;
    if (!C) C = auto_chunk(bf16, kda, dk);
    int DVS = dv_slice;
    if (!DVS) DVS = gdr::auto_dv_slice(bf16, kda, dk, dv, C, (long)s.num_seqs * s.num_heads);
    if (!gdr::prefill_supported(bf16, kda, dk, DVS, C))
        return fail(GDR_ERROR_NOT_SUPPORTED, "no prefill kernel for %s dk=%d dv_slice=%d chunk=%d",
                    bf16 ? "bf16" : "fp32", dk, DVS, C);

    const size_t es = dsize(qkv_dtype), gs = dsize(gate_dtype);
    const size_t nq = (size_t)tokens * hk * dk, nv = (size_t)tokens * s.num_heads * dv;
    const size_t ng = (size_t)tokens * s.num_heads;
    const size_t nla = kda ? ng * dk : ng;
    const size_t nstate = (size_t)s.num_seqs * s.num_heads * dv * dk;
    if (tokens > 0 && (!q || !k || !v || !beta || !log_alpha || !out))
        return fail(GDR_ERROR_INVALID_VALUE, "q, k, v, beta, log_alpha and out must be non-NULL");
    const void *aligned16[] = {q, k, v, out, initial_state, final_state};
    const char *names16[] = {"q", "k", "v", "out", "initial_state", "final_state"};
    for (int i = 0; i < 6; ++i)
        if (!aligned(aligned16[i], 16)) return fail(GDR_ERROR_INVALID_VALUE, "%s is not 16-byte aligned", names16[i]);
    if (!aligned(beta, gs) || !aligned(log_alpha, kda ? 4 * gs : gs) || !aligned(cu_seqlens, 4))
        return fail(GDR_ERROR_INVALID_VALUE, "beta must be %zu-byte aligned, cu_seqlens 4-byte, log_alpha %zu-byte",
                    gs, kda ? 4 * gs : gs);

    const PrefillWorkspace ws = fit_workspace(s, kda, bf16, C, packed, workspace_bytes);
    if ((ws.record_chunks + 8) * s.num_heads >= INT32_MAX)
        return fail(GDR_ERROR_NOT_SUPPORTED, "more than 2^31 (chunk, head) records in one pass");
    const size_t need_ws = ws.total;
    if (workspace_bytes < need_ws)
        return fail(GDR_ERROR_INSUFFICIENT_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need_ws);
    if (need_ws && !workspace) return fail(GDR_ERROR_INVALID_VALUE, "workspace is NULL");
    if (need_ws && !aligned(workspace, 256)) return fail(GDR_ERROR_INVALID_VALUE, "workspace is not 256-byte aligned");

    const Range in[] = {range("q", q, nq * es), range("k", k, nq * es), range("v", v, nv * es),
                        range("beta", beta, ng * gs), range("log_alpha", log_alpha, nla * gs),
                        range("initial_state", initial_state, nstate * 4),
                        range("cu_seqlens", cu_seqlens, packed ? 4 * ((size_t)s.num_seqs + 1) : 0)};
    const Range ro = range("out", out, nv * dsize(out_dtype));
    const Range rf = range("final_state", final_state, final_state ? nstate * 4 : 0);
    const Range rw = range("workspace", workspace, need_ws);
    for (const Range &r : in) {
        if (overlaps(ro, r)) return fail(GDR_ERROR_INVALID_VALUE, "out overlaps %s", r.name);
        if (overlaps(rw, r)) return fail(GDR_ERROR_INVALID_VALUE, "workspace overlaps %s", r.name);
        if (overlaps(rf, r) && !(r.lo == reinterpret_cast<uintptr_t>(initial_state) && final_state == initial_state))
            return fail(GDR_ERROR_INVALID_VALUE, "final_state overlaps %s", r.name);
    }
    if (overlaps(ro, rf) || overlaps(ro, rw) || overlaps(rf, rw))
        return fail(GDR_ERROR_INVALID_VALUE, "out, final_state and workspace must not overlap");

    if (tokens == 0 && !final_state) return ok();
    gdr::PrefillArgs a{};
    a.batch = s.batch;
    a.seqlen = s.seqlen;
    a.num_heads = s.num_heads;
    a.num_qk_heads = hk;
    a.dk = dk;
    a.dv = dv;
    a.num_seqs = s.num_seqs;
    a.kda = kda;
    a.bf16 = bf16;
    a.out_bf16 = out_dtype == GDR_BF16;
    a.chunk = C;
    a.dv_slice = DVS;
    a.q = q; a.k = k; a.v = v;
    a.beta = beta;
    a.log_alpha = log_alpha;
    a.gate_bf16 = gate_dtype == GDR_BF16;
    a.initial_state = initial_state;
    a.cu_seqlens = cu_seqlens;
    a.scale = scale;
    a.out = out;
    a.final_state = final_state;
    char *wsb = static_cast<char *>(workspace);
    a.order = packed ? reinterpret_cast<int32_t *>(wsb + ws.order_off) : nullptr;
    a.chunk_offset = packed ? reinterpret_cast<int32_t *>(wsb + ws.choff_off) : nullptr;
    a.records = wsb ? wsb + ws.rec_off : nullptr;
    a.record_chunks = ws.record_chunks;
    a.num_segments = ws.num_segments;
    a.segment_chunks = ws.segment_chunks;
    a.carry = wsb ? reinterpret_cast<float *>(wsb + ws.carry_off) : nullptr;
    return launch_status(gdr::launch_prefill(a, static_cast<hipStream_t>(hip_stream)), "gdr_prefill_chunked");
}

gdr_status gdr_prefill_chunked_static(const gdr_prefill_shape *shape, gdr_gate gate, gdr_dtype qkv_dtype,
                                      gdr_dtype gate_dtype, gdr_dtype out_dtype, const void *q, const void *k,
                                      const void *v, const void *beta, const void *log_alpha,
                                      const float *initial_state, const int32_t *cu_seqlens, int32_t chunk_size,
                                      int32_t dv_slice, float scale, void *out, float *final_state,
                                      void *hip_stream) {
    void *ws = nullptr;
    const hipError_t e = gdr::static_scratch(&ws);
    if (e != hipSuccess)
        return fail(GDR_ERROR_LAUNCH_FAILED, "gdr_prefill_chunked_static: static scratch address: %s", hipGetErrorString(e));
    const gdr_status st = gdr_prefill_chunked(shape, gate, qkv_dtype, gate_dtype, out_dtype, q, k, v, beta, log_alpha,
                                              initial_state, cu_seqlens, chunk_size, dv_slice, scale, out, final_state,
                                              ws, gdr::kStaticScratchBytes, hip_stream);
    if (st == GDR_ERROR_INSUFFICIENT_WORKSPACE) {
        char why[sizeof(g_last_error)];
        snprintf(why, sizeof why, "%s", g_last_error);
        return fail(st, "gdr_prefill_chunked_static: the problem needs more than the %zu-byte static scratch (%s)",
                    gdr::kStaticScratchBytes, why);
    }
    return st;
}

gdr_status gdr_decode_step(int32_t num_seqs, int32_t num_heads, int32_t num_qk_heads, int32_t head_dim_k,
                           int32_t head_dim_v, gdr_gate gate, gdr_dtype qkv_dtype, gdr_dtype gate_dtype,
                           gdr_dtype out_dtype, const void *q, const void *k, const void *v, const void *beta,
                           const void *log_alpha, float *state, float scale, void *out, void *hip_stream) {
    gdr::DecodeArgs a{};
    const gdr_status st = check_decode(num_seqs, 1, num_heads, num_qk_heads, head_dim_k, head_dim_v, gate, qkv_dtype,
                                       gate_dtype, out_dtype, q, k, v, beta, log_alpha, nullptr, nullptr, nullptr,
                                       state, num_seqs, scale, out, a);
    if (st != GDR_SUCCESS || num_seqs == 0) return st;
    return launch_status(gdr::launch_decode(a, static_cast<hipStream_t>(hip_stream)), "gdr_decode_step");
}

gdr_status gdr_decode_tokens(int32_t num_seqs, int32_t max_tokens, int32_t num_heads, int32_t num_qk_heads,
                             int32_t head_dim_k, int32_t head_dim_v, gdr_gate gate, gdr_dtype qkv_dtype,
                             gdr_dtype gate_dtype, gdr_dtype out_dtype, const void *q, const void *k,
                             const void *v, const void *beta, const void *log_alpha, const int32_t *num_tokens,
                             const int32_t *num_commit, const int32_t *state_slots, float *state_pool,
                             int32_t num_slots, float scale, void *out, void *hip_stream) {
    if (max_tokens < 1 || max_tokens > kMaxDecodeTokens)
        return fail(GDR_ERROR_INVALID_VALUE, "max_tokens %d not in [1, %d]", max_tokens, kMaxDecodeTokens);
    if (num_slots < 0) return fail(GDR_ERROR_INVALID_VALUE, "num_slots %d < 0", num_slots);
    if (!state_slots && num_slots < num_seqs)
        return fail(GDR_ERROR_INVALID_VALUE, "without state_slots the pool needs num_seqs slots (%d < %d)", num_slots,
                    num_seqs);
    gdr::DecodeArgs a{};
    const gdr_status st = check_decode(num_seqs, max_tokens, num_heads, num_qk_heads, head_dim_k, head_dim_v, gate,
                                       qkv_dtype, gate_dtype, out_dtype, q, k, v, beta, log_alpha, num_tokens,
                                       num_commit, state_slots, state_pool, num_slots, scale, out, a);
    if (st != GDR_SUCCESS || num_seqs == 0) return st;
    return launch_status(gdr::launch_decode_tokens(a, static_cast<hipStream_t>(hip_stream)), "gdr_decode_tokens");
}

gdr_status gdr_layer_prologue(const gdr_prefill_shape *shape, gdr_gate gate, gdr_dtype x_dtype, const void *x,
                              const float *conv_weight, const void *conv_state_in, void *conv_state_out,
                              const int32_t *cu_seqlens, int32_t flags, const float *a_logit, const float *b_logit,
                              void *q, void *k, void *v, float *beta, float *log_alpha, void *hip_stream) {
    if (!shape) return fail(GDR_ERROR_INVALID_VALUE, "shape is NULL");
    const gdr_prefill_shape s = *shape;
    if (s.batch < 1 || s.seqlen < 0 || s.num_heads < 1 || s.head_dim_k < 1 || s.head_dim_v < 1 || s.num_seqs < 0)
        return fail(GDR_ERROR_INVALID_VALUE, "bad shape (batch=%d seqlen=%d heads=%d dk=%d dv=%d num_seqs=%d)",
                    s.batch, s.seqlen, s.num_heads, s.head_dim_k, s.head_dim_v, s.num_seqs);
    int hk = 0;
    if (resolve_qk_heads(s.num_heads, s.num_qk_heads, hk) != GDR_SUCCESS) return GDR_ERROR_INVALID_VALUE;
    if (!valid_gate(gate)) return fail(GDR_ERROR_INVALID_VALUE, "unknown gate kind %d", (int)gate);
    if (!valid_dtype(x_dtype)) return fail(GDR_ERROR_INVALID_VALUE, "unknown dtype %d", (int)x_dtype);
    if (flags & ~(GDR_PROLOGUE_SILU | GDR_PROLOGUE_QK_NORM))
        return fail(GDR_ERROR_INVALID_VALUE, "unknown flags 0x%x", (unsigned)flags);
    const bool packed = cu_seqlens != nullptr;
    if (packed && s.batch != 1) return fail(GDR_ERROR_INVALID_VALUE, "cu_seqlens requires batch == 1");
    if (!packed && s.num_seqs != s.batch)
        return fail(GDR_ERROR_INVALID_VALUE, "dense batch needs num_seqs == batch (%d != %d)", s.num_seqs, s.batch);
    if (packed && s.num_seqs == 0 && s.seqlen > 0)
        return fail(GDR_ERROR_INVALID_VALUE, "packed tokens need at least one sequence");
    const int dk = s.head_dim_k, dv = s.head_dim_v;
    if (!(dk == 16 || dk == 32 || dk == 64 || dk == 128))
        return fail(GDR_ERROR_NOT_SUPPORTED, "head_dim_k %d not in {16, 32, 64, 128}", dk);
    if (dv % 8 != 0) return fail(GDR_ERROR_NOT_SUPPORTED, "head_dim_v %d not a multiple of 8", dv);
    const int64_t tokens = (int64_t)s.batch * s.seqlen;
    const int64_t C = 2 * (int64_t)hk * dk + (int64_t)s.num_heads * dv;
    if (tokens > INT32_MAX || C > INT32_MAX / 8) return fail(GDR_ERROR_INVALID_VALUE, "problem too large");
    const bool kda = gate == GDR_GATE_CHANNEL;
    if (tokens > 0 && (!x || !conv_weight || !a_logit || !b_logit || !q || !k || !v || !beta || !log_alpha))
        return fail(GDR_ERROR_INVALID_VALUE, "x, conv_weight, a_logit, b_logit, q, k, v, beta and log_alpha must be non-NULL");
    const void *a16[] = {x, conv_weight, conv_state_in, conv_state_out, q, k, v};
    const char *n16[] = {"x", "conv_weight", "conv_state_in", "conv_state_out", "q", "k", "v"};
    for (int i = 0; i < 7; ++i)
        if (!aligned(a16[i], 16)) return fail(GDR_ERROR_INVALID_VALUE, "%s is not 16-byte aligned", n16[i]);
    if (!aligned(a_logit, 4) || !aligned(b_logit, 4) || !aligned(beta, 4) || !aligned(log_alpha, 4) ||
        !aligned(cu_seqlens, 4))
        return fail(GDR_ERROR_INVALID_VALUE, "gates and cu_seqlens must be 4-byte aligned");
    const size_t es = dsize(x_dtype), ng = (size_t)tokens * s.num_heads, na = kda ? ng * dk : ng;
    const size_t st_bytes = (size_t)s.num_seqs * 3 * C * es;
    const Range in[] = {range("x", x, (size_t)tokens * C * es), range("conv_weight", conv_weight, (size_t)C * 16),
                        range("conv_state_in", conv_state_in, conv_state_in ? st_bytes : 0),
                        range("a_logit", a_logit, na * 4), range("b_logit", b_logit, ng * 4),
                        range("cu_seqlens", cu_seqlens, packed ? 4 * ((size_t)s.num_seqs + 1) : 0)};
    const Range outs[] = {range("q", q, (size_t)tokens * hk * dk * es), range("k", k, (size_t)tokens * hk * dk * es),
                          range("v", v, (size_t)tokens * s.num_heads * dv * es), range("beta", beta, ng * 4),
                          range("log_alpha", log_alpha, na * 4),
                          range("conv_state_out", conv_state_out, conv_state_out ? st_bytes : 0)};
    for (const Range &o : outs) {
        for (const Range &r : in) {
            const bool same_state = o.lo == reinterpret_cast<uintptr_t>(conv_state_out) &&
                                    r.lo == reinterpret_cast<uintptr_t>(conv_state_in) && conv_state_in == conv_state_out;
            if (overlaps(o, r) && !same_state) return fail(GDR_ERROR_INVALID_VALUE, "%s overlaps %s", o.name, r.name);
        }
        for (const Range &o2 : outs)
            if (&o2 != &o && overlaps(o, o2)) return fail(GDR_ERROR_INVALID_VALUE, "%s overlaps %s", o.name, o2.name);
    }
    if (tokens == 0 && !conv_state_out) return ok();
    gdr::PrologueArgs a{};
    a.batch = s.batch;
    a.seqlen = s.seqlen;
    a.num_seqs = s.num_seqs;
    a.num_heads = s.num_heads;
    a.num_qk_heads = hk;
    a.dk = dk;
    a.dv = dv;
    a.kda = kda;
    a.x_bf16 = x_dtype == GDR_BF16;
    a.silu = (flags & GDR_PROLOGUE_SILU) != 0;
    a.qk_norm = (flags & GDR_PROLOGUE_QK_NORM) != 0;
    a.x = x;
    a.conv_weight = conv_weight;
    a.state_in = conv_state_in;
    a.state_out = conv_state_out;
    a.cu_seqlens = cu_seqlens;
    a.a_logit = a_logit;
    a.b_logit = b_logit;
    a.q = q; a.k = k; a.v = v;
    a.beta = beta;
    a.log_alpha = log_alpha;
    return launch_status(gdr::launch_prologue(a, static_cast<hipStream_t>(hip_stream)), "gdr_layer_prologue");
}

gdr_status gdr_decode_step_prologue(int32_t num_seqs, int32_t num_heads, int32_t num_qk_heads, int32_t head_dim_k,
                                    int32_t head_dim_v, gdr_gate gate, gdr_dtype x_dtype, gdr_dtype out_dtype,
                                    const void *x, const float *conv_weight, const void *conv_state_in,
                                    void *conv_state_out, int32_t flags, const float *a_logit, const float *b_logit,
                                    float *state, float scale, void *out, void *hip_stream) {
    if (num_seqs < 0 || num_heads < 1 || head_dim_k < 1 || head_dim_v < 1)
        return fail(GDR_ERROR_INVALID_VALUE, "bad shape (num_seqs=%d heads=%d dk=%d dv=%d)", num_seqs, num_heads,
                    head_dim_k, head_dim_v);
    int hk = 0;
    if (resolve_qk_heads(num_heads, num_qk_heads, hk) != GDR_SUCCESS) return GDR_ERROR_INVALID_VALUE;
    if (!valid_gate(gate)) return fail(GDR_ERROR_INVALID_VALUE, "unknown gate kind %d", (int)gate);
    if (!valid_dtype(x_dtype) || !valid_dtype(out_dtype))
        return fail(GDR_ERROR_INVALID_VALUE, "unknown dtype (x=%d out=%d)", (int)x_dtype, (int)out_dtype);
    if (flags & ~(GDR_PROLOGUE_SILU | GDR_PROLOGUE_QK_NORM))
        return fail(GDR_ERROR_INVALID_VALUE, "unknown flags 0x%x", (unsigned)flags);
    const int dk = head_dim_k, dv = head_dim_v;
    if (!(dk == 16 || dk == 32 || dk == 64 || dk == 128))
        return fail(GDR_ERROR_NOT_SUPPORTED, "head_dim_k %d not in {16, 32, 64, 128}", dk);
    if (dv % 8 != 0 || dv > 256) return fail(GDR_ERROR_NOT_SUPPORTED, "head_dim_v %d not a multiple of 8 <= 256", dv);
    const int64_t C = 2 * (int64_t)hk * dk + (int64_t)num_heads * dv;
    if ((int64_t)num_seqs * num_heads > INT32_MAX || (int64_t)num_seqs * C > INT32_MAX)
        return fail(GDR_ERROR_INVALID_VALUE, "problem too large");
    if (num_seqs == 0) return ok();
    if (!x || !conv_weight || !a_logit || !b_logit || !state || !out)
        return fail(GDR_ERROR_INVALID_VALUE, "x, conv_weight, a_logit, b_logit, state and out must be non-NULL");
    const bool kda = gate == GDR_GATE_CHANNEL;
    const void *a16[] = {x, conv_weight, conv_state_in, conv_state_out, state, a_logit};
    const char *n16[] = {"x", "conv_weight", "conv_state_in", "conv_state_out", "state", "a_logit"};
    for (int i = 0; i < 6; ++i)
        if (!aligned(a16[i], i == 5 && !kda ? 4 : 16))
            return fail(GDR_ERROR_INVALID_VALUE, "%s is not %d-byte aligned", n16[i], i == 5 && !kda ? 4 : 16);
    if (!aligned(b_logit, 4) || !aligned(out, dsize(out_dtype)))
        return fail(GDR_ERROR_INVALID_VALUE, "b_logit and out must be aligned to their element size");
    const size_t es = dsize(x_dtype), ng = (size_t)num_seqs * num_heads;
    const size_t st_bytes = (size_t)num_seqs * 3 * C * es;
    const Range in[] = {range("x", x, (size_t)num_seqs * C * es), range("conv_weight", conv_weight, (size_t)C * 16),
                        range("conv_state_in", conv_state_in, conv_state_in ? st_bytes : 0),
                        range("a_logit", a_logit, (kda ? ng * dk : ng) * 4), range("b_logit", b_logit, ng * 4)};
    const Range outs[] = {range("state", state, ng * dv * dk * 4), range("out", out, ng * dv * dsize(out_dtype)),
                          range("conv_state_out", conv_state_out, conv_state_out ? st_bytes : 0)};
    for (const Range &o : outs) {
        for (const Range &r : in) {
            const bool same_state = o.lo == reinterpret_cast<uintptr_t>(conv_state_out) &&
                                    r.lo == reinterpret_cast<uintptr_t>(conv_state_in) && conv_state_in == conv_state_out;
            if (overlaps(o, r) && !same_state) return fail(GDR_ERROR_INVALID_VALUE, "%s overlaps %s", o.name, r.name);
        }
        for (const Range &o2 : outs)
            if (&o2 != &o && overlaps(o, o2)) return fail(GDR_ERROR_INVALID_VALUE, "%s overlaps %s", o.name, o2.name);
    }
    gdr::DecodePrologueArgs a{};
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_qk_heads = hk;
    a.dk = dk;
    a.dv = dv;
    a.kda = kda;
    a.x_bf16 = x_dtype == GDR_BF16;
    a.out_bf16 = out_dtype == GDR_BF16;
    a.silu = (flags & GDR_PROLOGUE_SILU) != 0;
    a.qk_norm = (flags & GDR_PROLOGUE_QK_NORM) != 0;
    a.x = x;
    a.conv_weight = conv_weight;
    a.conv_state_in = conv_state_in;
    a.conv_state_out = conv_state_out;
    a.a_logit = a_logit;
    a.b_logit = b_logit;
    a.state = state;
    a.scale = scale;
    a.out = out;
    return launch_status(gdr::launch_decode_prologue(a, static_cast<hipStream_t>(hip_stream)),
                         "gdr_decode_step_prologue");
}

}  // extern "C"
