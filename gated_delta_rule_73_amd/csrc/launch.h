// launch.h -- internal interface between the C-ABI layer (gdr_api.cpp) and
// the HIP kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

// num_heads value heads; value head h reads q/k head h / (num_heads / num_qk_heads)
struct DecodeArgs {
    int num_seqs, num_heads, num_qk_heads, dk, dv;
    bool kda, bf16, out_bf16;
    const void *q, *k, *v;
    const void *beta, *log_alpha;   // fp32, or bf16 when gate_bf16
    bool gate_bf16;
    float *state;                   // decode step: [num_seqs, H, dv, dk]; multi-token: the slot pool
    float scale;
    void *out;
    // multi-token decode only
    int max_tokens, num_slots;
    const int32_t *num_tokens, *num_commit, *slots;   // [num_seqs] each, or NULL
};

struct PrefillArgs {
    int batch, seqlen, num_heads, num_qk_heads, dk, dv, num_seqs;
    bool kda, bf16, out_bf16;
    int chunk, dv_slice;            // resolved (non-zero) values
    const void *q, *k, *v;
    const void *beta, *log_alpha;   // fp32, or bf16 when gate_bf16
    bool gate_bf16;
    const float *initial_state;
    const int32_t *cu_seqlens;
    float scale;
    void *out;
    float *final_state;
    // workspace (laid out by the C-ABI layer)
    int32_t *order;                 // packed only: longest-first sequence order [num_seqs]
    int32_t *chunk_offset;          // packed only: first record chunk of each sequence [num_seqs + 1]
    char *records;                  // per-chunk records, record_chunks * num_heads of them
    long record_chunks;             // chunk slots per head (one segment: all chunks)
    int num_segments;               // dense batches in a bounded workspace: chunk segments
    int segment_chunks;             //   chunks per segment (records of one segment resident)
    float *carry;                   //   state between segments [num_seqs, H, dv, dk]
};

// The prefill workspace of gdr_prefill_chunked_static (static_scratch.hip):
// one array of this size per device; static_scratch returns its address on
// the current device.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
hipError_t static_scratch(void **ptr);

// Size of one per-chunk record of the prefill (see ChunkRec in
// prefill_impl.h): decay row, K e^g, Q e^g, K_end^T, T diag(b), M.
// es = bytes per operand element (2 for fp16 operands, 4 for fp32).
constexpr size_t chunk_record_bytes(int dk, int chunk, bool kda, int es) {
    return (size_t)(kda ? dk : 4) * 4 + ((size_t)3 * chunk * dk + (size_t)2 * chunk * chunk) * (size_t)es;
}
constexpr size_t chunk_record_stride(int dk, int chunk, bool kda, int es) {
    return (chunk_record_bytes(dk, chunk, kda, es) + 255) & ~size_t(255);
}

// Layer prologue (prologue.hip): short convolution, optional SiLU and q/k
// norm, gate activations, convolution state.
struct PrologueArgs {
    int batch, seqlen, num_seqs, num_heads, num_qk_heads, dk, dv;
    bool kda, x_bf16, silu, qk_norm;
    const void *x;                  // [batch, seqlen, C], C = 2 Hk dk + H dv
    const float *conv_weight;       // [C, 4]
    const void *state_in;           // [num_seqs, 3, C] or NULL
    void *state_out;                // [num_seqs, 3, C] or NULL (may equal state_in)
    const int32_t *cu_seqlens;
    const float *a_logit, *b_logit;
    void *q, *k, *v;
    float *beta, *log_alpha;
};

// Gradients of the chunked prefill (backward.hip).  All gradients fp32.
struct BackwardArgs {
    int batch, seqlen, num_heads, num_qk_heads, dk, dv, num_seqs;
    bool kda, bf16, gate_bf16;
    const void *q, *k, *v;
    const void *beta, *log_alpha;   // fp32, or bf16 when gate_bf16
    const float *initial_state;     // [num_seqs, H, dv, dk] or NULL
    const int32_t *cu_seqlens;
    float scale;
    const float *d_out;             // [batch, seqlen, H, dv]
    const float *d_final_state;     // [num_seqs, H, dv, dk] or NULL (zeros)
    float *dq, *dk_out, *dv_out, *dbeta, *dlog_alpha;
    float *d_initial_state;         // or NULL
    // workspace (laid out by the C-ABI layer)
    int32_t *order, *chunk_offset;  // packed only
    float *records;                 // record_chunks * H records
    float *states, *dstates;        // record_chunks * H states of dv x dk each
    float *dq_heads, *dk_heads;     // grouped heads only: per-value-head dq, dk [batch, seqlen, H, dk]
    long record_chunks;             // chunk slots (packed: an upper bound; segments: one segment's)
    // dense batches in time segments (num_segments > 1): segment_chunks
    // chunks per segment; the states entering segments 1 .. num_segments - 1
    // and two state-gradient sets carried between segments
    int num_segments;
    long segment_chunks;
    float *boundary_states, *carry;
};

constexpr int kBackwardChunk = 32;
// One backward chunk record: e^{g_C} [dk], T and M [C][C], W, Q e^g and
// K_end [C][dk], fp32, padded to 256 bytes.
constexpr size_t backward_record_bytes(int dk) {
    return (((size_t)dk + 2 * kBackwardChunk * kBackwardChunk + 3 * (size_t)kBackwardChunk * dk + kBackwardChunk) * 4 +
            255) &
           ~size_t(255);
}
bool backward_supported(int dk, int dv);
hipError_t launch_backward(const BackwardArgs &a, hipStream_t st);
// Packed batches: longest-first order and first record chunk per sequence.
hipError_t launch_schedule(const int32_t *cu, int n, int chunk, int32_t *order, int32_t *chunk_offset,
                           hipStream_t st);

hipError_t launch_prologue(const PrologueArgs &a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs &p, hipStream_t st);

// Decode step with the layer prologue fused in (decode.hip): the token's
// projected channels x and the convolution state give q, k, v and the gates
// inside the decode kernel; a second small kernel then shifts the
// convolution state (so it may be updated in place).
struct DecodePrologueArgs {
    int num_seqs, num_heads, num_qk_heads, dk, dv;
    bool kda, x_bf16, out_bf16, silu, qk_norm;
    const void *x;                  // [num_seqs, C], C = 2 Hk dk + H dv
    const float *conv_weight;       // [C, 4]
    const void *conv_state_in;      // [num_seqs, 3, C] or NULL (zeros)
    void *conv_state_out;           // [num_seqs, 3, C] or NULL; may equal conv_state_in
    const float *a_logit, *b_logit; // [num_seqs, H(, dk)], [num_seqs, H]
    float *state;                   // [num_seqs, H, dv, dk]
    float scale;
    void *out;                      // [num_seqs, H, dv]
};
hipError_t launch_decode_prologue(const DecodePrologueArgs &p, hipStream_t st);
hipError_t launch_decode_tokens(const DecodeArgs &p, hipStream_t st);

// True when a prefill kernel is compiled for this combination.
bool prefill_supported(bool bf16, bool kda, int dk, int dv_slice, int chunk);
// Value-slice width when the caller passes 0: 16 or 32 (see prefill.hip).
int auto_dv_slice(bool bf16, bool kda, int dk, int dv, int chunk, long units);
hipError_t launch_prefill(const PrefillArgs &p, hipStream_t st);

}  // namespace gdr
