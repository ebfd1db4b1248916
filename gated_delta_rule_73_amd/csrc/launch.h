// launch.h -- internal interface between the C-ABI layer (gdr_api.cpp) and
// the HIP kernels.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

struct DecodeArgs {
    int num_seqs, num_heads, dk, dv;
    bool kda, bf16, out_bf16;
    const void *q, *k, *v;
    const float *beta, *log_alpha;
    float *state;
    float scale;
    void *out;
};

struct PrefillArgs {
    int batch, seqlen, num_heads, dk, dv, num_seqs;
    bool kda, bf16, out_bf16;
    int chunk, dv_slice;            // resolved (non-zero) values
    const void *q, *k, *v;
    const float *beta, *log_alpha, *initial_state;
    const int32_t *cu_seqlens;
    float scale;
    void *out;
    float *final_state;
    int32_t *order;                 // workspace: longest-first sequence order (packed only)
};

hipError_t launch_decode(const DecodeArgs &p, hipStream_t st);

// True when a prefill kernel is compiled for this combination.
bool prefill_supported(bool bf16, bool kda, int dk, int dv_slice, int chunk);
hipError_t launch_prefill(const PrefillArgs &p, hipStream_t st);

}  // namespace gdr
