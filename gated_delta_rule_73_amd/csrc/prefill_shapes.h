// prefill_shapes.h -- the (d_k, value-slice width, chunk) combinations the
// prefill kernel is compiled for.
#pragma once

// bf16 q/k/v: fp16/bf16 MFMA 16x16x32 needs d_k and the chunk to be
// multiples of 32; the UT-transform inverse handles two or four 16-token
// blocks (32- or 64-token chunks).
#define GDR_PREFILL_BF16_GDN_SHAPES(X) \
    X(32, 16, 32) X(32, 32, 32) X(64, 16, 32) X(64, 32, 32) X(128, 16, 32) X(128, 32, 32) X(128, 64, 32) \
    X(32, 16, 64) X(32, 32, 64) X(64, 16, 64) X(64, 32, 64) X(128, 16, 64) X(128, 32, 64)
#define GDR_PREFILL_BF16_KDA_SHAPES(X) \
    X(32, 16, 32) X(32, 32, 32) X(64, 16, 32) X(64, 32, 32) X(128, 16, 32) X(128, 32, 32) X(128, 64, 32) \
    X(32, 16, 64) X(32, 32, 64) X(64, 16, 64) X(64, 32, 64) X(128, 16, 64) X(128, 32, 64)

// fp32 q/k/v: fp32 MFMA 16x16x4, chunks of 16 or 32 tokens.
#define GDR_PREFILL_F32_GDN_SHAPES(X) \
    X(16, 16, 16) X(16, 16, 32) X(32, 16, 16) X(32, 16, 32) \
    X(64, 16, 16) X(64, 16, 32) X(128, 16, 16) X(128, 16, 32)
#define GDR_PREFILL_F32_KDA_SHAPES(X) \
    X(16, 16, 16) X(16, 16, 32) X(32, 16, 16) X(32, 16, 32) \
    X(64, 16, 16) X(64, 16, 32) X(128, 16, 16) X(128, 16, 32)
