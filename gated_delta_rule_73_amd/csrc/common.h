// common.h -- small device helpers shared by the gfx950 kernels of libgdr.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// ---- scalar conversions -------------------------------------------------
// fp32 -> bf16 uses the hardware round-to-nearest-even conversion of gfx950.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// ---- 4-wide loads of q/k/v rows (fp32 or bf16 storage) --------------------
__device__ __forceinline__ float4 load4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 load4(const __bf16 *p) {
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

// ---- cross-lane sums inside aligned groups of W lanes ---------------------
template <int W>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = 1; m < W; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

__host__ __device__ constexpr int div_up(int a, int b) { return (a + b - 1) / b; }

// Workgroup barrier that waits only for this wave's LDS operations: loads
// in flight to registers or to LDS keep going across it (the compiler's own
// barrier would drain them).  It orders LDS accesses only; waves that fill
// LDS with LDS-direct loads wait for them explicitly before it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace gdr
