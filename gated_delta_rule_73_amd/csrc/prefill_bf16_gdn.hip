// prefill_bf16_gdn.hip -- instances of the chunked prefill kernel
// (operand type __bf16, per-channel decay = false).
#include "prefill_impl.h"
#include "prefill_shapes.h"

namespace gdr {

hipError_t launch_prefill_bf16_gdn(const PrefillArgs &a, hipStream_t st) {
#define GDR_CASE(DK_, DVS_, C_) \
    if (a.dk == DK_ && a.dv_slice == DVS_ && a.chunk == C_) return launch_prefill_t<DK_, DVS_, C_, false, __bf16>(a, st);
    GDR_PREFILL_BF16_GDN_SHAPES(GDR_CASE)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

int chain_blocks_per_cu_bf16_gdn(int dk, int dv_slice, int chunk) {
    int n = 0;
#define GDR_CASE(DK_, DVS_, C_)                                                                                  \
    if (dk == DK_ && dv_slice == DVS_ && chunk == C_)                                                           \
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(                                                   \
                   &n, chain_kernel<DK_, DVS_, C_, false, __bf16, false>, 64 * (kLoaderWaves + DVS_ / 16), 0) == hipSuccess \
                   ? n : 0;
    GDR_PREFILL_BF16_GDN_SHAPES(GDR_CASE)
#undef GDR_CASE
    return 0;
}

}  // namespace gdr
