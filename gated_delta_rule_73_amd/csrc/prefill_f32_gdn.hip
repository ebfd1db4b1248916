// prefill_f32_gdn.hip -- instances of the chunked prefill kernel
// (operand type float, per-channel decay = false).
#include "prefill_impl.h"
#include "prefill_shapes.h"

namespace gdr {

hipError_t launch_prefill_f32_gdn(const PrefillArgs &a, hipStream_t st) {
#define GDR_CASE(DK_, DVS_, C_) \
    if (a.dk == DK_ && a.dv_slice == DVS_ && a.chunk == C_) return launch_prefill_t<DK_, DVS_, C_, false, float>(a, st);
    GDR_PREFILL_F32_GDN_SHAPES(GDR_CASE)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

int chain_blocks_per_cu_f32_gdn(int dk, int dv_slice, int chunk) {
    int n = 0;
#define GDR_CASE(DK_, DVS_, C_)                                                                                  \
    if (dk == DK_ && dv_slice == DVS_ && chunk == C_)                                                           \
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(                                                   \
                   &n, chain_kernel<DK_, DVS_, C_, false, float, false>, 64 * (kLoaderWaves + DVS_ / 16), 0) == hipSuccess \
                   ? n : 0;
    GDR_PREFILL_F32_GDN_SHAPES(GDR_CASE)
#undef GDR_CASE
    return 0;
}

}  // namespace gdr
