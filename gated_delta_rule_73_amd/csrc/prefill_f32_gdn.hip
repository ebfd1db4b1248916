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

}  // namespace gdr
