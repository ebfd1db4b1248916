// prefill_f32_kda.hip -- instances of the chunked prefill kernel
// (operand type float, per-channel decay = true).
#include "prefill_impl.h"
#include "prefill_shapes.h"

namespace gdr {

hipError_t launch_prefill_f32_kda(const PrefillArgs &a, hipStream_t st) {
#define GDR_CASE(DK_, DVS_, C_) \
    if (a.dk == DK_ && a.dv_slice == DVS_ && a.chunk == C_) return launch_prefill_t<DK_, DVS_, C_, true, float>(a, st);
    GDR_PREFILL_F32_KDA_SHAPES(GDR_CASE)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdr
