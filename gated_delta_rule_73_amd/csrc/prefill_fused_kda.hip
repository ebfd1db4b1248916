// prefill_fused_kda.hip -- instances of the fused prefill kernel for a
// per-key-channel decay (Kimi Delta Attention).
#include "fused_impl.h"

namespace gdr {

hipError_t launch_fused_kda(const FusedArgs &fa, int dk, int dvs, int grid, hipStream_t st) {
#define GDR_CASE(DK_, DVS_) if (dk == DK_ && dvs == DVS_) return launch_fused_t<DK_, DVS_, true>(fa, grid, st);
    GDR_CASE(32, 16) GDR_CASE(32, 32) GDR_CASE(64, 16) GDR_CASE(64, 32) GDR_CASE(128, 16) GDR_CASE(128, 32)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

}  // namespace gdr
