// sgemm_persist.hip -- the persistent store-overlapped kernel (kernel_persist.hpp) in a
// translation unit of its own. Its 4-wave form (one 64 x 128 wave per SIMD) holds two sets
// of 128 accumulators per lane, which fit only with the accumulators in AGPRs, and the
// build options of the rest of the library rule that out (they keep MFMA accumulators in
// VGPRs). The 8-wave form's two sets of 64 per lane (two 64 x 64 waves per SIMD) fit in
// VGPRs, where the compiler keeps them (238 VGPRs, no AGPRs).
#include <hip/hip_runtime.h>

#include "kernel_persist.hpp"

namespace sgemm {

// Launch handles for the variant table in sgemm_f32.hip, by waves per workgroup (4: one per
// SIMD, 8: two): K a multiple of 32, and any K.
void (*persist_kernel(int waves))(GemmArgs)
{
    return waves == 8 ? &k_sgemm_persist<8, false> : &k_sgemm_persist<4, false>;
}
void (*persist_ktail_kernel(int waves))(GemmArgs)
{
    return waves == 8 ? &k_sgemm_persist<8, true> : &k_sgemm_persist<4, true>;
}

}  // namespace sgemm
