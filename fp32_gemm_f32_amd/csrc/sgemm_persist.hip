// sgemm_persist.hip -- the persistent store-overlapped kernel (kernel_persist.hpp) in a
// translation unit of its own: its two sets of 128 accumulators per lane live in AGPRs,
// which the build options of the rest of the library rule out (they keep MFMA accumulators
// in VGPRs).
#include <hip/hip_runtime.h>

#include "kernel_persist.hpp"

namespace sgemm {

// Launch handles for the variant table in sgemm_f32.hip: K a multiple of 32, and any K.
void (*persist_kernel())(GemmArgs) { return &k_sgemm_persist<false>; }
void (*persist_ktail_kernel())(GemmArgs) { return &k_sgemm_persist<true>; }

}  // namespace sgemm
