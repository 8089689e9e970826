// sgemm_regpanel.hip -- the one-wave-per-SIMD kernel (kernel_regpanel.hpp) in a translation
// unit of its own: its 256 accumulators per lane live in AGPRs, which the build options of
// the rest of the library rule out (they keep MFMA accumulators in VGPRs).
#include <hip/hip_runtime.h>

#include "kernel_regpanel.hpp"

namespace sgemm {

// Launch handles of the plain and the stream-K form, for the variant table in sgemm_f32.hip.
void (*regpanel_kernel())(GemmArgs) { return &k_sgemm_regpanel<false>; }
void (*regpanel_streamk_kernel())(GemmArgs) { return &k_sgemm_regpanel<true>; }

}  // namespace sgemm
