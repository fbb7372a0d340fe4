// bf16 instantiations of the prefill prep with the short convolution fused into its
// loads (the scan that follows is the one of the plain prefill).
#include "prefill_impl.h"
namespace gdn {
hipError_t launch_prefill_conv_prep_bf16(const PrefillArgs& a, hipStream_t s) {
    return prefill_conv_prep_typed<bf16>(a, s);
}
}  // namespace gdn
