// fp32 instantiations of the chunked prefill (fp32 MFMA throughout).
#include "prefill_impl.h"
namespace gdn {
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
    return prefill_launch_typed<float>(a, s);
}
}  // namespace gdn
