// fp32 instantiations of the chunked prefill (fp32 MFMA operands and accumulation).
#include "prefill_impl.h"
namespace gdn {
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
    return prefill_launch_typed<float>(a, s);
}
hipError_t launch_prefill_scan_f32(const PrefillArgs& a, hipStream_t s) {
    return prefill_scan_typed<float>(a, s);
}
}  // namespace gdn
