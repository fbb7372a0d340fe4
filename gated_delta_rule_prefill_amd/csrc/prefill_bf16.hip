// bf16 instantiations of the chunked prefill (bf16 MFMA operands, fp32 accumulation/state).
#include "prefill_impl.h"
namespace gdn {
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
    return prefill_launch_typed<bf16>(a, s);
}
hipError_t launch_prefill_scan_bf16(const PrefillArgs& a, hipStream_t s) {
    return prefill_scan_typed<bf16>(a, s);
}
}  // namespace gdn
