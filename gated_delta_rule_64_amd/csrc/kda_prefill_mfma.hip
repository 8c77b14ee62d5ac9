// Matrix-core chunked prefill (placeholder until the MFMA kernels land).
#include "kda_prefill_mfma.h"

namespace kda {

bool mfma_prefill_supports(int, int, DT) { return false; }
size_t mfma_record_bytes() { return 0; }
hipError_t launch_prefill_mfma(const PrefillArgs&, hipStream_t, int32_t*, char*) {
    return hipErrorNotSupported;
}

}  // namespace kda
