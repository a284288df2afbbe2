// prefill.hip -- placeholder until the MFMA prefill kernel lands.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace pa {
hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace pa
