// Parallax causal prefill on CDNA4 (gfx950).
#include "device_common.h"
#include "kernels.h"

namespace parallax {

hipError_t launch_prefill(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace parallax
