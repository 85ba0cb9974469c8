// Causal prefill-chunk attention over a paged KV cache (MFMA path).
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {

int launch_prefill(const PrefillLaunch &, void *) { return (int)hipErrorNotSupported; }

}  // namespace pa
