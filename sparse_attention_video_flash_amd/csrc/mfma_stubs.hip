// Placeholder dispatch until the MFMA kernels land: the generic kernels run.
#include "internal.h"
namespace svg {
SVG_HIDDEN bool probe_mfma_supported(const ProbeArgs&) { return false; }
SVG_HIDDEN hipError_t launch_probe_mfma(const ProbeArgs&, const float*, const float2*, const float*, hipStream_t) { return hipErrorInvalidValue; }
}
