// Placeholder: the fp8 pre-processing kernel is not built yet.
#include "attn_params.h"
namespace attn {
hipError_t launch_fp8_prep(const PrepParams&, bool, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
