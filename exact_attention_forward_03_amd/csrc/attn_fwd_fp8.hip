// Placeholder: the e4m3 attention kernel is not built yet.
#include "attn_params.h"
namespace attn {
hipError_t launch_fwd_fp8(int, bool, const FwdParams&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
