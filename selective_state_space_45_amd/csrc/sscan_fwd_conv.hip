// Forward scan launch variants with the fused convolution prologue (causal
// depthwise conv1d over time + SiLU), for both discretization rules.
#include "sscan_fwd_kernel.h"

namespace sscan {

template hipError_t launch_fwd_variant<kFwdOut, false, true>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_fwd_variant<kFwdAgg, false, true>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_fwd_variant<kFwdOut, true, true>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_fwd_variant<kFwdAgg, true, true>(const FwdParams&, bool, hipStream_t);

}  // namespace sscan
