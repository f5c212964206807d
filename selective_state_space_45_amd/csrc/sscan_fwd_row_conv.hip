// Forward scan launch variants, states across the lanes of a row, with the fused
// convolution prologue (causal depthwise conv1d over time + SiLU), both rules.
#include "sscan_fwd_row.h"

namespace sscan {

template hipError_t launch_fwd_row<kFwdOutConv, false>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_fwd_row<kFwdOutConv, true>(const FwdParams&, bool, hipStream_t);

}  // namespace sscan
