// Checkpoint pass with the backward pass's reverse segment aggregates (row layout).
#include "sscan_fwd_row.h"

namespace sscan {

template hipError_t launch_fwd_row<kFwdCkptAgg, false>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_fwd_row<kFwdCkptAgg, true>(const FwdParams&, bool, hipStream_t);

}  // namespace sscan
