// Forward scan launch variants, states across the lanes of a row: zero-order hold.
#include "sscan_fwd_row.h"

namespace sscan {

template hipError_t launch_fwd_row<kFwdOut, false>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_fwd_row<kFwdCkpt, false>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_fwd_row<kFwdOutCkpt, false>(const FwdParams&, bool, hipStream_t);

}  // namespace sscan
