// Forward scan launch variants, states across the lanes of a row: Euler rule (Bbar = Delta B).
#include "sscan_fwd_row.h"

namespace sscan {

template hipError_t launch_fwd_row<kFwdOut, true>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_fwd_row<kFwdCkpt, true>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_fwd_row<kFwdOutCkpt, true>(const FwdParams&, bool, hipStream_t);

}  // namespace sscan
