// Forward scan launch variants: Euler rule (Bbar = Delta B).
#include "sscan_fwd_kernel.h"

namespace sscan {

template hipError_t launch_fwd_variant<kFwdOut, true, false>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_fwd_variant<kFwdAgg, true, false>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_fwd_variant<kFwdOutCkpt, true, false>(const FwdParams&, bool, hipStream_t);

}  // namespace sscan
