// Forward scan launch variants: zero-order hold.
#include "sscan_fwd_kernel.h"

namespace sscan {

template hipError_t launch_fwd_variant<kFwdOut, false, false>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_fwd_variant<kFwdAgg, false, false>(const FwdParams&, bool, hipStream_t);
template hipError_t launch_fwd_variant<kFwdOutCkpt, false, false>(const FwdParams&, bool, hipStream_t);

}  // namespace sscan
