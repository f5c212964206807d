// Forward scan launch variant, states across the lanes of a row: zero-order hold with
// the factored staging of a rank-one A (A[d, n] = c_d a_n, flag SSCAN_FLAG_STRUCTURED_A).
#include "sscan_fwd_row.h"

namespace sscan {

template hipError_t launch_fwd_row<kFwdOut, false, true>(const FwdParams&, bool, hipStream_t);

}  // namespace sscan
