// Dense-expand N:M tile kernel (nm_spmm_expand.hpp), f16 weights: every
// N:M instantiated for this weight dtype and its two output dtypes.
#include "nm_spmm_expand.hpp"

namespace nm {

hipError_t launch_spmm_expand_f16(const SpmmArgs& a, hipStream_t s) { return launch_wt<NM_F16>(a, s); }

}  // namespace nm
