// Dense-expand N:M tile kernel (nm_spmm_expand.hpp), bf16 weights: every
// N:M instantiated for this weight dtype and its two output dtypes.
#include "nm_spmm_expand.hpp"

namespace nm {

hipError_t launch_spmm_expand_bf16(const SpmmArgs& a, hipStream_t s) { return launch_wt<NM_BF16>(a, s); }

}  // namespace nm
