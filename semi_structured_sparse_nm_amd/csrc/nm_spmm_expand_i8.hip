// Dense-expand N:M tile kernel (nm_spmm_expand.hpp), i8 weights: every
// N:M instantiated for this weight dtype and its two output dtypes.
#include "nm_spmm_expand.hpp"

namespace nm {

hipError_t launch_spmm_expand_i8(const SpmmArgs& a, hipStream_t s) { return launch_wt<NM_I8>(a, s); }

bool expand_supported(int N, int M) {
  return (M == 4) || (M == 8 && (N == 1 || N == 2 || N == 4 || N == 8));
}

hipError_t launch_spmm_expand(const SpmmArgs& a, hipStream_t s) {
  if (a.wdt == NM_I8) return launch_spmm_expand_i8(a, s);
  if (a.wdt == NM_F16) return launch_spmm_expand_f16(a, s);
  return launch_spmm_expand_bf16(a, s);
}

}  // namespace nm
