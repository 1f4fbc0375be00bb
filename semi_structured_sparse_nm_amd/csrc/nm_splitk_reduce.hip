// Split-K finish: Y = epilogue(sum of the K slices' partial sums).
//
// Adaptive parallelism ("Realizable N:M Sparse Transformer Inference via
// Search-Kernel Co-Design", Sec. 4.1): when an operator's output has too few
// tiles to occupy every compute unit, the tile kernels cut K into slices that
// run as separate work items and write raw partial sums (int32 for int8
// operands, fp32 otherwise) to the workspace, laid out [slice][R][T] with row
// pitch T.  This kernel adds the slices in slice order (exact for int32; a
// fixed order for fp32, so results do not depend on timing) and applies the
// epilogue the tile kernels would have applied: bias, then int8
// requantisation or the rounding to the output type.
//
// One thread per 4 consecutive tokens of a row: 16-byte partial loads, one
// 4-, 8- or 16-byte store (element stores when Y's rows are not aligned for
// them).  The partials are read once: non-temporal loads.
#include "nm_common.hpp"

namespace nm {

namespace {

template <bool I8IN, int OUT, bool VEC>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(SpmmArgs a, int64_t nq) {
  typedef typename std::conditional<I8IN, v4i, v4f>::type Acc;
  const int64_t T4 = a.T / 4;
  const Acc* ws = static_cast<const Acc*>(a.ws);
  const int64_t ys4 = a.ys / 4;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < nq; q += (int64_t)gridDim.x * 256) {
    const int64_t r = q / T4;
    const int64_t t = (q - r * T4) * 4;
    Acc s = __builtin_nontemporal_load(ws + q);
    for (int k = 1; k < a.ksplit; ++k) s += __builtin_nontemporal_load(ws + k * ys4 + q);
    const int64_t o = r * a.ldy + t;
    if constexpr (I8IN) {
      if (a.bias) s += static_cast<const int32_t*>(a.bias)[r];
      if constexpr (OUT == NM_I32) {
        int32_t* y = static_cast<int32_t*>(a.Y) + o;
        if constexpr (VEC) {
          *reinterpret_cast<v4i*>(y) = s;
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) y[v] = s[v];
        }
      } else {
        const float sc = a.scale[r];
        uint32_t packed = 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int q = a.act ? requant_act_i8<true>(s[v], sc, a.out_scale) : requant_i8(s[v], sc);
          packed |= (uint32_t)(q & 0xFF) << (8 * v);
        }
        int8_t* y = static_cast<int8_t*>(a.Y) + o;
        if constexpr (VEC) {
          *reinterpret_cast<uint32_t*>(y) = packed;
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) y[v] = (int8_t)(packed >> (8 * v));
        }
      }
    } else {
      if (a.bias) s += static_cast<const float*>(a.bias)[r];
      if (a.act) {
#pragma unroll
        for (int v = 0; v < 4; ++v) s[v] = gelu_f32(s[v]);
      }
      if constexpr (OUT == NM_F32) {
        float* y = static_cast<float*>(a.Y) + o;
        if constexpr (VEC) {
          *reinterpret_cast<v4f*>(y) = s;
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) y[v] = s[v];
        }
      } else {
        uint16_t h[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) h[v] = OUT == NM_F16 ? f32_to_f16_bits(s[v]) : f32_to_bf16_bits(s[v]);
        uint16_t* y = static_cast<uint16_t*>(a.Y) + o;
        if constexpr (VEC) {
          typedef uint32_t v2u __attribute__((ext_vector_type(2)));
          *reinterpret_cast<v2u*>(y) = v2u{h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16)};
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) y[v] = h[v];
        }
      }
    }
  }
}

template <bool I8IN, int OUT>
hipError_t launch_out(const SpmmArgs& a, hipStream_t s) {
  const int64_t nq = a.g.R * (a.T / 4);
  const int ob = dtype_bytes(OUT);
  const bool vec = a.ldy % 4 == 0 && (uintptr_t)a.Y % (size_t)(4 * ob) == 0;
  int64_t blocks = (nq + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (vec)
    hipLaunchKernelGGL((splitk_reduce_kernel<I8IN, OUT, true>), dim3((unsigned)blocks), dim3(256), 0, s, a, nq);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<I8IN, OUT, false>), dim3((unsigned)blocks), dim3(256), 0, s, a, nq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_splitk_reduce(const SpmmArgs& a, hipStream_t s) {
  if (a.T % 4 != 0 || a.ys % 4 != 0 || a.ksplit < 1 || (uintptr_t)a.ws % 16 != 0) return hipErrorInvalidValue;
  switch (a.ydt) {
    case NM_I32: return launch_out<true, NM_I32>(a, s);
    case NM_I8: return launch_out<true, NM_I8>(a, s);
    case NM_F32: return launch_out<false, NM_F32>(a, s);
    case NM_F16: return launch_out<false, NM_F16>(a, s);
    case NM_BF16: return launch_out<false, NM_BF16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nm
