// Register expansion of packed N:M windows into dense matrix-core
// fragments, shared by the dense-expand kernels (the pages' micro-dense
// execution, "Realizable N:M Sparse Transformer Inference via Search-Kernel
// Co-Design", Sec. 4.2: kept values placed at their in-window positions so
// the matrix cores see only regular dense operands).
//
// Lane assignment: over the two dense MFMA steps of one packed block (KB
// dense columns), lane group g of a 16x16 fragment takes the dense run
// [LR g, LR (g + 1)): its kept values are one contiguous run of VB bytes of
// the packed block row (at offset g VB) and its positions one contiguous run
// of MBL meta bits (from bit g MBL).  Step s covers the run's elements
// [LR s / 2, LR (s + 1) / 2); the B operand (X) must follow the same k order.
#pragma once

#include <type_traits>

#include "nm_common.hpp"

namespace nm {

// Per-dtype geometry: EB element bytes, LR dense elements per lane per
// block, a step (one MFMA) covers LR / 2.
template <int WT> struct Ty {
  static constexpr int EB = (WT == NM_I8) ? 1 : 2;
  static constexpr int LR = (WT == NM_I8) ? 32 : 16;
};

// Dense 16-byte A fragment of step S from a lane's packed run: vd holds the
// run's kept values (element e at byte e EB), mb its positions (W bits each,
// element e at bit e W).  Group q of the step occupies bytes q M EB .. of
// the fragment.
template <int WT, int NN, int MM, int S>
__device__ __forceinline__ v4i expand_step(const uint32_t* vd, uint64_t mb) {
  constexpr int EB = Ty<WT>::EB;
  constexpr int RUN = Ty<WT>::LR / 2;             // dense elements per step
  constexpr int G = RUN / MM;                     // groups per step
  constexpr int KS = G * NN;                      // kept per step
  constexpr int W = (NN == MM) ? 0 : (MM == 4 ? 2 : 3);
  if constexpr (NN == MM) {
    return v4i{(int)vd[4 * S], (int)vd[4 * S + 1], (int)vd[4 * S + 2], (int)vd[4 * S + 3]};
  } else {
    uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < G; ++q) {
      uint64_t lo = 0, hi = 0;                    // the group's 64 (or 128) bits
#pragma unroll
      for (int j = 0; j < NN; ++j) {
        const int e = S * KS + q * NN + j;        // element of the lane's run
        const uint32_t el = (vd[(e * EB) >> 2] >> (8 * ((e * EB) & 3))) & (EB == 1 ? 0xFFu : 0xFFFFu);
        const uint32_t pos = (uint32_t)(mb >> (e * W)) & ((1u << W) - 1u);
        if constexpr (MM * EB == 4) {
          lo |= (uint64_t)(el << (8 * pos));
        } else if constexpr (MM * EB == 8) {
          lo |= (uint64_t)el << ((8 * EB) * pos);
        } else {                                  // fp16, M = 8: 128 bits
          const uint64_t sh = (uint64_t)el << (16 * (pos & 3));
          lo |= (pos < 4) ? sh : 0;
          hi |= (pos < 4) ? 0 : sh;
        }
      }
      if constexpr (MM * EB == 4) {
        o[q] = (uint32_t)lo;
      } else if constexpr (MM * EB == 8) {
        o[2 * q] = (uint32_t)lo;
        o[2 * q + 1] = (uint32_t)(lo >> 32);
      } else {
        o[0] = (uint32_t)lo; o[1] = (uint32_t)(lo >> 32);
        o[2] = (uint32_t)hi; o[3] = (uint32_t)(hi >> 32);
      }
    }
    return v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
  }
}

template <int WT>
__device__ __forceinline__ auto mfma_dense(v4i a, v4i b, typename std::conditional<WT == NM_I8, v4i, v4f>::type c) {
  if constexpr (WT == NM_I8)
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  else if constexpr (WT == NM_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0,
                                                   0, 0);
}

// Lane-run geometry of one N:M and weight dtype (see the header comment).
template <int WT, int NN, int MM> struct Run {
  static constexpr int EB = Ty<WT>::EB;
  static constexpr int LR = Ty<WT>::LR;
  static constexpr int KL = LR * NN / MM;          // kept per lane per block
  static constexpr int VB = KL * EB;               // their bytes
  static constexpr int VD = VB / 4;
  static constexpr int W = (NN == MM) ? 0 : (MM == 4 ? 2 : 3);
  static constexpr int MBL = KL * W;               // meta bits per lane per block
  static constexpr int C_B = 4 * VB;               // packed row bytes per block
  static constexpr int MRB = W ? ((4 * MBL + 7) / 8 + 3) / 4 * 4 : 0;   // meta row bytes
  static_assert(VB % 4 == 0 && VD <= 8, "lane runs of whole dwords, at most 32 bytes");
  static_assert(MBL <= 48, "a lane's positions fit a 64-bit window at any bit offset used");
  // The lane's positions start at bit g MBL of its row's meta: read a 64-bit
  // window from the dword holding that bit (one dword back when the window
  // would leave the row, whose last dword then holds all of them).  Returns
  // the window's first dword and the shift of the first position in it.
  __device__ static void meta_window(int g, int& dword, int& shift) {
    dword = (g * MBL) >> 5;
    shift = (g * MBL) & 31;
    if (MRB >= 8 && 4 * dword + 8 > MRB) { dword -= 1; shift += 32; }
  }
};

}  // namespace nm
