// Launch arguments of the three-layer format product (nm_hybrid_spmm).
// Internal; the format itself is documented at nm_hybrid in nm_sparse.h.
#pragma once

#include "nm_common.hpp"

namespace nm {

struct HybridArgs {
  int64_t R, K;
  int64_t nRB, nKB, nSeg;      // 16-row blocks, 64-column blocks, 8-block segments
  int wdt;                     // NM_F16 / NM_BF16
  int ydt;                     // NM_F16 / NM_BF16 / NM_F32
  int act;                     // NM_ACT_NONE / NM_ACT_GELU
  const uint8_t* values;       // Sparse-TC layer (2:4 layout)
  const uint8_t* meta;
  const uint8_t* codes;        // Slot-Filling codes, 8 B per fill unit
  const int32_t* res_ptr;      // residual CSR
  const uint32_t* res_ent;
  int64_t values_bytes, meta_bytes, codes_bytes, res_ptr_bytes, res_ent_bytes;
  const void* X;               // [K][ldx]
  int64_t ldx, T;
  void* Y;                     // [R][ldy]
  int64_t ldy;
  const float* bias;           // float[R] or nullptr
  int G;                       // workgroups along the row blocks (row blocks b, b + G, ...)
  int nChunk;                  // chunks of four segments
  // X[K-1][T-1] when the 4-byte piece holding it ends past X (odd T with
  // ldx == T): the range check zeroes that piece, so the element is read
  // again on its own; false otherwise
  bool patch_last;
};

// Waves per workgroup (= 512-column segments per activation chunk) and row
// blocks one workgroup takes at most, [plain 2:4, three-layer].
constexpr int kHybridWaves[2] = {8, 4};
constexpr int kHybridMaxRB[2] = {3, 4};

// hy = false: the plain 2:4 layer alone (values / meta of an nm_pack 2:4
// weight; codes and residual unused) with the same schedule.
hipError_t launch_spmm_hybrid(const HybridArgs& a, bool hy, hipStream_t s);

}  // namespace nm
