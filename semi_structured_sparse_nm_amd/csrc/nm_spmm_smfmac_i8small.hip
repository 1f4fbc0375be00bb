// int8 2:4 sparse x dense product for shapes the tile kernels do not take
// (T not a multiple of 16, activation or output rows not 16-byte aligned),
// on the gfx950 sparse matrix cores (v_smfmac_i32_16x16x128_i8), with the
// fused bias + requantisation (+ GELU) epilogue.
//
// The kernel side of "Realizable N:M Sparse Transformer Inference via
// Search-Kernel Co-Design", Sec. 4.1 (inference-scale parallelism: small
// layers must still spread over the device): one wave per 16 x 16 output
// tile, four waves per workgroup on consecutive token tiles of one 16-row
// block, so a ViT-Tiny slice (192 x 192 x 197) is 156 waves that each make
// one round trip to memory.
//
// Operands: the packed 16 x 128 block is the v_smfmac A operand byte for
// byte (16 kept values per lane, index word per lane), as in the tile
// kernels.  The B operand is gathered straight from X with byte loads: lane
// (i, g) takes token t0 + i and the 32 rows 16 g .. 16 g + 15 and
// 64 + 16 g .. 64 + 16 g + 15 of the column block (the k order the tile
// kernels' transposing LDS reads produce), so no row alignment is needed.
// Rows past K read as zero through the buffer range check (the packed values
// there are zero too); tokens past T read whatever lies there and are never
// stored.  Outputs: rows 16 rb + 4 g + v, token t0 + i of lane (i, g); int32
// stored as dwords, int8 as bytes, tokens past T and rows past R dropped.
#include "nm_common.hpp"

namespace nm {

namespace {

constexpr int NWS = 4;   // waves per workgroup (consecutive token tiles)

template <bool OUT_I8, bool ACT>
__global__ void __launch_bounds__(NWS * 64) smfmac_i8small_kernel(SpmmArgs a, int ntt) {
  // device pass only (device-only types and builtins)
#if defined(__HIP_DEVICE_COMPILE__)
  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int nKB = (int)g.nKB;
  const int ngrp = (ntt + NWS - 1) / NWS;
  const int rb = blockIdx.x / ngrp;
  const int tt = (blockIdx.x - rb * ngrp) * NWS + wave;
  if (tt >= ntt) return;
  const int t = tt * 16 + li;                 // this lane's token
  const int ldx = (int)a.ldx;

  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values), 0, (int)g.values_bytes(), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.meta), 0, (int)g.meta_bytes(), 0x00020000);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.X), 0, (int)(g.K * a.ldx), 0x00020000);

  // bias rows 16 rb + 4 g + v as the accumulator's start (zero when absent;
  // rows past R read as zero)
  v4i acc = {0, 0, 0, 0};
  if (a.bias) {
    const __amdgpu_buffer_rsrc_t rbias =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.bias), 0, (int)(g.R * 4), 0x00020000);
#pragma unroll
    for (int v = 0; v < 4; ++v)
      acc[v] = (int)__builtin_amdgcn_raw_buffer_load_b32(rbias, 4 * (16 * rb + 4 * lg + v), 0, 0);
  }

  const int voff_v = li * 64 + lg * 16;
  const int voff_m = li * 16 + lg * 4;
  for (int kb = 0; kb < nKB; ++kb) {
    const int blk = rb * nKB + kb;
    const v4i av = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v, blk * 1024, 0));
    const int ai = (int)__builtin_amdgcn_raw_buffer_load_b32(rm, voff_m, blk * 256, 0);
    // B: dword d holds rows r(d) .. r(d) + 3, r(d) = 16 g + 4 d (d < 4) or
    // 64 + 16 g + 4 (d - 4), byte j of a dword = row r(d) + j
    const int base = (kb * 128 + 16 * lg) * ldx + t;
    v8i b;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int r = (d < 4 ? 4 * d : 64 + 4 * (d - 4));
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t x = __builtin_amdgcn_raw_buffer_load_b8(rx, base + (r + j) * ldx, 0, 0);
        w |= x << (8 * j);
      }
      b[d] = (int)w;
    }
    acc = __builtin_amdgcn_smfmac_i32_16x16x128_i8(av, b, acc, ai, 0, 0);
  }

  const bool t_ok = t < (int)a.T;
  const int row0 = 16 * rb + 4 * lg;
  if constexpr (OUT_I8) {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.scale), 0, (int)(g.R * 4), 0x00020000);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (row0 + v), 0, 0));
      const int q = requant_act_i8<ACT>(acc[v], s, a.out_scale);
      const int off = t_ok ? (row0 + v) * (int)a.ldy + t : (int)(g.R * a.ldy);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)q, ry, off, 0, 0);
    }
  } else {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy * 4), 0x00020000);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int off = t_ok ? 4 * ((row0 + v) * (int)a.ldy + t) : (int)(g.R * a.ldy * 4);
      __builtin_amdgcn_raw_buffer_store_b32(acc[v], ry, off, 0, 0);
    }
  }
#endif
}

template <bool OUT_I8, bool ACT>
hipError_t launch_cfg(const SpmmArgs& a, hipStream_t s) {
  const int ntt = (int)((a.T + 15) / 16);
  const int ngrp = (ntt + NWS - 1) / NWS;
  const int64_t grid = a.g.nRB * ngrp;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((smfmac_i8small_kernel<OUT_I8, ACT>), dim3((unsigned)grid), dim3(NWS * 64), 0, s, a, ntt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_spmm_smfmac_i8small(const SpmmArgs& a, hipStream_t s) {
  if (a.ydt == NM_I8 && a.act) return launch_cfg<true, true>(a, s);
  if (a.ydt == NM_I8) return launch_cfg<true, false>(a, s);
  return launch_cfg<false, false>(a, s);
}

}  // namespace nm
