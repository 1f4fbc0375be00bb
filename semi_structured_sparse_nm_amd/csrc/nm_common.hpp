// Shared definitions of the HIP library: packed-layout geometry, launch
// argument bundles and small device helpers.  Internal; the public surface is
// include/nm_sparse.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/nm_sparse.h"

namespace nm {

// ---------------------------------------------------------------- layout
// Geometry of the blocked packed layout (documented with nm_packed in the
// public header): 16-row x KB-column blocks, KB = 128 / element bytes.
struct Geometry {
  int64_t R, K;
  int N, M;
  int eb;          // element bytes (1 or 2)
  int KB;          // dense columns per block
  int GB;          // groups per block row
  int C;           // kept slots per block row
  int w;           // index bits (2 or 3), 0 when N == M
  int MR;          // meta bytes per block row (multiple of 4), 0 when N == M
  int64_t nRB, nKB;
  int64_t vblk;    // value bytes per block
  int64_t mblk;    // meta bytes per block

  static Geometry make(int64_t R, int64_t K, int N, int M, int eb) {
    Geometry g;
    g.R = R; g.K = K; g.N = N; g.M = M; g.eb = eb;
    g.KB = 128 / eb;
    g.GB = g.KB / M;
    g.C = g.GB * N;
    g.w = (N == M) ? 0 : (M == 4 ? 2 : 3);
    int mr = (g.C * g.w + 7) / 8;
    g.MR = (mr + 3) / 4 * 4;
    g.nRB = (R + 15) / 16;
    g.nKB = (K + g.KB - 1) / g.KB;
    g.vblk = (int64_t)16 * g.C * eb;
    g.mblk = (int64_t)16 * g.MR;
    return g;
  }
  __host__ __device__ size_t values_bytes() const { return (size_t)(nRB * nKB * vblk); }
  __host__ __device__ size_t meta_bytes() const { return (size_t)(nRB * nKB * mblk); }
};

inline int dtype_bytes(int dt) {
  switch (dt) {
    case NM_I8: return 1;
    case NM_F16: case NM_BF16: return 2;
    case NM_I32: case NM_F32: return 4;
    default: return 0;
  }
}

// ---------------------------------------------------------------- launches
struct SpmmArgs {
  Geometry g;
  int wdt;                 // weight / activation dtype (NM_I8, NM_F16, NM_BF16)
  int ydt;                 // output dtype
  const uint8_t* values;
  const uint8_t* meta;
  const void* X;
  int64_t ldx;
  int64_t T;
  void* Y;
  int64_t ldy;
  const void* bias;        // int32[R] or float[R] or nullptr
  const float* scale;      // float[R] (int8 output) or nullptr
  void* ws;                // workspace
  size_t ws_bytes;
  // K split across workgroups (the tile kernels that take it: fp16 / bf16
  // 2:4 and dense-expand).  Work item = (tile, K slice s); slice s covers
  // column blocks s kbs .. s kbs + kbs - 1.  With ksplit > 1 the kernel runs
  // with a 32-bit output type, no bias, Y = the workspace and ldy = T, and
  // writes slice s's raw partial sums at Y + s ys elements;
  // launch_splitk_reduce then adds the slices and applies the epilogue.
  int ksplit;              // K slices (1: no split)
  int kbs;                 // column blocks per slice (nKB / ksplit)
  int64_t ys;              // elements between consecutive slices' partials
  // Activation fused into the epilogue (NM_ACT_NONE / NM_ACT_GELU): fp
  // outputs take act(acc + bias); int8 outputs take
  // sat(rne(act(f32(acc + bias) * scale[r]) * out_scale)).
  int act;
  float out_scale;
  // operand layout: NM_LAYOUT_KT (X [K][ldx], Y [R][ldy]) or NM_LAYOUT_TK
  // (X [T][ldx] with K contiguous, Y [T][ldy] with R contiguous)
  int layout;
};

// Kernel variants; each launcher returns hipSuccess or the launch error.
hipError_t launch_pack(const void* W, int64_t ldw, const Geometry& g, int wdt, uint8_t* values,
                       uint8_t* meta, hipStream_t s);
hipError_t launch_spmm_generic(const SpmmArgs& a, hipStream_t s);
hipError_t launch_spmm_smfmac_i8(const SpmmArgs& a, int cfg, hipStream_t s);
hipError_t launch_spmm_smfmac_i8p(const SpmmArgs& a, int cfg, hipStream_t s);
hipError_t launch_spmm_smfmac_i8tk(const SpmmArgs& a, hipStream_t s);   // [T][K] layout
hipError_t launch_spmm_smfmac_h(const SpmmArgs& a, hipStream_t s);
hipError_t launch_spmm_smfmac_h8(const SpmmArgs& a, hipStream_t s);   // 8-wave workgroups
hipError_t launch_spmm_smfmac_hd(const SpmmArgs& a, hipStream_t s);
hipError_t launch_spmm_smfmac_i8s(const SpmmArgs& a, hipStream_t s);
bool smfmac_i8s_supported(int64_t nKB);   // column-block counts launch_spmm_smfmac_i8s instantiates
hipError_t launch_spmm_expand(const SpmmArgs& a, hipStream_t s);
hipError_t launch_spmm_expand_decode(const SpmmArgs& a, hipStream_t s);
hipError_t launch_spmm_expand32(const SpmmArgs& a, hipStream_t s);
bool expand32_supported(int N, int M);   // N:M instantiated by launch_spmm_expand32
bool expand_supported(int N, int M);   // N:M instantiated by launch_spmm_expand
// N:M patterns with at most two kept members in every aligned group of four
// columns (1:4, 1:8, 2:8), and their re-pack into the 2:4 layout of the same
// matrix (gd: Geometry::make(R, K, 2, 4, eb)), written to dvalues / dmeta.
bool repack24_supported(const Geometry& g);
hipError_t launch_repack24(const Geometry& gs, const uint8_t* values, const uint8_t* meta, const Geometry& gd,
                           uint8_t* dvalues, uint8_t* dmeta, hipStream_t s);
// dst[j][i] = src[i][j] (i < rows, j < cols), zeros for rows <= i < dst_cols;
// elements of eb bytes, row pitches lds / ldd in elements.
hipError_t launch_transpose(const void* src, int64_t rows, int64_t cols, int64_t lds, void* dst, int64_t ldd,
                            int64_t dst_cols, int eb, hipStream_t s);
// Y = epilogue(sum over the a.ksplit slices of the partials at a.ws) with
// a's own output type, bias and scale (T a multiple of 4).
hipError_t launch_splitk_reduce(const SpmmArgs& a, hipStream_t s);

// ---------------------------------------------------------------- device
// Cache policy of the output stores (gfx950 buffer-store cache bits: sc0 |
// nt).  The output is written once and never read back by the kernel;
// streaming it past the L2 keeps the packed weights and the activation strip
// that the next tiles reuse resident there instead of being evicted by it.
constexpr int kStreamStore = 3;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// binary32 -> binary16 / bfloat16 bits, round to nearest even (finite inputs;
// bfloat16 NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32 rounds to nearest even
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// erf by the rational approximation of Abramowitz & Stegun, Handbook of
// Mathematical Functions, eq. 7.1.26: for z >= 0
//   erf(z) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2) + e(z),
//   t = 1 / (1 + p z),  |e(z)| <= 1.5e-7,
// extended oddly to z < 0.  Branch-free: one reciprocal and one exp2 on the
// transcendental unit, the rest fused multiply-adds.  Evaluated in binary32
// the absolute error stays below 6e-7.
__device__ __forceinline__ float erf_as(float x) {
  const float z = __builtin_fabsf(x);
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, z, 1.0f));
  float q = __builtin_fmaf(t, 1.061405429f, -1.453152027f);
  q = __builtin_fmaf(t, q, 1.421413741f);
  q = __builtin_fmaf(t, q, -0.284496736f);
  q = __builtin_fmaf(t, q, 0.254829592f);
  q = q * t;
  const float e = __builtin_amdgcn_exp2f(-(z * z) * 1.44269504088896341f);
  return __builtin_copysignf(__builtin_fmaf(-q, e, 1.0f), x);
}

// GELU(x) = x Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), binary32 with erf_as:
// absolute error below 2.5e-7 |x| + 2.4e-7 |GELU(x)|.
__device__ __forceinline__ float gelu_f32(float x) {
  return 0.5f * x * (1.0f + erf_as(x * 0.70710678118654752440f));
}

// fp epilogue value with the activation applied (ACT) or not.
template <bool ACT>
__device__ __forceinline__ float fp_act(float x) {
  if constexpr (ACT)
    return gelu_f32(x);
  else
    return x;
}

// int8 output before rounding and saturation: f32(acc) * s, and with the
// activation act(f32(acc) * s) * os (each product one rounded binary32
// multiply).  `acc` already includes the bias.
template <bool ACT>
__device__ __forceinline__ float i8_pre(int acc, float s, float os) {
  float f = __fmul_rn((float)acc, s);
  if constexpr (ACT) f = __fmul_rn(gelu_f32(f), os);
  return f;
}

// int8 requantisation: sat(rne(f32(a) * s)); `a` already includes the bias.
// The product is one rounded binary32 multiply (no contraction into an fma),
// then round-half-even and saturation.
__device__ __forceinline__ int requant_i8(int a, float s) {
  float f = (float)a;
  float q = __fmul_rn(f, s);
  q = __builtin_rintf(q);
  q = fminf(fmaxf(q, -128.0f), 127.0f);
  return (int)q;
}

// the same with the activation between the two scales (i8_pre)
template <bool ACT>
__device__ __forceinline__ int requant_act_i8(int a, float s, float os) {
  float q = __builtin_rintf(i8_pre<ACT>(a, s, os));
  q = fminf(fmaxf(q, -128.0f), 127.0f);
  return (int)q;
}

}  // namespace nm
