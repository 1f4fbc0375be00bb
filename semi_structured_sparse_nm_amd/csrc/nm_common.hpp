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
  // second 2:4 layer of a weight split into two (launch_split24; values /
  // meta hold the first): same geometry g, same block layout; nullptr else
  const uint8_t* values2 = nullptr;
  const uint8_t* meta2 = nullptr;
};

// Kernel variants; each launcher returns hipSuccess or the launch error.
hipError_t launch_pack(const void* W, int64_t ldw, const Geometry& g, int wdt, uint8_t* values,
                       uint8_t* meta, hipStream_t s);
hipError_t launch_spmm_generic(const SpmmArgs& a, hipStream_t s);
hipError_t launch_spmm_smfmac_i8p(const SpmmArgs& a, int cfg, hipStream_t s);
hipError_t launch_spmm_smfmac_i8tk(const SpmmArgs& a, hipStream_t s);   // [T][K] layout
hipError_t launch_spmm_smfmac_i8ws(const SpmmArgs& a, hipStream_t s);   // weight-stationary, K <= 768
// weight-stationary over a weight split into two 2:4 layers (a.values /
// a.meta and a.values2 / a.meta2), K <= 768
hipError_t launch_spmm_smfmac_i8ws2(const SpmmArgs& a, hipStream_t s);
// the same kernel on a dense int8 weight (N = M, its own packing), the two
// layers taken in registers (columns 0, 1 and 2, 3 of every group of four)
hipError_t launch_spmm_smfmac_i8ws2_dense(const SpmmArgs& a, hipStream_t s);
hipError_t launch_spmm_smfmac_i8wstk(const SpmmArgs& a, hipStream_t s);   // weight-stationary, [T][K] layout
hipError_t launch_spmm_smfmac_i8small(const SpmmArgs& a, hipStream_t s);   // any T, unaligned rows
hipError_t launch_spmm_smfmac_h(const SpmmArgs& a, hipStream_t s);
hipError_t launch_spmm_smfmac_hd(const SpmmArgs& a, hipStream_t s);
hipError_t launch_spmm_expand(const SpmmArgs& a, hipStream_t s);
hipError_t launch_spmm_expand_decode(const SpmmArgs& a, hipStream_t s);
bool expand_supported(int N, int M);   // N:M instantiated by launch_spmm_expand
// N:M patterns with at most two kept members in every aligned group of four
// columns (1:4, 1:8, 2:8), and their re-pack into the 2:4 layout of the same
// matrix (gd: Geometry::make(R, K, 2, 4, eb)), written to dvalues / dmeta.
bool repack24_supported(const Geometry& g);
hipError_t launch_repack24(const Geometry& gs, const uint8_t* values, const uint8_t* meta, const Geometry& gd,
                           uint8_t* dvalues, uint8_t* dmeta, hipStream_t s);
// Any N:M weight (M 4 or 8) split exactly into two 2:4 layers of the same
// matrix (gd: Geometry::make(R, K, 2, 4, eb)): in every aligned group of four
// columns the first two nonzero kept members (ascending position) go to the first
// layer, the others (at most two) to the second.
bool split24_supported(const Geometry& g);
hipError_t launch_split24(const Geometry& gs, const uint8_t* values, const uint8_t* meta, const Geometry& gd,
                          uint8_t* dvalues0, uint8_t* dmeta0, uint8_t* dvalues1, uint8_t* dmeta1, hipStream_t s);
// dst[j][i] = src[i][j] (i < rows, j < cols), zeros for rows <= i < dst_cols;
// elements of eb bytes, row pitches lds / ldd in elements.
hipError_t launch_transpose(const void* src, int64_t rows, int64_t cols, int64_t lds, void* dst, int64_t ldd,
                            int64_t dst_cols, int eb, hipStream_t s);
// Y = epilogue(sum over the a.ksplit slices of the partials at a.ws) with
// a's own output type, bias and scale (T a multiple of 4).
hipError_t launch_splitk_reduce(const SpmmArgs& a, hipStream_t s);

// Compute units of a device (cached per device; safe to call from several
// threads at once: a racing first call only repeats the query).
int cu_count(int device);

// Row tiles per group of a persistent kernel's grouped tile order (groups of
// gm row tiles, row tile fastest inside a group, then the next token tile).
// The nconc workgroups of one XCD that run together cover about gm row tiles
// x nconc / gm token tiles; per 128-column step they fetch a weight block of
// wk bytes per row tile and an activation block of xk bytes per token tile,
// and share them through the XCD's L2.  A weight that fits in the L2 (4 MB)
// stays there across token tiles, so only the activation counts: all row
// tiles in one group.  Otherwise the gm with the fewest bytes per step.
inline int tile_group_rows(int mtiles, int ntiles, int nconc, double wk, double xk, double w_total) {
  if (w_total <= 4.0 * 1024 * 1024 || mtiles <= 1) return mtiles;
  int best = mtiles;
  double best_cost = 0;
  for (int gm = 1; gm <= mtiles; ++gm) {
    const int rows = gm < nconc ? gm : nconc;
    int toks = (nconc + rows - 1) / rows;
    if (toks > ntiles) toks = ntiles;
    const double cost = rows * wk + toks * xk;
    if (gm == 1 || cost < best_cost) {
      best_cost = cost;
      best = gm;
    }
  }
  return best;
}

// ---------------------------------------------------------------- device
// Cache policy of the output stores (gfx950 buffer-store cache bits: sc0 |
// nt).  The output is written once and never read back by the kernel;
// streaming it past the L2 keeps the packed weights and the activation strip
// that the next tiles reuse resident there instead of being evicted by it.
constexpr int kStreamStore = 3;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Read the launch arguments a tile kernel's prologue needs in one batch.
// Left to itself the compiler loads each argument from the kernel-argument
// segment where it is first used, which puts several dependent scalar
// memory round trips between the workgroup's start and its first operand
// loads; an empty asm that takes them as scalar operands makes it issue
// those loads together, before any of them is waited for.
__device__ __forceinline__ void load_args_early(const SpmmArgs& a) {
  asm volatile("" ::"s"(a.X), "s"(a.Y), "s"(a.values), "s"(a.meta), "s"(a.bias), "s"(a.scale), "s"(a.ldx),
               "s"(a.ldy), "s"(a.T), "s"(a.g.R), "s"(a.g.K), "s"(a.g.nRB), "s"(a.g.nKB), "s"(a.g.vblk),
               "s"(a.g.mblk), "s"(a.out_scale));
}

// compile-time integer as a type (unrolled stage / part indices)
template <int N> struct ic { static constexpr int value = N; };

// Barrier without a memory fence (the waits that make data visible are
// explicit); the memory clobber keeps memory accesses from moving across it.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt immediate (gfx9 encoding): vmcnt bits 3:0 and 15:14, expcnt 6:4
// (no wait), lgkmcnt 11:8.
constexpr int waitcnt(int vm, int lgkm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 0xF) << 8);
}

// Raw buffer resource over [p, p + num_records) bytes: offsets past the end
// read as zero and drop stores.
__device__ __forceinline__ v4i make_rsrc(const void* p, int num_records) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  return v4i{(int)(uint32_t)a, (int)((a >> 32) & 0xffff), num_records, 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// A page of zeros in device memory (one per code object).  Every load whose
// lanes would all fall outside its operand -- row blocks past R, activation
// rows past K, a null bias or scale, the load groups a pipelined kernel issues
// past its last block -- reads from here instead.  A buffer load with every
// lane out of its resource's range returns zeros at once, ahead of older
// loads still in flight, so counting it in an explicit vmcnt wait would let
// the wait pass with those older loads (another wave's part of a staged tile)
// still outstanding.  Loads from this page are ordinary in-range loads and
// complete in issue order like the rest.
static __device__ __attribute__((aligned(256))) uint8_t nm_zero_page[4096];
// a wave-uniform condition, made visibly uniform (scalar), so that a buffer
// resource chosen by it stays in scalar registers
__device__ __forceinline__ bool uniform(bool c) { return __builtin_amdgcn_readfirstlane((int)c) != 0; }
__device__ __forceinline__ v4i zero_rsrc() { return make_rsrc(nm_zero_page, (int)sizeof nm_zero_page); }
__device__ __forceinline__ __amdgpu_buffer_rsrc_t zero_brsrc() {
  return __builtin_amdgcn_make_buffer_rsrc(nm_zero_page, 0, (int)sizeof nm_zero_page, 0x00020000);
}

// Direct-to-LDS buffer loads: lane l's bytes land at M0 + size * l; offsets
// past the resource's range read as zero.  The compiler does not see these
// loads in its wait bookkeeping: completion is waited for explicitly (vmcnt,
// then a barrier where other waves read the data).  M0 is written here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(v4i rsrc, uint32_t lds, int voff, int soff) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  soff = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(v4i rsrc, uint32_t lds, int voff, int soff) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  soff = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop

// Transposing LDS reads (ds_read_b64_tr_b8 / _b16): each lane receives 8
// bytes gathered across the lanes of its 16-lane group.
__device__ __forceinline__ v2i lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(p));
}
__device__ __forceinline__ v2i lds_tr16(const uint8_t* p) {
  typedef short v4s_ __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(
      v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_*)(p)));
}

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

// Byte B of d = the low byte of f + m, the other bytes kept (B = 0: set to
// zero).  With m = 1.5 * 2^23 and f in [-128, 127] the sum is exact in
// binary32 after rounding f half-to-even to an integer, and its low byte is
// that integer as two's-complement int8: the requantised value lands in
// its packed position in one instruction (an SDWA destination select).
template <int B>
__device__ __forceinline__ void rne_i8_byte(uint32_t& d, float f, float m) {
  static_assert(B >= 0 && B < 4, "byte 0..3");
  if constexpr (B == 0)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:DWORD"
        : "=v"(d) : "v"(f), "v"(m));
  else if constexpr (B == 1)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(d) : "v"(f), "v"(m));
  else if constexpr (B == 2)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(d) : "v"(f), "v"(m));
  else
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:DWORD"
        : "+v"(d) : "v"(f), "v"(m));
}

// Four values already clamped to [-128, 127], rounded half-to-even and
// packed as the int8 bytes 0..3 of a dword (rne_i8_byte for each).
__device__ __forceinline__ uint32_t pack_rne_i8x4(float f0, float f1, float f2, float f3) {
  const float m = 12582912.0f;   // 1.5 * 2^23
  uint32_t d;
  rne_i8_byte<0>(d, f0, m);
  rne_i8_byte<1>(d, f1, m);
  rne_i8_byte<2>(d, f2, m);
  rne_i8_byte<3>(d, f3, m);
  return d;
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
