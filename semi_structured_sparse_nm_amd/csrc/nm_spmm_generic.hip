// Generic N:M sparse x dense product: every dtype pair, every N:M with
// M in {4, 8}, any R, K, T, any strides.  It is the fallback variant; the
// shape-specialised kernels cover the hot configurations.
//
// Execution (paper arXiv 2607.12505, Sec. 4.2 micro-dense execution): the kept
// values of each window are materialised at their positions inside a zero
// tile in LDS, so the matrix cores only ever see regular dense fragments;
// all irregularity stays in the load / decode step.  The dense MFMA then does
// the work of the full K (the zero slots included).
//
// Tile: 64 rows x 64 tokens per workgroup of 4 waves; wave w owns rows
// 16w..16w+15 and all 64 tokens (four 16x16 accumulators).  Per column block
// of KB = 128 / element-bytes dense columns:
//   X[kb*KB .. +KB][t0 .. t0+64] -> LDS transposed (tokens major, k contiguous)
//   packed W block rows          -> LDS dense (zeros + kept values)
//   MFMA 16x16x64 i8 / 16x16x32 f16 / bf16 over the block.
// Operand lanes: lane l = 16 g + i holds row (or token) i and the contiguous
// k-chunk g of the step for both A and B, so every k meets itself in the dot
// product.  Accumulator lane l, register v holds row 4 g + v, token i.
#include "nm_common.hpp"

namespace nm {

namespace {

constexpr int BM = 64, BN = 64;
constexpr int LDS_PAD = 16;  // bytes added to every LDS row

template <int V> struct int_tag {};

template <int WT>  // 0 = int8, 1 = f16, 2 = bf16
struct Elt {
  static constexpr int EB = WT == 0 ? 1 : 2;
  static constexpr int KB = 128 / EB;   // dense columns per packed block
  static constexpr int KS = WT == 0 ? 64 : 32;  // k per MFMA
};

// accumulator: int32 for int8 operands, fp32 otherwise
template <int WT> struct AccT { typedef v4f type; };
template <> struct AccT<0> { typedef v4i type; };

__device__ __forceinline__ v4i mfma_step(const v4i& a, const v4i& b, const v4i& c, int_tag<0>) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_step(const v4i& a, const v4i& b, const v4f& c, int_tag<1>) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c,
                                                0, 0, 0);
}
__device__ __forceinline__ v4f mfma_step(const v4i& a, const v4i& b, const v4f& c, int_tag<2>) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b),
                                                 c, 0, 0, 0);
}

// position of kept slot c of a block row from its meta bits
__device__ __forceinline__ int slot_pos(const uint8_t* mrow, int MR, int c, int w) {
  int bit = c * w;
  int word = bit >> 5;
  uint32_t lo = reinterpret_cast<const uint32_t*>(mrow)[word];
  uint64_t v = lo;
  if ((word + 1) * 4 < MR) v |= (uint64_t)reinterpret_cast<const uint32_t*>(mrow)[word + 1] << 32;
  return (int)((v >> (bit & 31)) & ((1u << w) - 1));
}

template <int WT>
__global__ void __launch_bounds__(256) spmm_generic_kernel(SpmmArgs a) {
  using E = Elt<WT>;
  constexpr int EB = E::EB, KB = E::KB, KS = E::KS;
  constexpr int ROWB = KB * EB + LDS_PAD;  // LDS row pitch in bytes
  __shared__ __attribute__((aligned(16))) uint8_t Wd[BM * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t Xt[BN * ROWB];

  const Geometry& g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * BN;
  const int64_t r0 = (int64_t)blockIdx.y * BM;
  const int64_t G = g.K / g.M;
  const uint8_t* X = static_cast<const uint8_t*>(a.X);

  typedef typename AccT<WT>::type Acc;
  Acc acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = Acc{0, 0, 0, 0};

  for (int64_t kb = 0; kb < g.nKB; ++kb) {
    // ---- X tile, transposed into LDS (zeros outside K x T)
    for (int e = tid; e < KB * BN; e += 256) {
      const int t = e % BN, k = e / BN;
      const int64_t kg = kb * KB + k, tg = t0 + t;
      uint8_t* dst = Xt + t * ROWB + k * EB;
      if (EB == 1) {
        uint8_t v = (kg < g.K && tg < a.T) ? X[kg * a.ldx + tg] : (uint8_t)0;
        *dst = v;
      } else {
        uint16_t v = (kg < g.K && tg < a.T) ? reinterpret_cast<const uint16_t*>(X)[kg * a.ldx + tg]
                                             : (uint16_t)0;
        *reinterpret_cast<uint16_t*>(dst) = v;
      }
    }
    // ---- packed W block rows, expanded to dense in LDS
    for (int e = tid; e < BM * g.GB; e += 256) {
      const int rr = e / g.GB, gl = e % g.GB;
      const int64_t r = r0 + rr;
      uint8_t* dst = Wd + rr * ROWB + gl * g.M * EB;
      for (int i = 0; i < g.M * EB; ++i) dst[i] = 0;
      if (r < g.nRB * 16) {
        const int64_t blk = (r >> 4) * g.nKB + kb;
        const uint8_t* vrow = a.values + blk * g.vblk + (int64_t)(r & 15) * g.C * EB;
        const uint8_t* mrow = g.w ? a.meta + blk * g.mblk + (int64_t)(r & 15) * g.MR : nullptr;
        for (int j = 0; j < g.N; ++j) {
          const int c = gl * g.N + j;
          const int pos = g.w ? slot_pos(mrow, g.MR, c, g.w) : j;
          for (int bb = 0; bb < EB; ++bb) dst[pos * EB + bb] = vrow[c * EB + bb];
        }
      }
      (void)G;
    }
    __syncthreads();
    // ---- MFMA over the block
#pragma unroll
    for (int s = 0; s < KB / KS; ++s) {
      const int koff = (s * KS + lg * (KS / 4)) * EB;  // byte offset of this lane's chunk
      const v4i av = *reinterpret_cast<const v4i*>(Wd + (wave * 16 + li) * ROWB + koff);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const v4i bv = *reinterpret_cast<const v4i*>(Xt + (n * 16 + li) * ROWB + koff);
        acc[n] = mfma_step(av, bv, acc[n], int_tag<WT>());
      }
    }
    __syncthreads();
  }

  // ---- epilogue
#pragma unroll
  for (int n = 0; n < 4; ++n) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t r = r0 + wave * 16 + lg * 4 + v;
      const int64_t t = t0 + n * 16 + li;
      if (r >= g.R || t >= a.T) continue;
      const int64_t o = r * a.ldy + t;
      if constexpr (WT == 0) {
        int x = acc[n][v];
        if (a.bias) x += static_cast<const int32_t*>(a.bias)[r];
        if (a.ydt == NM_I32)
          static_cast<int32_t*>(a.Y)[o] = x;
        else
          static_cast<int8_t*>(a.Y)[o] = (int8_t)requant_i8(x, a.scale[r]);
      } else {
        float x = acc[n][v];
        if (a.bias) x += static_cast<const float*>(a.bias)[r];
        if (a.ydt == NM_F32)
          static_cast<float*>(a.Y)[o] = x;
        else if (a.ydt == NM_F16)
          static_cast<uint16_t*>(a.Y)[o] = f32_to_f16_bits(x);
        else
          static_cast<uint16_t*>(a.Y)[o] = f32_to_bf16_bits(x);
      }
    }
  }
}

}  // namespace

hipError_t launch_spmm_generic(const SpmmArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.T + BN - 1) / BN), (unsigned)((a.g.R + BM - 1) / BM));
  if (a.wdt == NM_I8)
    hipLaunchKernelGGL(spmm_generic_kernel<0>, grid, dim3(256), 0, s, a);
  else if (a.wdt == NM_F16)
    hipLaunchKernelGGL(spmm_generic_kernel<1>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(spmm_generic_kernel<2>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace nm
