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
// Each thread issues every global load of a block (its X elements, its
// (row, group) entries' kept values and meta dwords) before its first LDS
// store, so a block costs one memory round trip; the kernel is templated on
// M so those counts are compile-time.
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

// TK: the PyTorch-linear layout, X [T][ldx] with K contiguous and Y [T][ldy]
// with R contiguous; otherwise X [K][ldx] and Y [R][ldy].
template <int WT, int MM, bool TK>
__global__ void __launch_bounds__(256) spmm_generic_kernel(SpmmArgs a) {
  using E = Elt<WT>;
  constexpr int EB = E::EB, KB = E::KB, KS = E::KS;
  constexpr int ROWB = KB * EB + LDS_PAD;  // LDS row pitch in bytes
  constexpr int TPR = 256 / KB;            // threads per X row of a block
  constexpr int XPT = BN / TPR;            // X elements per thread and block
  constexpr int GB = KB / MM;              // groups per block row
  constexpr int EPT = BM * GB / 256;       // (row, group) entries per thread and block
  static_assert(256 % KB == 0 && BN % TPR == 0 && (BM * GB) % 256 == 0, "staging shapes");
  __shared__ __attribute__((aligned(16))) uint8_t Wd[BM * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t Xt[BN * ROWB];

  const Geometry& g = a.g;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * BN;
  const int64_t r0 = (int64_t)blockIdx.y * BM;
  const uint8_t* X = static_cast<const uint8_t*>(a.X);
  const int N = g.N, w = g.w;

  typedef typename AccT<WT>::type Acc;
  Acc acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = Acc{0, 0, 0, 0};

  // Every load of a block is issued before the first LDS store, so a block
  // costs one memory round trip, not one per element.
  // [K][T]: this thread's X row and first token (tokens contiguous);
  // [T][K]: its token and first k (a contiguous run of XPT k)
  constexpr int TPT = 256 / BN;            // threads per token in the [T][K] layout
  static_assert(KB % TPT == 0 && KB / TPT == XPT, "[T][K] staging shape");
  const int xk = TK ? (tid % TPT) * XPT : tid / TPR;
  const int xt = TK ? tid / TPT : (tid % TPR) * XPT;
  for (int64_t kb = 0; kb < g.nKB; ++kb) {
    // ---- X tile (zeros outside K x T), token-major in LDS
    uint32_t xv[XPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int64_t kg = kb * KB + xk + (TK ? i : 0);
      const int64_t tg = t0 + xt + (TK ? 0 : i);
      const bool ok = kg < g.K && tg < a.T;
      const int64_t off = TK ? tg * a.ldx + kg : kg * a.ldx + tg;
      if constexpr (EB == 1)
        xv[i] = ok ? X[off] : 0u;
      else
        xv[i] = ok ? reinterpret_cast<const uint16_t*>(X)[off] : 0u;
    }
    // ---- packed W: entry (row, group) e = tid + 256 i; its N kept values
    // and the meta bits of its positions (two dwords around them)
    uint32_t wv[EPT][MM];
    uint32_t mw[EPT][2];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid + 256 * i;
      const int rr = e / GB, gl = e % GB;
      const int64_t r = r0 + rr;
      const bool live = r < g.nRB * 16;
      const int64_t blk = (r >> 4) * g.nKB + kb;
      const uint8_t* vrow = a.values + blk * g.vblk + (int64_t)(r & 15) * g.C * EB;
#pragma unroll
      for (int j = 0; j < MM; ++j) {
        uint32_t v = 0;
        if (live && j < N) {
          if constexpr (EB == 1)
            v = vrow[gl * N + j];
          else
            v = reinterpret_cast<const uint16_t*>(vrow)[gl * N + j];
        }
        wv[i][j] = v;
      }
      mw[i][0] = mw[i][1] = 0;
      if (live && w) {
        const uint8_t* mrow = a.meta + blk * g.mblk + (int64_t)(r & 15) * g.MR;
        const int word = (gl * N * w) >> 5;
        mw[i][0] = reinterpret_cast<const uint32_t*>(mrow)[word];
        if ((word + 1) * 4 < g.MR) mw[i][1] = reinterpret_cast<const uint32_t*>(mrow)[word + 1];
      }
    }
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      uint8_t* dst = TK ? Xt + xt * ROWB + (xk + i) * EB : Xt + (xt + i) * ROWB + xk * EB;
      if constexpr (EB == 1)
        *dst = (uint8_t)xv[i];
      else
        *reinterpret_cast<uint16_t*>(dst) = (uint16_t)xv[i];
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const int e = tid + 256 * i;
      const int rr = e / GB, gl = e % GB;
      uint8_t* dst = Wd + rr * ROWB + gl * MM * EB;
      uint32_t dense[MM];
#pragma unroll
      for (int p = 0; p < MM; ++p) dense[p] = 0;
      const uint64_t win = ((uint64_t)mw[i][1] << 32) | mw[i][0];
      const int bit0 = (gl * N * w) & 31;
#pragma unroll
      for (int j = 0; j < MM; ++j) {
        if (j < N) {
          const int pos = w ? (int)((win >> (bit0 + j * w)) & ((1u << w) - 1)) : j;
#pragma unroll
          for (int p = 0; p < MM; ++p)
            if (p == pos) dense[p] = wv[i][j];
        }
      }
#pragma unroll
      for (int p = 0; p < MM; ++p) {
        if constexpr (EB == 1)
          dst[p] = (uint8_t)dense[p];
        else
          reinterpret_cast<uint16_t*>(dst)[p] = (uint16_t)dense[p];
      }
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
      const int64_t o = TK ? t * a.ldy + r : r * a.ldy + t;
      if constexpr (WT == 0) {
        int x = acc[n][v];
        if (a.bias) x += static_cast<const int32_t*>(a.bias)[r];
        if (a.ydt == NM_I32)
          static_cast<int32_t*>(a.Y)[o] = x;
        else
          static_cast<int8_t*>(a.Y)[o] = (int8_t)(a.act ? requant_act_i8<true>(x, a.scale[r], a.out_scale)
                                                        : requant_i8(x, a.scale[r]));
      } else {
        float x = acc[n][v];
        if (a.bias) x += static_cast<const float*>(a.bias)[r];
        if (a.act) x = gelu_f32(x);
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
  void (*k)(SpmmArgs);
  const bool m4 = a.g.M == 4;
  if (a.layout == NM_LAYOUT_TK) {
    if (a.wdt == NM_I8)
      k = m4 ? spmm_generic_kernel<0, 4, true> : spmm_generic_kernel<0, 8, true>;
    else if (a.wdt == NM_F16)
      k = m4 ? spmm_generic_kernel<1, 4, true> : spmm_generic_kernel<1, 8, true>;
    else
      k = m4 ? spmm_generic_kernel<2, 4, true> : spmm_generic_kernel<2, 8, true>;
  } else {
    if (a.wdt == NM_I8)
      k = m4 ? spmm_generic_kernel<0, 4, false> : spmm_generic_kernel<0, 8, false>;
    else if (a.wdt == NM_F16)
      k = m4 ? spmm_generic_kernel<1, 4, false> : spmm_generic_kernel<1, 8, false>;
    else
      k = m4 ? spmm_generic_kernel<2, 4, false> : spmm_generic_kernel<2, 8, false>;
  }
  hipLaunchKernelGGL(k, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace nm
