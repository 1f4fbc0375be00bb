// Transpose between the two operand layouts, for the [T][K] calls that have
// no kernel of their own: X [T][K] -> X' [K][T'] (T' = T rounded up to 16,
// tokens T .. T' - 1 zero) before the [K][T] product, Y' [R][T'] -> Y [T][R]
// after it.
//
// dst[j][i] = src[i][j] for i < rows, j < cols; dst[j][i] = 0 for rows <= i
// < dst_cols (padding).  One workgroup per 64 x 64 tile of dst: the tile's
// source block is read along its rows (consecutive threads, consecutive
// elements), staged in LDS (a 65-slot row pitch, so the column reads do not
// collide on a bank) and written along dst's rows.  Elements of 1, 2 or 4
// bytes, moved as 16-byte pieces (or, for 1- and 2-byte elements, 4-byte
// words) where the pitches and pointers allow.  HBM-bound: every element is
// read and written once.
#include "nm_common.hpp"

namespace nm {

namespace {

template <int EB>
struct Elem;
template <> struct Elem<1> { typedef uint8_t T; };
template <> struct Elem<2> { typedef uint16_t T; };
template <> struct Elem<4> { typedef uint32_t T; };

template <int EB>
__global__ void __launch_bounds__(256) transpose_kernel(const uint8_t* __restrict__ src, int64_t rows, int64_t cols,
                                                        int64_t lds, uint8_t* __restrict__ dst, int64_t ldd,
                                                        int64_t dst_cols) {
  typedef typename Elem<EB>::T E;
  __shared__ E tile[64][65];
  const int64_t i0 = (int64_t)blockIdx.x * 64;   // dst column (src row) base
  const int64_t j0 = (int64_t)blockIdx.y * 64;   // dst row (src column) base
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const E* s = reinterpret_cast<const E*>(src);
  E* d = reinterpret_cast<E*>(dst);
#pragma unroll 4
  for (int r = ty; r < 64; r += 4) {
    const int64_t i = i0 + r, j = j0 + tx;
    tile[r][tx] = (i < rows && j < cols) ? s[i * lds + j] : (E)0;
  }
  __syncthreads();
#pragma unroll 4
  for (int r = ty; r < 64; r += 4) {
    const int64_t j = j0 + r, i = i0 + tx;
    if (j < cols && i < dst_cols) d[j * ldd + i] = tile[tx][r];
  }
}

// The same for 1- and 2-byte elements with 4-byte accesses on both sides
// (every row pitch and both pointers 4-byte aligned): a thread loads 4-byte
// words of source rows and, after the LDS round trip, assembles 4 / EB
// elements of one source column (consecutive source rows) into one 4-byte
// word of a destination row; consecutive threads touch consecutive words.
// Words past the matrix edges fall back to element accesses.
template <int EB>
__global__ void __launch_bounds__(256) transpose_words_kernel(const uint8_t* __restrict__ src, int64_t rows,
                                                              int64_t cols, int64_t lds, uint8_t* __restrict__ dst,
                                                              int64_t ldd, int64_t dst_cols) {
  typedef typename Elem<EB>::T E;
  constexpr int P = 4 / EB;                      // elements per 4-byte word
  constexpr int WPR = 64 / P;                    // words per 64-element row
  __shared__ E tile[64][64 + 2 * P];
  const int64_t i0 = (int64_t)blockIdx.x * 64;   // dst column (src row) base
  const int64_t j0 = (int64_t)blockIdx.y * 64;   // dst row (src column) base
  const int t = threadIdx.x;
  const E* s = reinterpret_cast<const E*>(src);
  E* d = reinterpret_cast<E*>(dst);
  // load: 64 source rows x WPR words
  for (int w = t; w < 64 * WPR; w += 256) {
    const int r = w / WPR, c = (w % WPR) * P;
    const int64_t i = i0 + r, j = j0 + c;
    E v[P];
    if (i < rows && j + P <= cols) {
      const uint32_t x = *reinterpret_cast<const uint32_t*>(s + i * lds + j);
#pragma unroll
      for (int q = 0; q < P; ++q) v[q] = (E)(x >> (8 * EB * q));
    } else {
#pragma unroll
      for (int q = 0; q < P; ++q) v[q] = (i < rows && j + q < cols) ? s[i * lds + j + q] : (E)0;
    }
#pragma unroll
    for (int q = 0; q < P; ++q) tile[r][c + q] = v[q];
  }
  __syncthreads();
  // store: 64 destination rows x WPR words
  for (int w = t; w < 64 * WPR; w += 256) {
    const int r = w / WPR, c = (w % WPR) * P;    // dst row j0 + r, dst columns i0 + c ..
    const int64_t j = j0 + r, i = i0 + c;
    if (j >= cols) continue;
    E v[P];
#pragma unroll
    for (int q = 0; q < P; ++q) v[q] = tile[c + q][r];
    if (i + P <= dst_cols) {
      uint32_t x = 0;
#pragma unroll
      for (int q = 0; q < P; ++q) x |= (uint32_t)v[q] << (8 * EB * q);
      *reinterpret_cast<uint32_t*>(d + j * ldd + i) = x;
    } else {
#pragma unroll
      for (int q = 0; q < P; ++q)
        if (i + q < dst_cols) d[j * ldd + i + q] = v[q];
    }
  }
}

// The same with 16-byte accesses on both sides (every row pitch and both
// pointers 16-byte aligned): a thread loads 16-byte pieces of source rows
// and, after the LDS round trip, gathers 16 / EB elements of one source
// column (consecutive source rows) into one 16-byte piece of a destination
// row.  Pieces past the matrix edges fall back to element accesses.
template <int EB>
__global__ void __launch_bounds__(256) transpose_vec_kernel(const uint8_t* __restrict__ src, int64_t rows,
                                                            int64_t cols, int64_t lds, uint8_t* __restrict__ dst,
                                                            int64_t ldd, int64_t dst_cols) {
  typedef typename Elem<EB>::T E;
  constexpr int P = 16 / EB;                     // elements per 16-byte piece
  constexpr int PPR = 64 / P;                    // pieces per 64-element row
  constexpr int PITCH = 64 + P;                  // tile row pitch in elements (16-byte multiple)
  __shared__ __attribute__((aligned(16))) E tile[64 * PITCH];
  const int64_t i0 = (int64_t)blockIdx.x * 64;   // dst column (src row) base
  const int64_t j0 = (int64_t)blockIdx.y * 64;   // dst row (src column) base
  const int t = threadIdx.x;
  const E* s = reinterpret_cast<const E*>(src);
  E* d = reinterpret_cast<E*>(dst);
  for (int w = t; w < 64 * PPR; w += 256) {
    const int r = w / PPR, c = (w % PPR) * P;
    const int64_t i = i0 + r, j = j0 + c;
    if (i < rows && j + P <= cols) {
      *reinterpret_cast<v4i*>(&tile[r * PITCH + c]) = *reinterpret_cast<const v4i*>(s + i * lds + j);
    } else {
#pragma unroll
      for (int q = 0; q < P; ++q) tile[r * PITCH + c + q] = (i < rows && j + q < cols) ? s[i * lds + j + q] : (E)0;
    }
  }
  __syncthreads();
  for (int w = t; w < 64 * PPR; w += 256) {
    const int r = w / PPR, c = (w % PPR) * P;    // dst row j0 + r, dst columns i0 + c ..
    const int64_t j = j0 + r, i = i0 + c;
    if (j >= cols) continue;
    E v[P];
#pragma unroll
    for (int q = 0; q < P; ++q) v[q] = tile[(c + q) * PITCH + r];
    if (i + P <= dst_cols) {
      uint32_t x[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int q = 0; q < P; ++q) x[(q * EB) / 4] |= (uint32_t)v[q] << (8 * ((q * EB) % 4));
      *reinterpret_cast<v4i*>(d + j * ldd + i) = v4i{(int)x[0], (int)x[1], (int)x[2], (int)x[3]};
    } else {
#pragma unroll
      for (int q = 0; q < P; ++q)
        if (i + q < dst_cols) d[j * ldd + i + q] = v[q];
    }
  }
}

}  // namespace

hipError_t launch_transpose(const void* src, int64_t rows, int64_t cols, int64_t lds, void* dst, int64_t ldd,
                            int64_t dst_cols, int eb, hipStream_t s) {
  if (rows < 0 || cols < 0 || dst_cols < rows || lds < cols || ldd < dst_cols) return hipErrorInvalidValue;
  if (cols == 0 || dst_cols == 0) return hipSuccess;
  const dim3 grid((unsigned)((dst_cols + 63) / 64), (unsigned)((cols + 63) / 64)), block(256);
  const uint8_t* sp = static_cast<const uint8_t*>(src);
  uint8_t* dp = static_cast<uint8_t*>(dst);
  const bool words = (eb == 1 || eb == 2) && (lds * eb) % 4 == 0 && (ldd * eb) % 4 == 0 &&
                     (uintptr_t)src % 4 == 0 && (uintptr_t)dst % 4 == 0;
  const bool vec = (lds * eb) % 16 == 0 && (ldd * eb) % 16 == 0 && (uintptr_t)src % 16 == 0 &&
                   (uintptr_t)dst % 16 == 0;
  switch (eb) {
    case 1:
      if (vec)
        hipLaunchKernelGGL((transpose_vec_kernel<1>), grid, block, 0, s, sp, rows, cols, lds, dp, ldd, dst_cols);
      else if (words)
        hipLaunchKernelGGL((transpose_words_kernel<1>), grid, block, 0, s, sp, rows, cols, lds, dp, ldd, dst_cols);
      else
        hipLaunchKernelGGL((transpose_kernel<1>), grid, block, 0, s, sp, rows, cols, lds, dp, ldd, dst_cols);
      break;
    case 2:
      if (vec)
        hipLaunchKernelGGL((transpose_vec_kernel<2>), grid, block, 0, s, sp, rows, cols, lds, dp, ldd, dst_cols);
      else if (words)
        hipLaunchKernelGGL((transpose_words_kernel<2>), grid, block, 0, s, sp, rows, cols, lds, dp, ldd, dst_cols);
      else
        hipLaunchKernelGGL((transpose_kernel<2>), grid, block, 0, s, sp, rows, cols, lds, dp, ldd, dst_cols);
      break;
    case 4:
      if (vec)
        hipLaunchKernelGGL((transpose_vec_kernel<4>), grid, block, 0, s, sp, rows, cols, lds, dp, ldd, dst_cols);
      else
        hipLaunchKernelGGL((transpose_kernel<4>), grid, block, 0, s, sp, rows, cols, lds, dp, ldd, dst_cols);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nm
