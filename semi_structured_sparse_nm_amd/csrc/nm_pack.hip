// nm_pack: select the kept members of every N:M group and write the blocked
// packed layout.
//
// Paper (arXiv 2607.12505) Sec. 2.1: N of every M consecutive weights are
// kept; Sec. 4.2: kept values are stored per window together with their
// positions (the packed representation), so the product kernel needs no
// separate index structure.  Selection: the N members of largest magnitude,
// equal magnitudes to the lower position.  Here that is a rank count over the
// group: member i is kept iff fewer than N members j beat it, where j beats i
// when key_j > key_i, or key_j == key_i and j < i.  Ranks are a permutation of
// 0..M-1, so exactly N members are kept, and walking i upwards emits them in
// ascending position order.  Keys: |w| for int8 (|-128| = 128), the
// sign-cleared bit pattern for fp16 / bf16 (monotone in |w| for finite values).
//
// One thread per (row, column block): it reads the row's KB dense columns,
// writes C kept values and the row's MR meta bytes.  Rows >= R and groups
// >= K / M inside the last block are padding: value 0, position = member
// number.  HBM-bound scan; run once per weight.
#include "nm_common.hpp"

namespace nm {

template <int EB, int M>
__global__ void __launch_bounds__(256) pack_kernel(const uint8_t* __restrict__ W, int64_t ldw_bytes,
                                                   Geometry g, uint8_t* __restrict__ values,
                                                   uint8_t* __restrict__ meta) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = g.nRB * 16 * g.nKB;
  if (tid >= total) return;
  const int64_t r = tid / g.nKB;
  const int64_t kb = tid - r * g.nKB;
  const int64_t rb = r >> 4;
  const int rr = (int)(r & 15);
  const int64_t blk = rb * g.nKB + kb;
  uint8_t* vrow = values + blk * g.vblk + (int64_t)rr * g.C * EB;
  uint32_t* mrow = (g.w != 0) ? reinterpret_cast<uint32_t*>(meta + blk * g.mblk + (int64_t)rr * g.MR)
                              : nullptr;
  const int64_t G = g.K / M;
  const int N = g.N;
  const int wbits = g.w;

  uint64_t bitbuf = 0;
  int nbits = 0;
  int mword = 0;
  int c = 0;
  for (int gl = 0; gl < g.GB; ++gl) {
    const int64_t grp = kb * g.GB + gl;
    const bool real = (r < g.R) && (grp < G);
    uint32_t key[M];
    uint32_t raw[M];
    if (real) {
      const uint8_t* src = W + r * ldw_bytes + grp * (int64_t)M * EB;
#pragma unroll
      for (int i = 0; i < M; ++i) {
        if (EB == 1) {
          int v = (int)(int8_t)src[i];
          raw[i] = (uint32_t)(uint8_t)v;
          key[i] = (uint32_t)(v < 0 ? -v : v);
        } else {
          uint32_t h = reinterpret_cast<const uint16_t*>(src)[i];
          raw[i] = h;
          key[i] = h & 0x7FFFu;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < M; ++i) {
        raw[i] = 0;
        key[i] = (uint32_t)(M - i);  // strictly decreasing: members 0..N-1 kept, value 0
      }
    }
#pragma unroll
    for (int i = 0; i < M; ++i) {
      int rank = 0;
#pragma unroll
      for (int j = 0; j < M; ++j)
        rank += (j != i) && ((key[j] > key[i]) || (key[j] == key[i] && j < i));
      if (rank < N) {
        if (EB == 1)
          vrow[c] = (uint8_t)raw[i];
        else
          reinterpret_cast<uint16_t*>(vrow)[c] = (uint16_t)raw[i];
        ++c;
        if (wbits) {
          bitbuf |= (uint64_t)i << nbits;
          nbits += wbits;
          if (nbits >= 32) {
            mrow[mword++] = (uint32_t)bitbuf;
            bitbuf >>= 32;
            nbits -= 32;
          }
        }
      }
    }
  }
  if (wbits) {
    if (nbits > 0) mrow[mword++] = (uint32_t)bitbuf;
    for (; mword < g.MR / 4; ++mword) mrow[mword] = 0u;
  }
}

hipError_t launch_pack(const void* W, int64_t ldw, const Geometry& g, int wdt, uint8_t* values,
                       uint8_t* meta, hipStream_t s) {
  const int64_t total = g.nRB * 16 * g.nKB;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  const int64_t ldw_bytes = ldw * g.eb;
  const uint8_t* w8 = static_cast<const uint8_t*>(W);
  (void)wdt;
  if (g.eb == 1 && g.M == 4)
    hipLaunchKernelGGL((pack_kernel<1, 4>), dim3(blocks), dim3(threads), 0, s, w8, ldw_bytes, g, values, meta);
  else if (g.eb == 1 && g.M == 8)
    hipLaunchKernelGGL((pack_kernel<1, 8>), dim3(blocks), dim3(threads), 0, s, w8, ldw_bytes, g, values, meta);
  else if (g.eb == 2 && g.M == 4)
    hipLaunchKernelGGL((pack_kernel<2, 4>), dim3(blocks), dim3(threads), 0, s, w8, ldw_bytes, g, values, meta);
  else
    hipLaunchKernelGGL((pack_kernel<2, 8>), dim3(blocks), dim3(threads), 0, s, w8, ldw_bytes, g, values, meta);
  return hipGetLastError();
}

}  // namespace nm
