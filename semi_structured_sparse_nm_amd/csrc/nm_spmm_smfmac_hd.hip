// fp16 / bf16 2:4 sparse x dense product for decode shapes (T <= 16 tokens)
// on the gfx950 sparse matrix cores (v_smfmac_f32_16x16x64_{f16,bf16}).
//
// With a handful of tokens the product is bound by streaming the packed
// weights once from HBM; the matrix cores idle.  The pages' adaptive
// parallelism ("Realizable N:M Sparse Transformer Inference via Search-Kernel
// Co-Design", Sec. 4.1: keep enough blocks in flight at inference-sized
// shapes) becomes a split of K inside a workgroup: one workgroup per 16-row
// block, its eight waves each take every eighth 64-column block, and their
// partial sums meet in LDS at the end, added in wave order (deterministic).
//
// Per wave and 64-column block, four direct-to-LDS loads bring X (64 k x 16
// tokens), the packed A fragment (1 KB) and its index words into one of
// three LDS slots of the wave; the wave waits for its own loads with an exact
// vmcnt count (no barrier in the loop) and reads A, the index words and the
// B fragment (ds_read_b64_tr_b16) from LDS.  Groups past the wave's last
// block re-read a valid block, which keeps the count exact.
// Operand mapping as in the large-T fp16 kernel (B lane group h: elements
// 0..7 = k 8 h .., 8..15 = k 32 + 8 h ..).
#include "nm_common.hpp"

namespace nm {

namespace {

typedef _Float16 v16h __attribute__((ext_vector_type(16)));
typedef __bf16 v16bf __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));

template <int WT>
__device__ __forceinline__ v4f smfmac(v4i a, v8i b, v4f c, int idx) {
  if constexpr (WT == NM_F16)
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v16h, b), c,
                                                    idx, 0, 0);
  else
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v16bf, b), c,
                                                     idx, 0, 0);
}

constexpr int NWD = 8;             // waves per workgroup (K split)
// LDS slots (load groups in flight) per wave: three slots of 3.25 KB per
// wave (78 KB per workgroup) let two workgroups share a CU, so one starts
// streaming while the other drains.  Measured on MI355X (LLaMA-7B T = 16):
// faster than four slots with one workgroup per CU (up 2:4 17.6 -> 15.0 us)
// and than six (18.8 us); two slots are within noise of three.
constexpr int D = 3;
constexpr int SLOT = 3328;         // bytes per slot: X 2 KB | A 1 KB | index words 256 B
constexpr int NLG = 4;             // loads per group

template <int WT, int OUT>
__global__ void __launch_bounds__(NWD * 64) smfmac_hd_kernel(SpmmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) uint8_t slots[NWD * D * SLOT];
  static_assert(NWD * D * SLOT <= 160 * 1024, "LDS");

  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int nKB = (int)g.nKB;
  const int ldx = (int)a.ldx;
  const int rb = blockIdx.x;                    // 16-row block
  // the waves take interleaved blocks (wave w: w, w + 8, ...), so the eight
  // waves of a workgroup stream adjacent blocks of its row block at a time
  // (measured on LLaMA-7B down 2:4, T = 16: 15.0 -> 14.5 us against
  // contiguous eighths of K)
  const int nblk = wave < nKB ? (nKB - 1 - wave) / NWD + 1 : 0;

  const v4i rx = make_rsrc(a.X, (int)(g.K * a.ldx * 2));
  const v4i rv = make_rsrc(a.values, (int)g.values_bytes());
  const v4i rm = make_rsrc(a.meta, (int)g.meta_bytes());
  uint8_t* const ws = slots + wave * (D * SLOT);

  // X slot: row r (k) at 32 r, 16-byte half h (tokens 8 h ..) at position
  // h ^ ((r >> 3) & 1).  Load j fills rows 32 j .. + 31: lane l -> row
  // 32 j + l / 2, position l % 2.
  int xoff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 32 * j + (lane >> 1);
    xoff[j] = r * ldx * 2 + 16 * ((lane & 1) ^ ((r >> 3) & 1));
  }
  // index words: 128 bytes per block; lanes 32..63 repeat lanes 0..31
  const int moff = 4 * (lane & 31);

  // group m (0 <= m < nblk: block w + 8 m) into slot m % D.  No load has all
  // its lanes outside its operand (such a load returns at once, ahead of
  // older loads; see nm_zero_page): groups past the wave's last block re-read
  // a valid block into a slot nobody reads, X rows entirely past K read the
  // zero page, so every group is the same NLG in-order loads.
  const v4i rz = zero_rsrc();
  const int kb_last = nblk > 0 ? wave + NWD * (nblk - 1) : nKB - 1;
  auto issue = [&](int m, int s) {
    const int kb = __builtin_amdgcn_readfirstlane(m < nblk ? wave + NWD * m : kb_last);
    const int krem = __builtin_amdgcn_readfirstlane((int)g.K - kb * 64);
    uint8_t* sp = ws + s * SLOT;
    const int xs = __builtin_amdgcn_readfirstlane(kb * 64 * ldx * 2);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (32 * j < krem)
        lds_dma16(rx, lds_addr(sp + 1024 * j), xoff[j], xs);
      else
        lds_dma16(rz, lds_addr(sp + 1024 * j), 16 * lane, 0);
    }
    const int blk = rb * nKB + kb;
    lds_dma16(rv, lds_addr(sp + 2048), 16 * lane, blk * 1024);
    lds_dma4(rm, lds_addr(sp + 3072), moff, blk * 128);
  };

  // B transpose reads: source lane 4 e + q reads row 8 g + e (+4, +32, +36),
  // tokens 4 q .. + 3 = half q / 2, byte 8 (q % 2)
  const int e_s = li >> 2, q_s = li & 3;
  const int bbase = (8 * lg + e_s) * 32 + 16 * ((q_s >> 1) ^ (lg & 1)) + 8 * (q_s & 1);
  const int aoff = 2048 + li * 64 + lg * 16;
  const int ioff = 3072 + li * 8 + (lg >> 1) * 4;
  const int ishift = 16 * (lg & 1);

  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < D; ++m) issue(m, m);
  for (int n = 0; n < nblk; ++n) {
    const int s = n % D;
    // D groups are in flight, this one the oldest
    __builtin_amdgcn_s_waitcnt(waitcnt(NLG * (D - 1), 15));
    const uint8_t* sp = ws + s * SLOT;
    const v4i av = *reinterpret_cast<const v4i*>(sp + aoff);
    const int idx = (int)(*reinterpret_cast<const uint32_t*>(sp + ioff) >> ishift);
    const v2i p0 = lds_tr16(sp + bbase);
    const v2i p1 = lds_tr16(sp + bbase + 128);
    const v2i p2 = lds_tr16(sp + bbase + 1024);
    const v2i p3 = lds_tr16(sp + bbase + 1152);
    acc = smfmac<WT>(av, v8i{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]}, acc, idx);
    // the slot's reads are consumed (the product waited for them): refill it
    __builtin_amdgcn_s_waitcnt(waitcnt(63, 0));
    issue(n + D, s);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));   // nothing lands in LDS after this

  // partial sums of the eight waves, added in wave order; a wave's partial
  // goes to the start of its own slots, which nothing reads or fills any more
  reinterpret_cast<v4f*>(ws)[lane] = acc;
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 256) {
    const int row = t >> 4, tok = t & 15;       // row of the block, token
    const int ln = 16 * (row >> 2) + tok, v = row & 3;
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < NWD; ++w) {
      const v4f p = reinterpret_cast<const v4f*>(slots + w * (D * SLOT))[ln];
      y += p[v];
    }
    const int64_t r = (int64_t)rb * 16 + row;
    if (r < g.R && tok < a.T) {
      if (a.bias) y += static_cast<const float*>(a.bias)[r];
      if (a.act) y = gelu_f32(y);
      const int64_t o = r * a.ldy + tok;
      if constexpr (OUT == NM_F32)
        static_cast<float*>(a.Y)[o] = y;
      else if constexpr (OUT == NM_F16)
        static_cast<uint16_t*>(a.Y)[o] = f32_to_f16_bits(y);
      else
        static_cast<uint16_t*>(a.Y)[o] = f32_to_bf16_bits(y);
    }
  }
#endif
}

}  // namespace

hipError_t launch_spmm_smfmac_hd(const SpmmArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.g.nRB), block(NWD * 64);
  if (a.wdt == NM_F16) {
    if (a.ydt == NM_F32)
      hipLaunchKernelGGL((smfmac_hd_kernel<NM_F16, NM_F32>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((smfmac_hd_kernel<NM_F16, NM_F16>), grid, block, 0, s, a);
  } else {
    if (a.ydt == NM_F32)
      hipLaunchKernelGGL((smfmac_hd_kernel<NM_BF16, NM_F32>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((smfmac_hd_kernel<NM_BF16, NM_BF16>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace nm
