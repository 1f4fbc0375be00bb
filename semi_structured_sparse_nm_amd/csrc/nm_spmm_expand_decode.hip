// N:M sparse x dense product for decode shapes (T <= 16 tokens), every N:M
// and weight dtype, on the gfx950 dense matrix cores.
//
// With a handful of tokens the product is bound by streaming the packed
// weights once from HBM, and a token-tiled kernel has too few tiles to keep
// the chip busy.  The pages' adaptive parallelism ("Realizable N:M Sparse
// Transformer Inference via Search-Kernel Co-Design", Sec. 4.1: keep enough
// blocks in flight at inference-sized shapes while bounding the reduction
// cost) becomes a split of K inside a workgroup: one workgroup per 16-row
// block, its eight waves each take every eighth column block, and the
// eight partial sums meet in LDS at the end, added in wave order (a fixed
// order, so fp32 results do not depend on timing).  The epilogue (bias,
// int8 requantisation or the output conversion) runs on the reduced sums.
//
// Per wave and column block, direct-to-LDS loads bring X (KB rows x 16
// tokens), the block's packed values and its meta into one of the wave's
// LDS slots (three, or two where three would not fit twice per CU); the
// wave waits for its own oldest group with an exact vmcnt count (no barrier
// in the loop).  A lane then reads its packed run and meta
// window from LDS, expands them into dense fragments in registers (Sec. 4.2
// micro-dense execution) and issues two dense MFMAs; the B fragments come
// from LDS transpose reads in the same k order.  Groups past a wave's last
// block re-read a valid block, which keeps the counts exact.
#include "nm_common.hpp"
#include "nm_expand.hpp"

namespace nm {

namespace {

typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int NWD = 8;             // waves per workgroup (K split)

// LDS slot of one column block: X (2 KB: KB rows x 16 tokens), the block's
// packed values (16 C_B bytes, in 1 KB and 256-byte loads), its meta (16 MRB
// bytes, in 256-byte loads that may run into the next block's meta).
template <int WT, int NN, int MM> struct Slot {
  typedef Run<WT, NN, MM> RG;
  static constexpr int XB = 2048;
  static constexpr int AB = 16 * RG::C_B;
  static constexpr int NAV16 = AB / 1024, NAV4 = (AB % 1024) / 256;
  static constexpr int NM4 = (16 * RG::MRB + 255) / 256;
  static constexpr int A_OFF = XB;
  static constexpr int M_OFF = XB + AB;
  static constexpr int BYTES = M_OFF + 256 * NM4;
  static constexpr int NLG = 2 + NAV16 + NAV4 + NM4;   // loads per group
  static_assert(AB % 256 == 0, "values of a block in whole 256-byte loads");
};

template <int WT, int NN, int MM, int OUT>
__global__ void __launch_bounds__(NWD * 64) expand_decode_kernel(SpmmArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef Run<WT, NN, MM> RG;
  typedef Slot<WT, NN, MM> SL;
  constexpr bool I8 = WT == NM_I8;
  constexpr int EB = RG::EB;
  typedef typename std::conditional<I8, v4i, v4f>::type Acc;

  // LDS slots (load groups in flight) per wave: three, or two where three
  // would not let two workgroups share a CU's 160 KB (one starts streaming
  // while the other drains).  Measured on MI355X (LLaMA-7B T = 16): up 4:8
  // 21.4 us with four slots and one workgroup per CU, 17.2 us with three.
  constexpr int D = (80 * 1024) / (NWD * SL::BYTES) >= 3 ? 3 : 2;
  static_assert(2 * NWD * D * SL::BYTES <= 160 * 1024, "two workgroups per CU");
  __shared__ __attribute__((aligned(1024))) uint8_t slots[NWD * D * SL::BYTES];

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

  const v4i rx = make_rsrc(a.X, (int)(g.K * a.ldx * EB));
  const v4i rv = make_rsrc(a.values, (int)g.values_bytes());
  const v4i rm = make_rsrc(a.meta, RG::W ? (int)g.meta_bytes() : 0);
  uint8_t* const ws = slots + wave * (D * SL::BYTES);

  // X slot: 16 bytes (int8) or 32 bytes (16-bit) of tokens per k row; row r
  // sits at row position s(r), which moves rows of the odd 32-row (int8) or
  // 16-row (16-bit) halves by 128 bytes so the transpose reads of lane groups
  // 0 and 1 (served together) use disjoint banks.  s is an involution.
  // Load j fills 1 KB of row positions: lane l -> position 64 j + l (int8),
  // 32 j + l / 2 and half l % 2 (16-bit).
  int xoff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if constexpr (I8) {
      const int p = 64 * j + lane;
      const int r = p ^ (((p >> 5) & 1) << 3);
      xoff[j] = r * ldx;
    } else {
      const int p = 32 * j + (lane >> 1);
      const int r = p ^ (((p >> 4) & 1) << 2);
      xoff[j] = r * ldx * 2 + 16 * (lane & 1);
    }
  }

  // group m (0 <= m < nblk: block w + 8 m) into slot m % D.  No load has all
  // its lanes outside its operand (such a load returns at once, ahead of
  // older loads; see nm_zero_page): groups past the wave's last block re-read
  // a valid block into a slot nobody reads, X rows entirely past K read the
  // zero page, so every group is the same NLG in-order loads.
  const v4i rz = zero_rsrc();
  const int kb_last = nblk > 0 ? wave + NWD * (nblk - 1) : nKB - 1;
  constexpr int XROWS = I8 ? 64 : 32;   // k rows one X load covers
  auto issue = [&](int m, int s) {
    const int kb = __builtin_amdgcn_readfirstlane(m < nblk ? wave + NWD * m : kb_last);
    const int krem = __builtin_amdgcn_readfirstlane((int)g.K - kb * (128 / EB));
    uint8_t* sp = ws + s * SL::BYTES;
    const int xs = __builtin_amdgcn_readfirstlane(kb * (128 / EB) * ldx * EB);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (XROWS * j < krem)
        lds_dma16(rx, lds_addr(sp + 1024 * j), xoff[j], xs);
      else
        lds_dma16(rz, lds_addr(sp + 1024 * j), 16 * lane, 0);
    }
    const int blk = rb * nKB + kb;
    const int vb = __builtin_amdgcn_readfirstlane(blk * SL::AB);
#pragma unroll
    for (int c = 0; c < SL::NAV16; ++c) lds_dma16(rv, lds_addr(sp + SL::A_OFF + 1024 * c), 16 * lane, vb + 1024 * c);
#pragma unroll
    for (int c = 0; c < SL::NAV4; ++c)
      lds_dma4(rv, lds_addr(sp + SL::A_OFF + 1024 * SL::NAV16 + 256 * c), 4 * lane, vb + 1024 * SL::NAV16 + 256 * c);
    const int mbase = __builtin_amdgcn_readfirstlane(blk * 16 * RG::MRB);
#pragma unroll
    for (int c = 0; c < SL::NM4; ++c) lds_dma4(rm, lds_addr(sp + SL::M_OFF + 256 * c), 4 * lane, mbase + 256 * c);
  };

  // A: lane (i, g) reads its run at row i, offset g VB; its meta window
  int mdw, mshift;
  RG::meta_window(lg, mdw, mshift);
  const int aoff = SL::A_OFF + li * RG::C_B + lg * RG::VB;
  const int moff = SL::M_OFF + li * RG::MRB + 4 * mdw;
  // B: transpose reads of rows k0 + (li >> 1) (int8: k0 = 32 g + 8 q, q = 0..3)
  // or k0 + (li >> 2) (16-bit: k0 = 16 g + 4 q); read q covers dense elements
  // 8 q .. (int8) / 4 q .. (16-bit) of the lane group's run
  // (row position: bit 7 of the byte address flips for lane groups 1 and 3)
  const int boff = I8 ? 16 * (32 * lg + (li >> 1)) + 8 * (li & 1) : 32 * (16 * lg + (li >> 2)) + 8 * (li & 3);
  const int bsw = 128 * (lg & 1);
  constexpr int BQ = 128;                       // bytes between the reads q (8 int8 or 4 16-bit rows)

  Acc acc;
#pragma unroll
  for (int v = 0; v < 4; ++v) acc[v] = 0;
#pragma unroll
  for (int m = 0; m < D; ++m) issue(m, m);
  for (int n = 0; n < nblk; ++n) {
    const int s = n % D;
    // D groups are in flight, this one the oldest
    __builtin_amdgcn_s_waitcnt(waitcnt(SL::NLG * (D - 1), 15));
    const uint8_t* sp = ws + s * SL::BYTES;
    uint32_t vd[RG::VD];
#pragma unroll
    for (int j = 0; j < RG::VD; ++j) vd[j] = *reinterpret_cast<const uint32_t*>(sp + aoff + 4 * j);
    uint64_t mb = 0;
    if constexpr (RG::W != 0) {
      uint64_t w = *reinterpret_cast<const uint32_t*>(sp + moff);
      if constexpr (RG::MRB >= 8) w |= (uint64_t)(*reinterpret_cast<const uint32_t*>(sp + moff + 4)) << 32;
      mb = w >> mshift;
    }
    const v4i da0 = expand_step<WT, NN, MM, 0>(vd, mb);
    const v4i da1 = expand_step<WT, NN, MM, 1>(vd, mb);
    v2i p[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (I8)
        p[q] = lds_tr8(sp + ((boff + BQ * q) ^ bsw));
      else
        p[q] = lds_tr16(sp + ((boff + BQ * q) ^ bsw));
    }
    acc = mfma_dense<WT>(da0, v4i{p[0][0], p[0][1], p[1][0], p[1][1]}, acc);
    acc = mfma_dense<WT>(da1, v4i{p[2][0], p[2][1], p[3][0], p[3][1]}, acc);
    // the slot's reads are consumed: refill it
    __builtin_amdgcn_s_waitcnt(waitcnt(63, 0));
    issue(n + D, s);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));   // nothing lands in LDS after this

  // partial sums of the eight waves, added in wave order
  // a wave's partial goes to the start of its own slots, which nothing reads
  // or fills any more
  reinterpret_cast<Acc*>(ws)[lane] = acc;
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 256) {
    const int row = t >> 4, tok = t & 15;       // row of the block, token
    const int ln = 16 * (row >> 2) + tok, v = row & 3;
    const int64_t r = (int64_t)rb * 16 + row;
    if (r < g.R && tok < a.T) {
      const int64_t o = r * a.ldy + tok;
      if constexpr (I8) {
        int y = 0;
#pragma unroll
        for (int w = 0; w < NWD; ++w) y += reinterpret_cast<const Acc*>(slots + w * (D * SL::BYTES))[ln][v];
        if (a.bias) y += static_cast<const int*>(a.bias)[r];
        if constexpr (OUT == NM_I8)
          static_cast<int8_t*>(a.Y)[o] = (int8_t)(a.act ? requant_act_i8<true>(y, a.scale[r], a.out_scale)
                                                        : requant_i8(y, a.scale[r]));
        else
          static_cast<int*>(a.Y)[o] = y;
      } else {
        float y = 0.f;
#pragma unroll
        for (int w = 0; w < NWD; ++w) y += reinterpret_cast<const Acc*>(slots + w * (D * SL::BYTES))[ln][v];
        if (a.bias) y += static_cast<const float*>(a.bias)[r];
        if (a.act) y = gelu_f32(y);
        if constexpr (OUT == NM_F32)
          static_cast<float*>(a.Y)[o] = y;
        else if constexpr (OUT == NM_F16)
          static_cast<uint16_t*>(a.Y)[o] = f32_to_f16_bits(y);
        else
          static_cast<uint16_t*>(a.Y)[o] = f32_to_bf16_bits(y);
      }
    }
  }
#endif
}

template <int WT, int NN, int MM, int OUT>
hipError_t launch_one(const SpmmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((expand_decode_kernel<WT, NN, MM, OUT>), dim3((unsigned)a.g.nRB), dim3(NWD * 64), 0, s, a);
  return hipGetLastError();
}

template <int WT, int NN, int MM>
hipError_t launch_nm(const SpmmArgs& a, hipStream_t s) {
  if constexpr (WT == NM_I8)
    return a.ydt == NM_I8 ? launch_one<WT, NN, MM, NM_I8>(a, s) : launch_one<WT, NN, MM, NM_I32>(a, s);
  else if constexpr (WT == NM_F16)
    return a.ydt == NM_F16 ? launch_one<WT, NN, MM, NM_F16>(a, s) : launch_one<WT, NN, MM, NM_F32>(a, s);
  else
    return a.ydt == NM_BF16 ? launch_one<WT, NN, MM, NM_BF16>(a, s) : launch_one<WT, NN, MM, NM_F32>(a, s);
}

template <int WT>
hipError_t launch_wt(const SpmmArgs& a, hipStream_t s) {
  const int N = a.g.N, M = a.g.M;
  if (M == 4) {
    if (N == 1) return launch_nm<WT, 1, 4>(a, s);
    if (N == 2) return launch_nm<WT, 2, 4>(a, s);
    if (N == 3) return launch_nm<WT, 3, 4>(a, s);
    return launch_nm<WT, 4, 4>(a, s);
  }
  if (N == 1) return launch_nm<WT, 1, 8>(a, s);
  if (N == 2) return launch_nm<WT, 2, 8>(a, s);
  if (N == 4) return launch_nm<WT, 4, 8>(a, s);
  if (N == 8) return launch_nm<WT, 8, 8>(a, s);
  return hipErrorInvalidValue;   // N:M not instantiated (the caller checks)
}

}  // namespace

hipError_t launch_spmm_expand_decode(const SpmmArgs& a, hipStream_t s) {
  if (a.wdt == NM_I8) return launch_wt<NM_I8>(a, s);
  if (a.wdt == NM_F16) return launch_wt<NM_F16>(a, s);
  return launch_wt<NM_BF16>(a, s);
}

}  // namespace nm
