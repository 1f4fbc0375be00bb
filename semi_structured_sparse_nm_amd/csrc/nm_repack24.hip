// Re-pack an N:M weight whose every aligned group of four columns holds at
// most two kept members (1:4, 1:8, 2:8) into the 2:4 packed layout of the
// same matrix, so that its product runs on the gfx950 sparse matrix
// instructions (v_smfmac, which take 2:4 operands) instead of the
// dense-expand kernels.
//
// Such a pattern is a 2:4 pattern ("Realizable N:M Sparse Transformer
// Inference via Search-Kernel Co-Design", Sec. 2.1: N kept of every M
// consecutive weights; with N = 1, or N = 2 and M = 8, no group of four
// consecutive columns can hold more than two kept members), so the re-pack
// loses nothing: the 2:4 copy describes the same dense matrix, bit for bit.
// Each group of four gets two slots at two distinct ascending positions:
//   two kept members (a 2:8 pair in one half): both, at their positions;
//   one kept member v at q: (v, 0) at (0, 1) when q = 0, else (0, v) at (0, q);
//   none: (0, 0) at (0, 1), which is also what nm_pack writes into padding.
// Positions are read as nm_pack writes them (ascending within a group), so
// two members of a 2:8 group in different halves are the first in the lower
// half and the second in the upper one.
//
// One thread per (row, column block, 32-column chunk): it reads the source's
// kept values and positions of those 32 columns (one load of 4 to 16 bytes
// and one or two dwords of positions, all issued before any is used) and
// writes 16 slots of 2:4 values (16 B for int8, 32 B for fp16 / bf16) and
// one 32-bit word of 2-bit positions.  Run inside the product call on its stream; the 2:4 copy
// lives in the caller's workspace.
#include "nm_common.hpp"

namespace nm {

namespace {

template <int EB, int M, int N>
__global__ void __launch_bounds__(256) repack24_kernel(Geometry gs, const uint8_t* __restrict__ sv,
                                                       const uint8_t* __restrict__ sm, Geometry gd,
                                                       uint8_t* __restrict__ dv, uint8_t* __restrict__ dm) {
  constexpr int KB = 128 / EB;          // dense columns per block
  constexpr int NCH = KB / 32;          // 32-column chunks per block row
  constexpr int SG = 32 / M;            // source groups per chunk
  constexpr int NS = SG * N;            // source slots per chunk
  constexpr int W = M == 4 ? 2 : 3;     // position bits
  constexpr int NVW = NS * EB / 4;      // dwords of source values per chunk (1, 2 or 4)
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = gs.nRB * 16 * gs.nKB * NCH;
  if (tid >= total) return;
  const int j = (int)(tid % NCH);
  const int64_t rk = tid / NCH;
  const int64_t kb = rk % gs.nKB;
  const int64_t r = rk / gs.nKB;         // row, padding rows included
  const int64_t blk = (r >> 4) * gs.nKB + kb;
  const int rr = (int)(r & 15);
  const int c0 = j * NS;                 // first source slot of the chunk

  // every load up front (one memory round trip): the chunk's values (NS EB
  // bytes at slot c0, aligned to their size) and the 64-bit window of the
  // row's position bitstream that holds its NS W bits; the second dword is
  // read only where the row has one (the chunk's bits never reach past the
  // row's own bytes)
  const uint32_t* vsrc =
      reinterpret_cast<const uint32_t*>(sv + blk * gs.vblk + (int64_t)rr * gs.C * EB + (int64_t)c0 * EB);
  uint32_t vw[NVW];
  if constexpr (NVW == 4) {
    const v4i t = *reinterpret_cast<const v4i*>(vsrc);
#pragma unroll
    for (int i = 0; i < 4; ++i) vw[i] = (uint32_t)t[i];
  } else if constexpr (NVW == 2) {
    typedef int v2i_ __attribute__((ext_vector_type(2)));
    const v2i_ t = *reinterpret_cast<const v2i_*>(vsrc);
    vw[0] = (uint32_t)t[0];
    vw[1] = (uint32_t)t[1];
  } else {
    vw[0] = vsrc[0];
  }
  const uint32_t* mrow = reinterpret_cast<const uint32_t*>(sm + blk * gs.mblk + (int64_t)rr * gs.MR);
  const int base = c0 * W, wi = base >> 5;
  uint64_t win = mrow[wi];
  if (wi + 1 < gs.MR / 4) win |= (uint64_t)mrow[wi + 1] << 32;
  win >>= (base & 31);

  uint32_t dval[16];                     // the chunk's 16 destination slots
  uint32_t dpos = 0;                     // their 2-bit positions
  // destination group d of the chunk: slots (s0, s1) at positions (q0, q1)
  auto put = [&](int d, uint32_t s0, uint32_t s1, uint32_t q0, uint32_t q1) {
    dval[2 * d] = s0;
    dval[2 * d + 1] = s1;
    dpos |= (q0 | (q1 << 2)) << (4 * d);
  };
  // one kept member v at q of a group of four; one_or_none: the member, or
  // none when it sits in the other half of its group of eight
  auto one = [&](int d, uint32_t v, uint32_t q) {
    put(d, q == 0 ? v : 0u, q == 0 ? 0u : v, 0u, q == 0 ? 1u : q);
  };
  auto one_or_none = [&](int d, bool here, uint32_t v, uint32_t q) {
    one(d, here ? v : 0u, here ? q : 0u);
  };
  const uint32_t vmask = EB == 1 ? 0xFFu : 0xFFFFu;
  auto value = [&](int sl) { return (vw[sl * EB / 4] >> (8 * ((sl * EB) & 3))) & vmask; };
  auto position = [&](int sl) { return (uint32_t)(win >> (sl * W)) & (uint32_t)(M - 1); };
#pragma unroll
  for (int q = 0; q < SG; ++q) {
    if constexpr (M == 4) {
      one(q, value(q), position(q));                       // 1:4
    } else if constexpr (N == 1) {
      const uint32_t v = value(q), p = position(q);        // 1:8
      one_or_none(2 * q, p < 4, v, p & 3);
      one_or_none(2 * q + 1, p >= 4, v, p & 3);
    } else {
      const uint32_t v0 = value(2 * q), p0 = position(2 * q);      // 2:8
      const uint32_t v1 = value(2 * q + 1), p1 = position(2 * q + 1);
      if ((p0 >> 2) == (p1 >> 2)) {
        // both in one half: that half holds the pair, the other none
        const bool lo = p0 < 4;
        put(2 * q, lo ? v0 : 0u, lo ? v1 : 0u, lo ? (p0 & 3) : 0u, lo ? (p1 & 3) : 1u);
        put(2 * q + 1, lo ? 0u : v0, lo ? 0u : v1, lo ? 0u : (p0 & 3), lo ? 1u : (p1 & 3));
      } else {
        one(2 * q, v0, p0 & 3);
        one(2 * q + 1, v1, p1 & 3);
      }
    }
  }

  uint8_t* vout = dv + blk * gd.vblk + (int64_t)rr * gd.C * EB + 16 * j * EB;
  if constexpr (EB == 1) {
    uint32_t wv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      wv[k] = dval[4 * k] | dval[4 * k + 1] << 8 | dval[4 * k + 2] << 16 | dval[4 * k + 3] << 24;
    *reinterpret_cast<v4i*>(vout) = v4i{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
  } else {
    uint32_t wv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) wv[k] = dval[2 * k] | dval[2 * k + 1] << 16;
    *reinterpret_cast<v4i*>(vout) = v4i{(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
    *reinterpret_cast<v4i*>(vout + 16) = v4i{(int)wv[4], (int)wv[5], (int)wv[6], (int)wv[7]};
  }
  *reinterpret_cast<uint32_t*>(dm + blk * gd.mblk + (int64_t)rr * gd.MR + 4 * j) = dpos;
}

// ---- split into two 2:4 layers.  Any N:M pattern (M = 4 or 8) holds at
// most four kept members in an aligned group of four columns, so two 2:4
// layers hold it exactly: the first layer takes the group's first two
// nonzero members in ascending position, the second the rest (the product
// is the sum of the two layers' products, each on the sparse matrix
// instructions; members holding zero add nothing and are left out, so
// padding stays in the packed format's padding form).
// A layer's group with two members stores them at their positions; with
// one member v at q, (v, 0) at (0, 1) when q = 0, else (0, v) at (0, q);
// with none, (0, 0) at (0, 1): two distinct ascending positions always.
// For M = 8 a group of eight is two groups of four: members below position
// 4 belong to the lower one, in order, the rest to the upper one.
//
// int8 only.  One thread per (row, column block, 8 columns): it loads the
// source's kept values and position bits of those 8 columns (a few dwords,
// all issued before any is used) and writes, per layer, the 4 value bytes
// (one dword) and the 8 position bits (one byte) of the 2:4 layout.
// Launch arguments of the split, 32-bit sizes (the buffers are below 2^31
// bytes), read by every thread in one batch at its start.
struct SplitArgs {
  const uint8_t* sv;   // source values / positions (the N:M packing)
  const uint8_t* sm;
  uint8_t* dv0;        // the two 2:4 layers
  uint8_t* dm0;
  uint8_t* dv1;
  uint8_t* dm1;
  int nKB;             // column blocks
  int total;           // threads: rows (padding included) x nKB x 16
  int C, vblk, MR, mblk;   // source: kept slots per block row, bytes per block, position bytes per row / block
  int vbytes, mbytes;      // source buffer sizes
};

template <int M, int N>
__global__ void __launch_bounds__(256) split24_kernel(SplitArgs a) {
  constexpr int SG = 8 / M;             // source groups per thread
  constexpr int NS = SG * N;            // source slots per thread (at most 8)
  constexpr int W = N == M ? 0 : (M == 4 ? 2 : 3);   // position bits (none when N = M)
  asm volatile("" ::"s"(a.sv), "s"(a.sm), "s"(a.dv0), "s"(a.dm0), "s"(a.dv1), "s"(a.dm1), "s"(a.nKB),
               "s"(a.total), "s"(a.C), "s"(a.vblk), "s"(a.MR), "s"(a.mblk), "s"(a.vbytes), "s"(a.mbytes));
  const int tid = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (tid >= a.total) return;
  const int t = tid & 15;                // 8-column group of the block row
  const int rk = tid >> 4;
  const int r = rk / a.nKB;              // row, padding rows included
  const int kb = rk - r * a.nKB;
  const int blk = (r >> 4) * a.nKB + kb;
  const int rr = r & 15;
  const int c0 = t * NS;                 // first source slot

  // every load up front, through range-checked buffer loads (past the end:
  // zero): the three dwords holding the NS value bytes and the two dwords
  // of the row's position bitstream holding the NS W bits (a dword past the
  // row's end belongs to the next row or reads zero; its bits are never used)
  const __amdgpu_buffer_rsrc_t rsv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.sv), 0, a.vbytes, 0x00020000);
  const int vb = blk * a.vblk + rr * a.C + c0;
  const int va = vb & ~3;
  const uint32_t w0 = __builtin_amdgcn_raw_buffer_load_b32(rsv, va, 0, 0);
  const uint32_t w1 = __builtin_amdgcn_raw_buffer_load_b32(rsv, va + 4, 0, 0);
  const uint32_t w2 = __builtin_amdgcn_raw_buffer_load_b32(rsv, va + 8, 0, 0);
  uint64_t pbits = 0;
  if constexpr (W != 0) {
    const __amdgpu_buffer_rsrc_t rsm =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.sm), 0, a.mbytes, 0x00020000);
    const int b0 = c0 * W;
    const int mo = blk * a.mblk + rr * a.MR + 4 * (b0 >> 5);
    const uint32_t m0 = __builtin_amdgcn_raw_buffer_load_b32(rsm, mo, 0, 0);
    const uint32_t m1 = __builtin_amdgcn_raw_buffer_load_b32(rsm, mo + 4, 0, 0);
    pbits = ((uint64_t)m0 | (uint64_t)m1 << 32) >> (b0 & 31);
  }
  const int sh = vb & 3;
  const uint64_t lo = ((uint64_t)w0 | (uint64_t)w1 << 32) >> (8 * sh);
  const uint64_t vbits = sh ? lo | ((uint64_t)w2 << (64 - 8 * sh)) : lo;
  auto value = [&](int sl) { return (uint32_t)(vbits >> (8 * sl)) & 0xFFu; };
  auto position = [&](int sl) -> uint32_t {
    if constexpr (W == 0)
      return (uint32_t)(sl % M);
    else
      return (uint32_t)(pbits >> (sl * W)) & (uint32_t)(M - 1);
  };

  uint32_t dval[2] = {0u, 0u};           // per layer: 4 slots, one byte each
  uint32_t dpos[2] = {0u, 0u};           // per layer: 4 slots, 2 bits each
#pragma unroll
  for (int q = 0; q < SG; ++q) {
    constexpr int H = M / 4;             // groups of four per source group
    uint32_t v[N], p[N], rank[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      v[i] = value(q * N + i);
      p[i] = position(q * N + i);
    }
    // rank of each nonzero member among the nonzero members of its group of four
#pragma unroll
    for (int i = 0; i < N; ++i) {
      rank[i] = 0;
#pragma unroll
      for (int j = 0; j < i; ++j)
        rank[i] += (v[j] != 0u && (M == 4 || (p[j] >> 2) == (p[i] >> 2))) ? 1u : 0u;
    }
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const int d = q * H + h;           // destination group of four (0 or 1)
#pragma unroll
      for (int L = 0; L < 2; ++L) {
        // the nonzero members of rank 2L and 2L + 1 within this group of four
        uint32_t xa = 0, pa = 0, xb = 0, pb = 0;
        bool ha = false, hb = false;
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const bool in = v[i] != 0u && (M == 4 || (p[i] >> 2) == (uint32_t)h);
          const bool a = in && rank[i] == (uint32_t)(2 * L), b = in && rank[i] == (uint32_t)(2 * L + 1);
          xa |= a ? v[i] : 0u;
          pa |= a ? (p[i] & 3u) : 0u;
          ha = ha || a;
          xb |= b ? v[i] : 0u;
          pb |= b ? (p[i] & 3u) : 0u;
          hb = hb || b;
        }
        uint32_t s0, s1, q0, q1;
        if (hb) {                        // two members (ascending positions)
          s0 = xa; s1 = xb; q0 = pa; q1 = pb;
        } else if (ha) {                 // one member
          s0 = pa == 0 ? xa : 0u; s1 = pa == 0 ? 0u : xa; q0 = 0u; q1 = pa == 0 ? 1u : pa;
        } else {                         // none
          s0 = 0u; s1 = 0u; q0 = 0u; q1 = 1u;
        }
        dval[L] |= (s0 | (s1 << 8)) << (16 * d);
        dpos[L] |= (q0 | (q1 << 2)) << (4 * d);
      }
    }
  }

  // the 2:4 layout: 64 value bytes and 16 position bytes per block row
  const int ov = blk * 1024 + rr * 64 + 4 * t;
  const int om = blk * 256 + rr * 16 + t;
  *reinterpret_cast<uint32_t*>(a.dv0 + ov) = dval[0];
  *reinterpret_cast<uint32_t*>(a.dv1 + ov) = dval[1];
  a.dm0[om] = (uint8_t)dpos[0];
  a.dm1[om] = (uint8_t)dpos[1];
}

}  // namespace

bool repack24_supported(const Geometry& g) {
  return g.w != 0 && ((g.M == 4 && g.N == 1) || (g.M == 8 && g.N <= 2));
}

hipError_t launch_repack24(const Geometry& gs, const uint8_t* values, const uint8_t* meta, const Geometry& gd,
                           uint8_t* dvalues, uint8_t* dmeta, hipStream_t s) {
  if (!repack24_supported(gs) || gd.N != 2 || gd.M != 4 || gd.eb != gs.eb || gd.nRB != gs.nRB ||
      gd.nKB != gs.nKB)
    return hipErrorInvalidValue;
  const int64_t total = gs.nRB * 16 * gs.nKB * (128 / gs.eb / 32);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
#define NM_REPACK(E_, M_, N_)                                                                            \
  if (gs.eb == E_ && gs.M == M_ && gs.N == N_) {                                                         \
    hipLaunchKernelGGL((repack24_kernel<E_, M_, N_>), grid, block, 0, s, gs, values, meta, gd, dvalues, dmeta); \
    return hipGetLastError();                                                                            \
  }
  NM_REPACK(1, 4, 1) NM_REPACK(1, 8, 1) NM_REPACK(1, 8, 2) NM_REPACK(2, 4, 1) NM_REPACK(2, 8, 1) NM_REPACK(2, 8, 2)
#undef NM_REPACK
  return hipErrorInvalidValue;
}


bool split24_supported(const Geometry& g) { return g.eb == 1 && (g.M == 4 || g.M == 8); }

hipError_t launch_split24(const Geometry& gs, const uint8_t* values, const uint8_t* meta, const Geometry& gd,
                          uint8_t* dvalues0, uint8_t* dmeta0, uint8_t* dvalues1, uint8_t* dmeta1, hipStream_t s) {
  if (!split24_supported(gs) || gd.N != 2 || gd.M != 4 || gd.eb != gs.eb || gd.nRB != gs.nRB || gd.nKB != gs.nKB ||
      gd.vblk != 1024 || gd.mblk != 256)
    return hipErrorInvalidValue;
  const int64_t total = gs.nRB * 16 * gs.nKB * 16;
  if (total >= (1ll << 31) || gs.values_bytes() >= (1ull << 31) || gd.values_bytes() >= (1ull << 31))
    return hipErrorInvalidValue;
  SplitArgs a;
  a.sv = values;
  a.sm = meta ? meta : values;           // N = M: no positions (never read)
  a.dv0 = dvalues0;
  a.dm0 = dmeta0;
  a.dv1 = dvalues1;
  a.dm1 = dmeta1;
  a.nKB = (int)gs.nKB;
  a.total = (int)total;
  a.C = gs.C;
  a.vblk = (int)gs.vblk;
  a.MR = gs.MR;
  a.mblk = (int)gs.mblk;
  a.vbytes = (int)gs.values_bytes();
  a.mbytes = meta ? (int)gs.meta_bytes() : 0;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
#define NM_SPLIT(M_, N_)                                                                   \
  if (gs.M == M_ && gs.N == N_) {                                                          \
    hipLaunchKernelGGL((split24_kernel<M_, N_>), grid, block, 0, s, a);                   \
    return hipGetLastError();                                                              \
  }
  NM_SPLIT(4, 1) NM_SPLIT(4, 2) NM_SPLIT(4, 3) NM_SPLIT(4, 4)
  NM_SPLIT(8, 1) NM_SPLIT(8, 2) NM_SPLIT(8, 3) NM_SPLIT(8, 4) NM_SPLIT(8, 5) NM_SPLIT(8, 6) NM_SPLIT(8, 7)
  NM_SPLIT(8, 8)
#undef NM_SPLIT
  return hipErrorInvalidValue;
}

}  // namespace nm
