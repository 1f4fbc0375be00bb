// int8 2:4 sparse x dense product on the gfx950 sparse matrix cores
// (v_smfmac_i32_16x16x128_i8), with the bias + requantisation epilogue fused.
//
// Paper (arXiv 2607.12505) Sec. 4.1 lists the kernel's mechanisms: packed
// weights for light decoding, micro-dense MMA-aligned execution, adaptive
// parallelism.  On CDNA4 the matrix core itself takes a 2:4 operand: the A
// operand of v_smfmac_i32_16x16x128_i8 holds, per lane (row i, lane group g),
// 16 kept int8 values covering dense k = 32 g .. 32 g + 31 of a 128-column
// block, and a 32-bit index word whose bits [2c, 2c+1] give slot c's position
// inside its group of four.  The packed layout (16-row x 128-column blocks,
// row-major kept values, little-endian 2-bit positions) is byte for byte that
// operand: lane (i, g) loads 16 bytes at row i, offset 16 g of the block and
// meta dword g of row i.  No decode step is left in the kernel; the paper's
// Sec. 4.2 aim (irregularity confined to packing and loading) is met by the
// format itself.
//
// B operand (X, [K][T] row-major, tokens contiguous): lane (token j, group g)
// needs X[k][j] for k = 16 g .. 16 g + 15 and k = 64 + 16 g .. 64 + 16 g + 15.
// X tiles stream into LDS with direct-to-LDS buffer loads (lane l's 16 bytes
// land at M0 + 16 l, out-of-range offsets read as zero) and are read back with
// ds_read_b64_tr_b8, which gives lane l of each 16-lane group byte i =
// LDS[addr(lane 2 i + l / 8) + l % 8], i.e. eight consecutive k of one token.
//
// LDS layout of one X stage (128 k x BN tokens): BN / 32 "quarters" of 32
// tokens; a quarter is 128 rows of 32 bytes (two 16-token halves), the halves
// swapped on rows with bit 4 set.  A transpose read by one lane group touches
// eight consecutive rows (8 distinct 8-dword bank groups) and the two lane
// groups served together use opposite halves, so reads are conflict-free, and
// every read address is an immediate offset from one of two per-lane bases.
//
// Pipeline: four X stages in LDS (X for block kb + 3 is in flight while block
// kb is computed) and two register sets of A fragments (block kb + 1 in
// flight); one barrier per block.
//
// Epilogue (int8 output): acc started at bias[r]; f32(acc) * scale, clamp to
// [-128, 127], add 1.5 * 2^23 so the low byte is the round-half-even int8;
// four rows are packed per dword and written token-major to LDS (16-byte
// column blocks XOR-swizzled by token), then transpose-read back so each lane
// holds eight consecutive tokens of one row and stores 8 bytes.
// int32 output: direct stores.
//
// Workgroups: 4 waves stacked over rows, each 64 rows x 128 tokens; the
// launch maps each XCD (round-robin dispatch over 8 XCDs) to a contiguous
// range of token strips, all row tiles of a strip consecutively, so a strip
// of X comes from HBM once into that XCD's L2.
#include "nm_common.hpp"

namespace nm {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

template <int N> struct ic { static constexpr int value = N; };

// Workgroup barrier without a memory fence: the waits that make the data
// visible are explicit s_waitcnt instructions before it (a fenced barrier
// would also wait for every direct-to-LDS load still in flight).  The memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt
// 6:4 (left at its maximum: no wait), lgkmcnt 11:8; 63 / 15 mean "no wait".
constexpr int waitcnt(int vm, int lgkm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 0xF) << 8);
}

__device__ __forceinline__ v2i lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(p));
}

template <int RB, int TN, bool OUT_I8>
__global__ void __launch_bounds__(256, 2) smfmac_i8_kernel(SpmmArgs a, int mtiles, int ntiles) {
  // device pass only (the body uses device-only types and builtins)
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = 4;                       // waves per workgroup, stacked over rows
  constexpr int BM = NW * RB * 16;            // rows per tile
  constexpr int BN = TN * 16;                 // tokens per tile
  constexpr int NQ = BN / 32;                 // 32-token quarters
  constexpr int QB = 128 * 32;                // bytes per quarter of a stage
  constexpr int STAGE = NQ * QB;              // bytes per X stage (128 x BN)
  constexpr int S = 4;                        // X stages in LDS (prefetch distance 3)
  constexpr int SA = 2;                       // A register sets (prefetch distance 1)
  constexpr int NDMA = STAGE / 1024;          // 1 KB direct-to-LDS loads per stage
  static_assert(NDMA % NW == 0, "stage loads must split over the waves");
  constexpr int DPW = NDMA / NW;
  static_assert(!OUT_I8 || (BN == 128 && BN * BM <= 2 * STAGE), "output staging must fit two X stages");
  static_assert(BM == 256, "the output swizzle assumes 16 column blocks per token row");
  // one array per stage: the loads in flight into one stage provably do not
  // alias reads of another, so no wait is forced before those reads
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[STAGE];

  const Geometry& g = a.g;
  const int ntot = mtiles * ntiles;
  const int per_xcd = (ntot + 7) / 8;
  const int L = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (L >= ntot) return;
  const int nt = L / mtiles, mt = L - nt * mtiles;
  const int r0 = mt * BM;
  const int t0 = nt * BN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int rb0 = (r0 >> 4) + wave * RB;      // first row block of this wave
  const int nKB = (int)g.nKB;
  const int ldx = (int)a.ldx;

  // ---- buffer resources (hardware range checks replace bounds tests)
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.X), 0, (int)(g.K * a.ldx), 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.values), 0, (int)g.values_bytes(), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.meta), 0, (int)g.meta_bytes(), 0x00020000);

  // ---- X stage loads: wave w issues loads d = w * DPW + j; load d covers
  // quarter d / 4, rows 32 (d % 4) .. + 31; lane l -> row 32 (d % 4) + l / 2,
  // stored half l % 2, global half (l % 2) ^ (row bit 4).
  int xoff[DPW];
#pragma unroll
  for (int j = 0; j < DPW; ++j) {
    const int d = wave * DPW + j;
    const int q = d >> 2, m = d & 3;
    const int row = 32 * m + (lane >> 1);
    const int c = (lane & 1) ^ ((row >> 4) & 1);
    xoff[j] = row * ldx + t0 + 32 * q + 16 * c;
  }
  auto stage_ptr = [&](auto stage_c) -> uint8_t* {
    constexpr int ST = decltype(stage_c)::value;
    return ST == 0 ? lds0 : (ST == 1 ? lds1 : (ST == 2 ? lds2 : lds3));
  };
  auto load_x = [&](int kb, auto stage_c) {
    uint8_t* sp = stage_ptr(stage_c);
    const int soff = __builtin_amdgcn_readfirstlane(kb * 128 * ldx);
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const int d = wave * DPW + j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (lds_void*)(sp + (d >> 2) * QB + (d & 3) * 1024), 16, xoff[j], soff, 0, 0);
    }
  };

  // ---- A fragments
  const int voff_v = li * 64 + lg * 16;
  const int voff_m = li * 16 + lg * 4;
  v4i av[SA][RB];
  int ai[SA][RB];
  auto load_a = [&](int kb, v4i* v, int* ix) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int blk = __builtin_amdgcn_readfirstlane((rb0 + rb) * nKB + kb);
      v[rb] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v, blk * 1024, 0));
      ix[rb] = (int)__builtin_amdgcn_raw_buffer_load_b32(rm, voff_m, blk * 256, 0);
    }
  };

  v4i acc[RB][TN];

  // ---- transpose-read bases: row kq + (li >> 1) of a quarter, half li & 1,
  // stored 16-byte half c ^ (lg & 1); kq = 16 lg (+8, +64, +72)
  const int rbase = 32 * (16 * lg + (li >> 1)) + 8 * (li & 1);
  const int tb0 = rbase + 16 * (lg & 1);         // token half 0 of a quarter
  const int tb1 = rbase + 16 * ((lg & 1) ^ 1);   // token half 1

  auto compute = [&](auto stage_c, const v4i* A, const int* I) {
    const uint8_t* sb = stage_ptr(stage_c);
#pragma unroll
    for (int tt = 0; tt < TN; ++tt) {
      const uint8_t* p = sb + (tt >> 1) * QB + ((tt & 1) ? tb1 : tb0);
      const v2i p0 = lds_tr8(p);
      const v2i p1 = lds_tr8(p + 8 * 32);
      const v2i p2 = lds_tr8(p + 64 * 32);
      const v2i p3 = lds_tr8(p + 72 * 32);
      const v8i bv = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][tt] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(A[rb], bv, acc[rb][tt], I[rb], 0, 0);
    }
  };

  // ---- bias rows of this lane, loaded first: vector loads complete in
  // order, so waiting for these does not wait for the pipeline loads below
  v4i bias_v[RB];
  {
    const __amdgpu_buffer_rsrc_t rbias = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(a.bias), 0, a.bias ? (int)(g.R * 4) : 0, 0x00020000);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      bias_v[rb] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                               rbias, 4 * (16 * (rb0 + rb) + 4 * lg), 0, 0));
  }

  // ---- prologue: X blocks 0..2 and A block 0 in flight.  Every step issues
  // its loads unconditionally (blocks at or past nKB read X as zero, out of
  // range, and are never computed), so the load stream has no branches and
  // the compiler counts outstanding loads exactly.
  load_x(0, ic<0>());
  load_a(0, av[0], ai[0]);
  load_x(1, ic<1>());
  load_x(2, ic<2>());
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int tt = 0; tt < TN; ++tt) acc[rb][tt] = bias_v[rb];   // bias == NULL reads as zero


  // one pipeline step on X stage ST, A set ST % 2.  Issue order per step:
  // A(kb + 1), then (after the barrier) X(kb + 3).  Vector loads complete in
  // issue order; at least 2 DPW + 4 RB loads are issued after X(kb) by the
  // time of this wait (prologue: A0 X1 X2 A1 / X2 A1 X3 A2; later more), so
  // waiting down to that many makes this wave's part of block kb land.  The
  // barrier then makes all of it visible and frees stage (ST + 3) % 4.  The
  // A registers of block kb are waited for by the compiler where used.
  constexpr int AHEAD = 2 * DPW + 4 * RB;
  static_assert(AHEAD < 64, "vmcnt range");
  auto step = [&](auto stage_c, int kb) {
    constexpr int ST = decltype(stage_c)::value;
    constexpr int NX = (ST + 3) % S;
    constexpr int CA = ST % SA, NA = (ST + 1) % SA;
    load_a(kb + 1, av[NA], ai[NA]);
    __builtin_amdgcn_s_waitcnt(waitcnt(AHEAD, 0));
    barrier_nofence();
    load_x(kb + 3, ic<NX>());
    compute(stage_c, av[CA], ai[CA]);
  };
  // the loop leaves as soon as the blocks run out; the path back to its top
  // always runs all four steps, so load counts at the top are exact
  for (int kb = 0;; kb += S) {
    step(ic<0>(), kb);
    if (kb + 1 >= nKB) break;
    step(ic<1>(), kb + 1);
    if (kb + 2 >= nKB) break;
    step(ic<2>(), kb + 2);
    if (kb + 3 >= nKB) break;
    step(ic<3>(), kb + 3);
    if (kb + 4 >= nKB) break;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));   // nothing lands in LDS after this
  barrier_nofence();

  // ---- epilogue
  if constexpr (OUT_I8) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.scale), 0, (int)(g.R * 4), 0x00020000);
    // token-major staging: token row t (256 bytes = 16 column blocks of 16
    // rows); column block cb stored at position cb ^ (t % 16)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // whole-vector cast: element-wise bit casts of vector lvalues are
      // miscompiled (every element reads lane 0 of the vector)
      const v4f sv = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rs, 4 * (16 * (rb0 + rb) + 4 * lg), 0, 0));
      const int cb = wave * RB + rb;
      const int wbase = 256 * li + 16 * (cb ^ li) + 4 * lg;
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) {
        uint8_t* ob = (tt < 4) ? lds0 : lds1;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float f = __fmul_rn((float)acc[rb][tt][v], sv[v]);
          f = __builtin_amdgcn_fmed3f(f, -128.0f, 127.0f);
          // byte v of the dword for rows 4 lg .. 4 lg + 3 (a byte store
          // needs no packing; each lane writes its own dword)
          ob[4096 * (tt & 3) + wbase + v] = (uint8_t)__builtin_bit_cast(uint32_t, f + 12582912.0f);
        }
      }
    }
    // Each wave re-reads only the rows it wrote, and LDS accesses of one
    // wave complete in order, so no barrier is needed from here on.
    // Read back (transpose): lane group G owns column block cb = 4 wave + G
    // (rows 16 cb + li), 8 tokens per read; the two groups served together
    // read opposite octets of each 16 tokens.
    const int cb = wave * RB + lg;
    const int s8 = 8 * (lg & 1);
    const int i8 = li >> 1, h8 = li & 1;
    const int rdA = (s8 + i8) * 256 + 16 * (cb ^ (s8 + i8)) + 8 * h8;
    const int sB = 8 - s8;
    const int rdB = (sB + i8) * 256 + 16 * (cb ^ (sB + i8)) + 8 * h8;
    // second staging, row-major: tile row r (128 bytes = 8 chunks of 16
    // tokens), chunk c stored at position c ^ ((r >> 1) & 7); rows 0..127 in
    // stage 2, 128..255 in stage 3.  Row r = 16 cb + li of this lane:
    // (r >> 1) & 7 = li >> 1.
    uint8_t* rowbuf = (wave < 2) ? lds2 : lds3;
    const int rl = (16 * cb + li) & 127;                 // row inside its stage
    const int wrA = rl * 128 + 8 * (lg & 1);
    const int wrB = rl * 128 + 8 * ((lg & 1) ^ 1);
#pragma unroll
    for (int m = 0; m < BN / 16; ++m) {
      const uint8_t* ob = (m < 4) ? lds0 : lds1;
      const v2i va = lds_tr8(ob + 4096 * (m & 3) + rdA);
      const v2i vb = lds_tr8(ob + 4096 * (m & 3) + rdB);
      const int cpos = 16 * (m ^ (li >> 1));
      *reinterpret_cast<v2i*>(rowbuf + wrA + cpos) = va;
      *reinterpret_cast<v2i*>(rowbuf + wrB + cpos) = vb;
    }
    // rows of this wave, 8 lanes per row (16 tokens each): every store
    // instruction writes eight whole 128-byte row segments
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        a.Y, 0, (int)(g.R * a.ldy), 0x00020000);
    const int c = lane & 7;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int rw = 64 * wave + 8 * k + (lane >> 3);    // tile row
      const int rs = rw & 127;
      const v4i v = *reinterpret_cast<const v4i*>(rowbuf + rs * 128 + 16 * (c ^ ((rs >> 1) & 7)));
      if (t0 + 16 * c < a.T)
        __builtin_amdgcn_raw_buffer_store_b128(v, ry, (r0 + rw) * (int)a.ldy + t0 + 16 * c, 0, kStreamStore);
    }
  } else {
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        a.Y, 0, (int)(g.R * a.ldy * 4), 0x00020000);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int tt = 0; tt < TN; ++tt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 16 * (rb0 + rb) + 4 * lg + v;
          const int t = t0 + tt * 16 + li;
          if (t < a.T)
            __builtin_amdgcn_raw_buffer_store_b32(acc[rb][tt][v], ry, 4 * (r * (int)a.ldy + t), 0, kStreamStore);
        }
  }
#endif
}

template <int RB, int TN>
hipError_t launch_cfg(const SpmmArgs& a, hipStream_t s) {
  constexpr int BM = 4 * RB * 16, BN = TN * 16;
  const int mtiles = (int)((a.g.R + BM - 1) / BM);
  const int ntiles = (int)((a.T + BN - 1) / BN);
  const int ntot = mtiles * ntiles;
  const int grid = 8 * ((ntot + 7) / 8);
  if (a.ydt == NM_I8)
    hipLaunchKernelGGL((smfmac_i8_kernel<RB, TN, true>), dim3(grid), dim3(256), 0, s, a, mtiles, ntiles);
  else
    hipLaunchKernelGGL((smfmac_i8_kernel<RB, TN, false>), dim3(grid), dim3(256), 0, s, a, mtiles, ntiles);
  return hipGetLastError();
}

}  // namespace

// 256 x 128 tile (4 waves of 64 rows x 128 tokens)
hipError_t launch_spmm_smfmac_i8(const SpmmArgs& a, int cfg, hipStream_t s) {
  switch (cfg) {
    case 0: return launch_cfg<4, 8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nm
