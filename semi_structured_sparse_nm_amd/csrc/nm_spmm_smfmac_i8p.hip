// Persistent int8 2:4 sparse x dense product on the gfx950 sparse matrix
// cores (v_smfmac_i32_16x16x128_i8), fused bias + requantisation epilogue.
//
// Operand mapping as in the tile-per-workgroup kernel: the packed 16 x 128
// block is the v_smfmac A operand byte for byte (16 kept values per lane,
// 2-bit positions in one index word); X streams into LDS with direct-to-LDS
// buffer loads and is read back k-contiguous with ds_read_b64_tr_b8.
//
// Scheduling (the kernel side of "Realizable N:M Sparse Transformer Inference
// via Search-Kernel Co-Design", Sec. 4.1, adaptive parallelism, taken to the
// launch level): two workgroups per CU stay resident and walk a list of
// 256 x 128 output tiles.  Their loads form one continuous stream over
// (tile, 128-column block) pairs, one block ahead of the compute, so the first
// block of the next tile is in flight while the current tile's last block is
// multiplied and requantised; no tile starts cold.
//
// Waits: every step starts with vmcnt(0) -- all loads and stores issued
// before it, at least one step earlier, are complete -- and a barrier.  The
// count is exact on every path, so the compiler's own waitcnt insertion
// (which sees the register loads) needs no extra waits inside the step.
// The direct-to-LDS loads are inline asm and invisible to that pass; were
// they visible it would wait for all of them before every LDS read, because
// it cannot tell which LDS array such a load writes.
//
// Tile order: each XCD (dispatch is round-robin over 8 XCDs) owns a
// contiguous range of tiles, row tile fastest; its workgroups sweep that
// range together, so the row tiles of one 128-token strip of X run at about
// the same time on one XCD and the strip comes from HBM once into its L2.
//
// Epilogue (int8 output): f32(acc + bias[r]) * scale[r] (a separately
// rounded product), clamp to [-128, 127], add 1.5 * 2^23 so the low byte is
// the round-half-even int8, written as a byte into a per-wave row-major LDS
// staging area (16-byte chunks XOR-swizzled by row so the byte writes and the
// 16-byte reads spread over the banks), then stored as 16-byte pieces, eight
// lanes per 128-byte row segment.  int32 output: acc + bias, direct stores.
#include "nm_common.hpp"

namespace nm {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));

template <int N> struct ic { static constexpr int value = N; };

// Barrier without a memory fence (the waits that make data visible are
// explicit); the memory clobber keeps memory accesses from moving across it.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt immediate (gfx9): vmcnt bits 3:0 and 15:14, expcnt 6:4 (no
// wait), lgkmcnt 11:8.
constexpr int waitcnt(int vm, int lgkm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 0xF) << 8);
}

// Direct-to-LDS buffer loads: lane l's bytes land at M0 + size * l; offsets
// past num_records read as zero.  Completion is waited for explicitly
// (vmcnt, then a barrier).  M0 is written here; nothing else in these
// kernels uses it.
__device__ __forceinline__ v4i make_rsrc(const void* p, int num_records) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  return v4i{(int)(uint32_t)a, (int)((a >> 32) & 0xffff), num_records, 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
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

__device__ __forceinline__ v2i lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(p));
}

constexpr int RB = 4;              // row blocks (16 rows) per wave
constexpr int TN = 8;              // token tiles (16 tokens) per wave
constexpr int NW = 4;              // waves per workgroup, stacked over rows
constexpr int BM = NW * RB * 16;   // 256 rows per tile
constexpr int BN = TN * 16;        // 128 tokens per tile
[[maybe_unused]] constexpr int QB = 128 * 32;       // bytes per 32-token quarter of an X stage
constexpr int STAGE = 128 * BN;    // bytes per X stage (16 KB)
[[maybe_unused]] constexpr int DPW = STAGE / 1024 / NW;   // direct-to-LDS loads per wave per block (4)

template <bool OUT_I8>
__global__ void __launch_bounds__(256, 2) smfmac_i8p_kernel(SpmmArgs a, int mtiles, int ntiles,
                                                            int nwg_xcd) {
  // device pass only (device-only types and builtins)
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) uint8_t xs0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ostage[OUT_I8 ? NW * 64 * 128 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t bsbuf[NW * 1024];

  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int nKB = (int)g.nKB;
  const int ldx = (int)a.ldx;
  const int nRB = (int)g.nRB;

  // ---- my tiles: XCD x owns [x * per_xcd, (x + 1) * per_xcd); its nwg_xcd
  // workgroups take tiles j, j + nwg_xcd, ... of that range
  const int ntot = mtiles * ntiles;
  const int per_xcd = (ntot + 7) / 8;
  const int xcd = blockIdx.x % 8, jw = blockIdx.x / 8;
  const int lo = xcd * per_xcd;
  const int hi = min(lo + per_xcd, ntot);
  if (lo + jw >= hi) return;
  const int nmine = (hi - lo - jw + nwg_xcd - 1) / nwg_xcd;
  auto tile_of = [&](int k, int& r0, int& t0) {
    const int L = lo + jw + k * nwg_xcd;
    const int nt = L / mtiles;
    r0 = (L - nt * mtiles) * BM;
    t0 = nt * BN;
  };

  // ---- buffer resources (hardware range checks replace bounds tests)
  const v4i rx = make_rsrc(a.X, (int)(g.K * a.ldx));
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values), 0, (int)g.values_bytes(), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.meta), 0, (int)g.meta_bytes(), 0x00020000);
  const v4i rbias = make_rsrc(a.bias, a.bias ? (int)(g.R * 4) : 0);
  const v4i rscale = make_rsrc(a.scale, a.scale ? (int)(g.R * 4) : 0);

  // ---- X block loads.  Load d of a block (wave w issues d = w DPW + j)
  // covers quarter d / 4, rows 32 (d % 4) .. + 31; lane l -> row 32 (d % 4) +
  // l / 2, stored half l % 2, global half (l % 2) ^ (row bit 4).  The tile's
  // first token and the block's first row go into the scalar offset.
  int xoff[DPW];
#pragma unroll
  for (int j = 0; j < DPW; ++j) {
    const int d = wave * DPW + j;
    const int row = 32 * (d & 3) + (lane >> 1);
    const int c = (lane & 1) ^ ((row >> 4) & 1);
    xoff[j] = row * ldx + 32 * (d >> 2) + 16 * c;
  }
  auto xstage = [&](auto st) -> uint8_t* { return decltype(st)::value == 0 ? xs0 : xs1; };
  auto load_x = [&](auto st, int kb, int t0) {
    uint8_t* sp = xstage(st);
    const int soff = __builtin_amdgcn_readfirstlane(kb * 128 * ldx + t0);
#pragma unroll
    for (int j = 0; j < DPW; ++j) {
      const int d = wave * DPW + j;
      lds_dma16(rx, lds_addr(sp + (d >> 2) * QB + (d & 3) * 1024), xoff[j], soff);
    }
  };

  // ---- A fragments (lane (i, g): 16 bytes at row i, offset 16 g of a block,
  // meta dword g of row i) of row blocks rb0 .. rb0 + RB - 1, rb0 counting
  // in this wave's 64-row offset
  const int voff_v = li * 64 + lg * 16;
  const int voff_m = li * 16 + lg * 4;
  v4i av[2][RB];
  int ai[2][RB];
  auto load_a = [&](v4i* v, int* ix, int kb, int rb0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // row blocks past the matrix read past the end (zeros), without
      // letting the offset wrap
      const int blk = __builtin_amdgcn_readfirstlane(rb0 + rb < nRB ? (rb0 + rb) * nKB + kb : nRB * nKB);
      v[rb] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v, blk * 1024, 0));
      ix[rb] = (int)__builtin_amdgcn_raw_buffer_load_b32(rm, voff_m, blk * 256, 0);
    }
  };

  v4i acc[RB][TN];
  // transpose-read bases: row kq + (li >> 1) of a quarter, half li & 1,
  // stored 16-byte half c ^ (lg & 1); kq = 16 lg (+8, +64, +72)
  const int rbase = 32 * (16 * lg + (li >> 1)) + 8 * (li & 1);
  const int tb0 = rbase + 16 * (lg & 1);
  const int tb1 = rbase + 16 * ((lg & 1) ^ 1);
  auto bfrag = [&](const uint8_t* sb, int tt) -> v8i {
    const uint8_t* p = sb + (tt >> 1) * QB + ((tt & 1) ? tb1 : tb0);
    const v2i p0 = lds_tr8(p);
    const v2i p1 = lds_tr8(p + 8 * 32);
    const v2i p2 = lds_tr8(p + 64 * 32);
    const v2i p3 = lds_tr8(p + 72 * 32);
    return v8i{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  };
  // bias and scale of a tile's rows go to LDS by direct-to-LDS loads (4
  // bytes per lane: this wave's 64 rows), double-buffered by tile parity,
  // issued one tile ahead; rows past R and absent vectors read as zero.
  // Tile k's bias is read at its first block (it is the accumulator's start
  // value), its scale at its epilogue.
  uint8_t* const bsw = bsbuf + wave * 1024;
  auto load_bias_scale = [&](int k, int r0) {
    uint8_t* bs = bsw + 512 * (k & 1);
    const int soff = __builtin_amdgcn_readfirstlane(4 * (r0 + 64 * wave));
    lds_dma4(rbias, lds_addr(bs), 4 * lane, soff);
    if constexpr (OUT_I8) lds_dma4(rscale, lds_addr(bs + 256), 4 * lane, soff);
  };
  auto bias_vec = [&](int k, int rb) {
    return *reinterpret_cast<const v4i*>(bsw + 512 * (k & 1) + 4 * (16 * rb + 4 * lg));
  };
  auto scale_vec = [&](int k, int rb) {
    return *reinterpret_cast<const v4f*>(bsw + 512 * (k & 1) + 256 + 4 * (16 * rb + 4 * lg));
  };

  // acc += A x B over one block (FIRST: acc = A x B + bias, the bias, read
  // per use as an LDS broadcast, as the accumulator input).  The B fragment
  // of token tile tt + 1 is read before the products of tile tt are issued,
  // so the transpose reads' latency hides behind this wave's own SMFMACs.
  auto compute = [&](auto st, auto first, const v4i* A, const int* I, int kn) {
    constexpr bool FIRST = decltype(first)::value != 0;
    const uint8_t* sb = xstage(st);
    v8i bcur = bfrag(sb, 0);
#pragma unroll
    for (int tt = 0; tt < TN; ++tt) {
      v8i bnext;
      if (tt + 1 < TN) bnext = bfrag(sb, tt + 1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][tt] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(A[rb], bcur, FIRST ? bias_vec(kn, rb) : acc[rb][tt],
                                                               I[rb], 0, 0);
      if (tt + 1 < TN) bcur = bnext;
    }
    // issue order: reads of tile 0, then (reads of tile tt + 1, products of
    // tile tt), then the products of the last tile
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int tt = 0; tt + 1 < TN; ++tt) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
  };

  // int8 output staging: this wave's 64 rows x 128 tokens, row-major, the
  // 16-byte chunk c of row rl at position c ^ ((rl >> 2) & 7), so that the
  // byte writes of one instruction (16 tokens x 4 row groups) and the 16-byte
  // reads (8 whole rows) spread over all banks.  Byte (row 16 rb + 4 lg + v,
  // token 16 tt + li) sits at obase[tt & 3] + an immediate.
  uint8_t* const os = ostage + wave * (64 * 128);
  const int c8 = lane & 7;
  int obase[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) obase[j] = 512 * lg + 16 * (j ^ lg) + li;
  // requantise acc[rb][tt] (bias already in it): f32(acc) * scale, separately
  // rounded; clamp to [-128, 127]; + 1.5 * 2^23 leaves the round-half-even
  // integer in the low byte
  auto requant = [&](int rb, int tt, v4f sv) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float f = __fmul_rn((float)acc[rb][tt][v], sv[v]);
      f = __builtin_amdgcn_fmed3f(f, -128.0f, 127.0f);
      os[obase[tt & 3] + 2048 * rb + 128 * v + 16 * ((tt & 4) ^ (4 * (rb & 1)))] =
          (uint8_t)__builtin_bit_cast(uint32_t, f + 12582912.0f);
    }
  };
  // staged rows -> Y: piece k is row 8 k + lane / 8 of this wave, tokens
  // 16 (lane % 8) .. + 15, eight lanes per 128-byte row segment
  auto store_staged = [&](int r0, int t0) {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy), 0x00020000);
    const bool tok_ok = t0 + 16 * c8 < a.T;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int rl = 8 * k + (lane >> 3);
      const v4i piece = *reinterpret_cast<const v4i*>(os + rl * 128 + 16 * (c8 ^ ((rl >> 2) & 7)));
      if (tok_ok)
        __builtin_amdgcn_raw_buffer_store_b128(piece, ry, (r0 + 64 * wave + rl) * (int)a.ldy + t0 + 16 * c8, 0, 0);
      // a few pieces in flight at a time (registers)
      if (k & 1) __builtin_amdgcn_sched_barrier(0);
    }
  };
  // int32 output: acc (bias included) stored directly
  auto store_i32 = [&](int r0, int t0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy * 4), 0x00020000);
    const int rw = r0 + 64 * wave + 4 * lg;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) {
        if (t0 + 16 * tt >= a.T) break;
        const int t = t0 + 16 * tt + li;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          __builtin_amdgcn_raw_buffer_store_b32(acc[rb][tt][v], ry, 4 * ((rw + 16 * rb + v) * (int)a.ldy + t),
                                                0, 0);
      }
  };

  // int8 epilogue of tile k (rows r0, tokens t0)
  auto epilogue_i8 = [&](int k, int r0, int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const v4f sv = scale_vec(k, rb);
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) requant(rb, tt, sv);
    }
    store_staged(r0, t0);
  };

  // ---- cursors.  Compute: tile ck (rows cr0, tokens ct0), block ckb.  The
  // loads run one block ahead: tile lk, block lkb.
  int ck = 0, ckb = 0, cr0, ct0;
  tile_of(0, cr0, ct0);
  int lk = 0, lkb = 0, lr0 = cr0, lt0 = ct0;
  auto load_next = [&](auto st) {
    if (lk >= nmine) return;
    load_x(st, lkb, lt0);
    load_a(av[decltype(st)::value], ai[decltype(st)::value], lkb, (lr0 >> 4) + RB * wave);
    if (++lkb == nKB) {
      lkb = 0;
      if (++lk < nmine) tile_of(lk, lr0, lt0);
    }
  };

  // prologue: bias / scale of tile 0, block 0
  load_bias_scale(0, cr0);
  load_next(ic<0>());

  // One block on stage / register set ST (the next block goes to the
  // other).  Every step starts by waiting for all loads and stores issued
  // before it (at least one step earlier) and a barrier.
  bool done = false;
  auto step = [&](auto st) {
    constexpr int ST = decltype(st)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
    barrier_nofence();
    load_next(ic<ST ^ 1>());
    if (ckb == 0) {
      compute(st, ic<1>(), av[ST], ai[ST], ck);
      // tile ck - 1's bias / scale are read: their buffer takes tile ck + 1's
      if (ck + 1 < nmine) {
        int nr0, nt0;
        tile_of(ck + 1, nr0, nt0);
        __builtin_amdgcn_s_waitcnt(waitcnt(63, 0));
        load_bias_scale(ck + 1, nr0);
      }
    } else {
      compute(st, ic<0>(), av[ST], ai[ST], ck);
    }
    if (++ckb < nKB) return;
    ckb = 0;
    if constexpr (OUT_I8)
      epilogue_i8(ck, cr0, ct0);
    else
      store_i32(cr0, ct0);
    if (++ck == nmine) {
      done = true;
      return;
    }
    tile_of(ck, cr0, ct0);
  };
  for (;;) {
    step(ic<0>());
    if (done) break;
    step(ic<1>());
    if (done) break;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
#endif
}

int persistent_wgs(int device) {
  static int cache[64];
  if (device < 0 || device >= 64) return 512;
  if (!cache[device]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
      cus = 256;
    cache[device] = 2 * cus;   // two resident workgroups per CU
  }
  return cache[device];
}

}  // namespace

hipError_t launch_spmm_smfmac_i8p(const SpmmArgs& a, hipStream_t s) {
  const int mtiles = (int)((a.g.R + BM - 1) / BM);
  const int ntiles = (int)((a.T + BN - 1) / BN);
  const int ntot = mtiles * ntiles;
  const int per_xcd = (ntot + 7) / 8;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int nwg_xcd = persistent_wgs(dev) / 8;
  if (nwg_xcd > per_xcd) nwg_xcd = per_xcd;
  if (nwg_xcd < 1) nwg_xcd = 1;
  const int grid = 8 * nwg_xcd;
  if (a.ydt == NM_I8)
    hipLaunchKernelGGL((smfmac_i8p_kernel<true>), dim3(grid), dim3(256), 0, s, a, mtiles, ntiles, nwg_xcd);
  else
    hipLaunchKernelGGL((smfmac_i8p_kernel<false>), dim3(grid), dim3(256), 0, s, a, mtiles, ntiles, nwg_xcd);
  return hipGetLastError();
}

}  // namespace nm
