// Weight-stationary int8 2:4 sparse x dense product on the gfx950 sparse
// matrix cores (v_smfmac_i32_16x16x128_i8), fused bias + requantisation, for
// reduction lengths of up to 8 column blocks (K <= 1024: the ViT-B QKV,
// projection and FC1 layers).
//
// The packed weights are what every token tile of a row block shares, so
// this kernel keeps them in registers: each wave holds the packed values and
// index words of its 32 rows over the whole of K (NKB blocks x 2 row blocks x
// 5 VGPRs), and its workgroup walks a run of token tiles of one row block,
// streaming only X through LDS.  Per 256 x 128 output tile the vector memory
// path then carries the X strip and the output, not the weights again: about
// 2.5 times fewer vector memory instructions per tile than a kernel that
// re-reads the weights for every tile, which is the resource such a kernel
// runs out of first.  The pages' adaptive parallelism ("Realizable N:M Sparse
// Transformer Inference via Search-Kernel Co-Design", Sec. 4.1) is the
// work split: each XCD owns a contiguous range of token strips (about 1 MB
// of X that stays in its L2) for all row blocks, and its workgroups take
// equal contiguous runs of its (row block, token strip) list, row block
// major, so a workgroup loads the weights of one or two row blocks.
//
// Per wave: 32 rows (two 16-row blocks) x 128 tokens, eight waves per
// workgroup (256 rows), one workgroup per CU (two waves per SIMD).  X stages
// (128 k x 128 tokens) arrive by direct-to-LDS loads, NST deep (NST divides
// NKB, so the stage of a block is known at compile time); B fragments are
// read k-contiguous with ds_read_b64_tr_b8.  Operand mapping as in the other
// int8 2:4 kernels: the packed 16 x 128 block is the A operand byte for byte
// (lane (i, g): 16 bytes at row i, offset 16 g; index word g of row i).
//
// Waits: a step waits until at most the X loads of the NST - 2 later groups
// are outstanding (loads complete in order among themselves; stores and
// weight reloads issued later only make the wait longer), then a barrier
// publishes every wave's part of the stage.  Weight and bias registers are
// ordinary loads that the compiler waits for.
//
// Epilogue as in the dense-expand kernel (two 16-row blocks per wave): fp32
// scale, clamp, round half to even through a 1.5 * 2^23 add, four rows
// packed per dword, LDS staging, transpose reads, 16-byte streaming stores.
#include "nm_common.hpp"

namespace nm {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));

template <int N> struct ic { static constexpr int value = N; };

__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }
constexpr int waitcnt(int vm, int lgkm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 0xF) << 8);
}
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

constexpr int NW = 8;              // waves per workgroup
constexpr int BM = 256;            // rows per tile
constexpr int BN = 128;            // tokens per tile
constexpr int STAGE = 128 * BN;    // bytes per X stage (16 KB)
constexpr int DPW = STAGE / 1024 / NW;   // 1 KB direct-to-LDS loads per wave per block

// X stages: the largest of 3, 4, 2 that divides NKB, else NKB itself
constexpr int nst_for(int nkb) { return nkb % 3 == 0 ? 3 : (nkb % 4 == 0 ? 4 : (nkb % 2 == 0 ? 2 : nkb)); }

// Per wave 2 row blocks (16 rows) x 8 token tiles (16 tokens), waves stacked
// over the 256 rows.  (A 4 x 4 layout, with half the LDS B reads per product
// and twice the weight registers, measured slower on the ViT-B shapes: FC1
// 35.2 us against 33.1 us.)
template <int NKB, bool OUT_I8>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
smfmac_i8s_kernel(SpmmArgs a, int mtiles, int ntiles) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int RB = 2;                      // row blocks per wave
  constexpr int TN = 8;                      // token tiles per wave
  constexpr int WR = BM / (16 * RB);         // waves over the rows
  static_assert(WR * (BN / (16 * TN)) == NW, "waves tile the 256 x 128 output");
  constexpr int NST = nst_for(NKB);
  static_assert(NKB % NST == 0 && NST >= 2, "the stage of a block is its column block mod NST");
  constexpr int ALLOW = DPW * (NST - 2);     // X loads of later groups a step may leave in flight

  __shared__ __attribute__((aligned(1024))) uint8_t xs[NST][STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ostage[OUT_I8 ? NW * 1024 * RB : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t bsbuf[NW * 512];   // per wave: bias | scale rows

  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int wr = wave % WR, wt = wave / WR;  // the wave's rows 16 RB wr .., tokens 16 TN wt ..
  const int ldx = (int)a.ldx;
  const int nRB = (int)g.nRB;

  // ---- my tiles: XCD x owns token strips [tx0, tx1) of every row block;
  // its workgroups split the (row block, strip) list, row block major, into
  // equal contiguous runs
  const int nwg_xcd = gridDim.x / 8;
  const int xcd = blockIdx.x % 8, jw = blockIdx.x / 8;
  const int tx0 = xcd * ntiles / 8, tx1 = (xcd + 1) * ntiles / 8, ntx = tx1 - tx0;
  const int Tx = mtiles * ntx;
  const int L0 = jw * Tx / nwg_xcd, L1 = (jw + 1) * Tx / nwg_xcd;
  const int nmine = L1 - L0;
  if (nmine <= 0) return;
  const int total = nmine * NKB;               // blocks this workgroup computes
  auto tile_of = [&](int k, int& rbt, int& t0) {
    const int L = L0 + k;
    rbt = L / ntx;
    t0 = (tx0 + L - rbt * ntx) * BN;
  };

  const v4i rx = make_rsrc(a.X, (int)(g.K * a.ldx));
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values), 0, (int)g.values_bytes(), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.meta), 0, (int)g.meta_bytes(), 0x00020000);
  const v4i rbias = make_rsrc(a.bias, a.bias ? (int)(g.R * 4) : 0);
  const v4i rscale = make_rsrc(a.scale, a.scale ? (int)(g.R * 4) : 0);

  // ---- X stage layout: 128 rows (k) of 128 bytes (tokens); the 16-byte
  // chunk of tokens 16 c .. + 15 of row r sits at position c ^ f(r),
  // f(r) = (r & 7) ^ ((r >> 4) & 1).  Load d (wave w issues d = w DPW + j)
  // fills rows 8 d .. + 7: lane l -> row 8 d + l / 8, position l % 8.
  auto xoff = [&](int j) {
    const int d = wave * DPW + j;
    const int row = 8 * d + (lane >> 3);
    const int c = (lane & 7) ^ (row & 7) ^ ((row >> 4) & 1);
    return row * ldx + 16 * c;
  };

  // ---- load cursor over (tile, block) groups: ln issued, tile lk (row
  // block lrb, tokens lt0), block lkb.  Groups past the end load zeros into
  // a stage nobody reads again, so every group is DPW loads.
  int ln = 0, lk = 0, lkb = 0, lrb = 0, lt0 = 0;
  tile_of(0, lrb, lt0);
  int g_soff = 0;
  auto issue_part = [&](auto st, auto part) {
    constexpr int S = decltype(st)::value;
    constexpr int J = decltype(part)::value;
    if constexpr (J == 0)
      g_soff = __builtin_amdgcn_readfirstlane(ln < total ? lkb * 128 * ldx + lt0 : (int)(g.K * a.ldx));
    const int d = wave * DPW + J;
    lds_dma16(rx, lds_addr(&xs[S][d * 1024]), xoff(J), g_soff);
    if constexpr (J == DPW - 1) {
      if (ln < total && ++lkb == NKB) {
        lkb = 0;
        if (++lk < nmine) tile_of(lk, lrb, lt0);
      }
      ++ln;
    }
  };
  static_assert(DPW == 2, "two X loads per wave and block");

  // ---- stationary weights of the current row block: lane (i, g) of row
  // block rb, column block kb: 16 value bytes at row i, offset 16 g; index
  // word g of row i.  Bias and scale of the wave's rows go to its LDS slot
  // (64 rows from its first; rows past R read as zero).
  v4i av[NKB][RB];
  int ai[NKB][RB];
  uint8_t* const bsw = bsbuf + wave * 512;
  auto bias_vec = [&](int rb) { return *reinterpret_cast<const v4i*>(bsw + 4 * (16 * rb + 4 * lg)); };
  auto scale_vec = [&](int rb) { return *reinterpret_cast<const v4f*>(bsw + 256 + 4 * (16 * rb + 4 * lg)); };
  const int voff_v = li * 64 + lg * 16;
  const int voff_m = li * 16 + lg * 4;
  auto load_weights = [&](int rbt) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rbi = __builtin_amdgcn_readfirstlane(rbt * (BM / 16) + RB * wr + rb);
      const int rbc = min(rbi, nRB);             // past the matrix: reads zeros
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int blk = rbc * NKB + kb;
        av[kb][rb] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v, blk * 1024, 0));
        ai[kb][rb] = (int)__builtin_amdgcn_raw_buffer_load_b32(rm, voff_m, blk * 256, 0);
      }
    }
    const int boff = 4 * (rbt * BM + 16 * RB * wr + lane);
    lds_dma4(rbias, lds_addr(bsw), boff, 0);
    if constexpr (OUT_I8) lds_dma4(rscale, lds_addr(bsw + 256), boff, 0);
    // wait here for the whole reload (loads complete in order, so this also
    // drains the X groups in flight; it happens once or twice per
    // workgroup), so no path reaches the block loop with these registers
    // still pending -- otherwise the compiler's own waits at their first use,
    // merged over both paths and with stores outstanding, would drain the
    // pipeline at every tile
    __builtin_amdgcn_s_waitcnt(waitcnt(0, 15));
  };

  // ---- B fragments: lane (i, g) reads rows kq + 16 g + i / 2 (kq = 0, 8,
  // 64, 72), tokens 16 tt + 8 (i & 1) .. + 7 (chunk tt at tt ^ f(r))
  const int xb = (128 * (16 * lg + (li >> 1)) + 8 * (li & 1)) | (16 * ((li >> 1) ^ (lg & 1)));
  auto bfrag = [&](const uint8_t* sb, int tt) -> v8i {
    int o = xb ^ (16 * (TN * wt + tt));
    asm volatile("" : "+v"(o));
    const uint8_t* p = sb + o;
    const v2i p0 = lds_tr8(p);
    const v2i p1 = lds_tr8(p + 8 * 128);
    const v2i p2 = lds_tr8(p + 64 * 128);
    const v2i p3 = lds_tr8(p + 72 * 128);
    return v8i{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  };

  v4i acc[RB][TN];
  auto init_acc = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const v4i b = bias_vec(rb);
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) acc[rb][tt] = b;
    }
  };

  // one block: wait for its group, publish the stage, 8 token tiles x 2 row
  // blocks of sparse products; the group NST - 1 blocks ahead is issued in
  // two parts after the first two token tiles
  auto step = [&](auto kbc) {
    constexpr int KB = decltype(kbc)::value;
    constexpr int ST = KB % NST;
    constexpr int NX = (KB + NST - 1) % NST;
    __builtin_amdgcn_s_waitcnt(waitcnt(ALLOW, 15));
    barrier_nofence();
    const uint8_t* sb = xs[ST];
    v8i bf[3];
#pragma unroll
    for (int tt = 0; tt < 3; ++tt) bf[tt] = bfrag(sb, tt);
    auto tile = [&](auto ttc) {
      constexpr int tt = decltype(ttc)::value;
      if constexpr (tt >= 1 && tt + 2 < TN) bf[(tt + 2) % 3] = bfrag(sb, tt + 2);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][tt] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(av[KB][rb], bf[tt % 3], acc[rb][tt], ai[KB][rb], 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (tt < DPW) issue_part(ic<NX>(), ic<tt>());
      __builtin_amdgcn_sched_barrier(0);
    };
    tile(ic<0>()); tile(ic<1>()); tile(ic<2>()); tile(ic<3>());
    tile(ic<4>()); tile(ic<5>()); tile(ic<6>()); tile(ic<7>());
  };
  // steps 0 .. NKB - 1 (a generic lambda that calls itself with the next index)
  auto steps_from = [&](auto self, auto kbc) -> void {
    constexpr int KB = decltype(kbc)::value;
    step(kbc);
    if constexpr (KB + 1 < NKB) self(self, ic<KB + 1>());
  };

  // ---- epilogues.  The wave's output block: rows r0 + 16 RB wr .., tokens
  // t0 + 16 TN wt ..
  uint8_t* const os = ostage + (OUT_I8 ? wave * 1024 * RB : 0);
  // Per half (64 tokens), staging position p = 8 g + 4 rb + v of a token
  // holds wave row 16 rb + 4 g + v; token t (0..63) is a 32-byte row,
  // f(t) = ((t >> 4) & 1) << 1 over 8-byte chunks; reads: lane 16 G + 2 i + h
  // reads token 16 G + 8 j + i, chunk (2 s + h) ^ 2 (G & 1); output lane l
  // then holds position 16 s + l, tokens 16 G + 8 j .. + 7.
  auto requant4 = [&](int rb, int tt, auto actc) {
    constexpr bool ACT = decltype(actc)::value != 0;
    const float osc = a.out_scale;
    const v4f sv = scale_vec(rb);
    uint32_t bb[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float f = i8_pre<ACT>(acc[rb][tt][v], sv[v], osc);
      f = __builtin_amdgcn_fmed3f(f, -128.0f, 127.0f);
      bb[v] = __builtin_bit_cast(uint32_t, f + 12582912.0f);
    }
    return (int)(__builtin_amdgcn_perm(bb[1], bb[0], 0x0c0c0400u) | __builtin_amdgcn_perm(bb[3], bb[2], 0x04000c0cu));
  };
  auto epilogue_i8 = [&](int r0, int t0, auto actc) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy), 0x00020000);
    const int oob = (int)(g.R * a.ldy);
    const int rw0 = r0 + 16 * RB * wr, tw0 = t0 + 16 * TN * wt;
    int wb = 32 * li + 8 * lg;
    int rbs = (32 * (16 * lg + (li >> 1))) | (8 * ((li & 1) ^ (2 * (lg & 1))));
    asm volatile("" : "+v"(wb), "+v"(rbs));
    const int orow = 16 * ((li >> 2) & 1) + 4 * (li >> 3) + (li & 3);   // + 8 s
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int tt = 4 * h + u;
        *reinterpret_cast<v2i*>(os + ((512 * u + wb) ^ (16 * (u & 1)))) = v2i{requant4(0, tt, actc), requant4(1, tt, actc)};
      }
      // staging writes complete before the transpose reads
      __builtin_amdgcn_s_waitcnt(waitcnt(63, 0));
      // every lane stores; pieces past T go past the buffer's end (dropped)
      const int tok = tw0 + 64 * h + 16 * lg;
      const bool tok_ok = tok < a.T;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const v2i x0 = lds_tr8(os + (rbs ^ (16 * s)));
        const v2i x1 = lds_tr8(os + (rbs ^ (16 * s)) + 256);
        const int off = tok_ok ? (rw0 + orow + 8 * s) * (int)a.ldy + tok : oob;
        __builtin_amdgcn_raw_buffer_store_b128(v4i{x0[0], x0[1], x1[0], x1[1]}, ry, off, 0, kStreamStore);
      }
    }
  };
  auto store_i32 = [&](int r0, int t0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy * 4), 0x00020000);
    const int rw = r0 + 16 * RB * wr + 4 * lg;
    const int oob = (int)(g.R * a.ldy * 4);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) {
        const int t = t0 + 16 * TN * wt + 16 * tt + li;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          __builtin_amdgcn_raw_buffer_store_b32(acc[rb][tt][v], ry,
                                                t < a.T ? 4 * ((rw + 16 * rb + v) * (int)a.ldy + t) : oob, 0,
                                                kStreamStore);
      }
  };

  // ---- prologue: groups 0 .. NST - 2 into stages 0 .. NST - 2, then the
  // first row block's weights
  auto prologue_from = [&](auto self, auto mc) -> void {
    constexpr int M = decltype(mc)::value;
    issue_part(mc, ic<0>());
    issue_part(mc, ic<1>());
    if constexpr (M + 2 < NST) self(self, ic<M + 1>());
  };
  prologue_from(prologue_from, ic<0>());
  int crb, ct0;
  tile_of(0, crb, ct0);
  load_weights(crb);
  init_acc();

  for (int k = 0; k < nmine; ++k) {
    steps_from(steps_from, ic<0>());
    if constexpr (OUT_I8) {
      if (a.act)
        epilogue_i8(crb * BM, ct0, ic<1>());
      else
        epilogue_i8(crb * BM, ct0, ic<0>());
    } else {
      store_i32(crb * BM, ct0);
    }
    if (k + 1 < nmine) {
      const int prb = crb;
      tile_of(k + 1, crb, ct0);
      if (crb != prb) load_weights(crb);
      init_acc();
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
#endif
}

int cu_count(int device) {
  static int cache[64];
  if (device < 0 || device >= 64) return 256;
  if (!cache[device]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
      cus = 256;
    cache[device] = cus;
  }
  return cache[device];
}

template <int NKB>
hipError_t launch_nkb(const SpmmArgs& a, hipStream_t s) {
  const int mtiles = (int)((a.g.R + BM - 1) / BM);
  const int ntiles = (int)((a.T + BN - 1) / BN);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int nwg_xcd = cu_count(dev) / 8;                // one eight-wave workgroup per CU
  const int tiles_xcd = mtiles * ((ntiles + 7) / 8);
  if (nwg_xcd > tiles_xcd) nwg_xcd = tiles_xcd;
  if (nwg_xcd < 1) nwg_xcd = 1;
  const dim3 grid(8 * nwg_xcd), block(NW * 64);
  if (a.ydt == NM_I8)
    hipLaunchKernelGGL((smfmac_i8s_kernel<NKB, true>), grid, block, 0, s, a, mtiles, ntiles);
  else
    hipLaunchKernelGGL((smfmac_i8s_kernel<NKB, false>), grid, block, 0, s, a, mtiles, ntiles);
  return hipGetLastError();
}

}  // namespace

bool smfmac_i8s_supported(int64_t nKB) { return nKB >= 2 && nKB <= 8; }

hipError_t launch_spmm_smfmac_i8s(const SpmmArgs& a, hipStream_t s) {
  switch ((int)a.g.nKB) {
    case 2: return launch_nkb<2>(a, s);
    case 3: return launch_nkb<3>(a, s);
    case 4: return launch_nkb<4>(a, s);
    case 5: return launch_nkb<5>(a, s);
    case 6: return launch_nkb<6>(a, s);
    case 7: return launch_nkb<7>(a, s);
    case 8: return launch_nkb<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nm
