// Persistent N:M sparse x dense product for every N:M the sparse matrix
// instructions do not take directly (1:4, 3:4, 1:8, 2:8, 4:8, N = M), int8
// and fp16 / bf16, on the gfx950 dense matrix cores.
//
// This is the pages' micro-dense execution ("Realizable N:M Sparse
// Transformer Inference via Search-Kernel Co-Design", Sec. 4.2): the kept
// values of each window are placed at their positions inside a dense
// fragment so the matrix core sees only regular dense operands, and the
// irregularity stays in load and decode.  Here the decode is done in
// registers, per lane, with compile-time N and M: each kept value's position
// (log2(M) bits of the packed row's meta) becomes a shift inside its group's
// 32- or 64-bit slice of the fragment.
//
// The k-to-lane assignment of the dense MFMA is free as long as both
// operands use the same one.  Lane group g takes, over the two MFMA steps of
// a packed block, the dense run [LR g, LR (g + 1)) (LR = 32 int8 / 16 fp16
// elements): its kept values are one contiguous run of the packed row and
// its positions one contiguous run of meta bits, so a lane loads its whole
// share of a row block with one or two loads.  The B fragments (X) follow
// the same assignment.
//
// Workgroups of eight waves (one per CU, two waves per SIMD), each wave 32
// rows x 128 tokens, persistent over a per-XCD tile list; X in three LDS
// stages by direct-to-LDS loads; A in three register sets; exact vmcnt
// counts and one barrier per block, as in the 2:4 kernels.  Epilogues: int8
// bias + requant, int32, fp16 / bf16 (LDS transpose and 16-byte row pieces),
// fp32 (direct).
#pragma once
#include "nm_common.hpp"
#include "nm_expand.hpp"

namespace nm {

namespace {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int RB = 2;              // row blocks (16 rows) per wave
constexpr int TN = 8;              // token tiles (16 tokens) per wave
constexpr int NW = 8;              // waves per workgroup, stacked over rows
constexpr int BM = NW * RB * 16;   // 256 rows per tile
constexpr int BN = TN * 16;        // 128 tokens per tile
constexpr int STAGE = 16384;       // bytes per X stage (128 B of dense k x 128 tokens)
constexpr int DPW = STAGE / 1024 / NW;

template <int OUT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (OUT == NM_F16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2h));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2bf));
}

template <int WT, int NN, int MM, int OUT>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
expand_kernel(SpmmArgs a, int mtiles, int ntiles, int nwg_xcd, int gm) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr bool I8 = WT == NM_I8;
  typedef Run<WT, NN, MM> RG;
  constexpr int EB = RG::EB, VB = RG::VB, VD = RG::VD, W = RG::W, C_B = RG::C_B, MRB = RG::MRB;
  constexpr int NVL = (VB + 15) / 16;             // value loads per row block
  constexpr int LA = NVL + (W ? 1 : 0);           // A loads per row block (values, positions)
  constexpr bool OUT16 = OUT == NM_F16 || OUT == NM_BF16;
  typedef typename std::conditional<I8, v4i, v4f>::type Acc;

  __shared__ __attribute__((aligned(1024))) uint8_t xs0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs2[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ostage[(OUT == NM_I8 || OUT16) ? NW * 2048 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t bsbuf[NW * 4 * 512];

  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int nKB = (int)g.nKB;
  const int ldx = (int)a.ldx;
  const int nRB = (int)g.nRB;

  // work items: (tile, K slice); the tiles of one slice are contiguous, in
  // groups of gm row tiles (row tile fastest inside a group, then the next
  // token tile; tile_group_rows), so the workgroups an XCD runs together
  // share both operands' blocks through its L2
  const int kbs = a.kbs;                     // column blocks per work item
  const int ntile = mtiles * ntiles;
  const int ntot = ntile * a.ksplit;
  const int per_xcd = (ntot + 7) / 8;
  const int xcd = blockIdx.x % 8, jw = blockIdx.x / 8;
  const int lo = xcd * per_xcd;
  const int hi = min(lo + per_xcd, ntot);
  if (lo + jw >= hi) return;
  const int nmine = (hi - lo - jw + nwg_xcd - 1) / nwg_xcd;
  const int total = nmine * kbs;
  auto tile_of = [&](int k, int& r0, int& t0, int& ks) {
    const int L = lo + jw + k * nwg_xcd;
    ks = L / ntile;
    const int Lt = L - ks * ntile;
    const int grp = Lt / (gm * ntiles);
    const int in = Lt - grp * gm * ntiles;
    const int rows = min(gm, mtiles - grp * gm);
    const int nt = in / rows;
    r0 = (grp * gm + in - nt * rows) * BM;
    t0 = nt * BN;
  };

  const v4i rx = make_rsrc(a.X, (int)(g.K * a.ldx * EB));
  const __amdgpu_buffer_rsrc_t rvv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values), 0, (int)g.values_bytes(), 0x00020000);
  const __amdgpu_buffer_rsrc_t rmm = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.meta), 0, W ? (int)g.meta_bytes() : 0, 0x00020000);
  const v4i rbias = make_rsrc(a.bias, a.bias ? (int)(g.R * 4) : 0);
  const v4i rscale = make_rsrc(a.scale, a.scale ? (int)(g.R * 4) : 0);

  // ---- X stage layouts (chunk positions swizzled so the transpose reads of
  // the two lane groups served together hit disjoint banks).
  // int8: 128 rows (k) x 128 B; 16-byte chunk c of row r at c ^ f(r),
  //       f(r) = (r & 7) ^ (((r >> 4) ^ (r >> 5)) & 1); load d: rows 8 d ..
  //       + 7, lane l -> row 8 d + l / 8, position l % 8.
  // 16-bit: 64 rows x 256 B; 32-byte chunk c of row r at c ^ h(r),
  //       h(r) = (r & 7) ^ 4 ((r >> 4) & 1); load d: rows 4 d .. + 3, lane l
  //       -> row 4 d + l / 16, position (l % 16) / 2, half l % 2.
  auto xoff = [&](int j) {
    const int d = wave * DPW + j;
    if constexpr (I8) {
      const int row = 8 * d + (lane >> 3);
      const int c = (lane & 7) ^ (row & 7) ^ (((row >> 4) ^ (row >> 5)) & 1);
      return row * ldx + 16 * c;
    } else {
      const int row = 4 * d + (lane >> 4);
      const int c = ((lane & 15) >> 1) ^ (row & 7) ^ (((row >> 4) & 1) << 2);
      return row * ldx * 2 + 32 * c + 16 * (lane & 1);
    }
  };
  auto xstage = [&](auto st) -> uint8_t* {
    constexpr int S = decltype(st)::value;
    return S == 0 ? xs0 : (S == 1 ? xs1 : xs2);
  };

  // ---- A: lane (i, g) of row block rb loads its run (VB bytes at row i,
  // offset g VB of the block) and the 64-bit meta window holding its
  // positions (one dword when a row's meta is one dword)
  const int voff_v = li * C_B + lg * VB;
  int mdw, mshift;
  RG::meta_window(lg, mdw, mshift);
  const int voff_m = li * MRB + 4 * mdw;
  uint32_t av[3][RB][VD];
  uint64_t am[3][RB];

  uint8_t* const bsw = bsbuf + wave * 2048;
  auto bias_i = [&](int k, int rb) {
    return *reinterpret_cast<const v4i*>(bsw + 512 * (k & 3) + 4 * (16 * rb + 4 * lg));
  };
  auto bias_f = [&](int k, int rb) {
    return *reinterpret_cast<const v4f*>(bsw + 512 * (k & 3) + 4 * (16 * rb + 4 * lg));
  };
  auto scale_vec = [&](int k, int rb) {
    return *reinterpret_cast<const v4f*>(bsw + 512 * (k & 3) + 256 + 4 * (16 * rb + 4 * lg));
  };

  int ln = 0, lk = 0, lkb = 0, lr0 = 0, lt0 = 0, lks = 0;
  tile_of(0, lr0, lt0, lks);
  lks *= kbs;                                // first column block of the slice
  int g_live = 0, g_rb0 = 0, g_soff = 0;
  // group parts: 0, 1: A of row block 0, 1; 2, 3: X halves; 4: bias / scale
  // on a tile's first block and the cursor
  // No load has all its lanes outside its operand (such a load returns at
  // once, ahead of older loads; see nm_zero_page): row blocks past R and
  // groups past the end read valid blocks (data nobody uses), X rows
  // entirely past K and absent bias / scale rows read the zero page; rows
  // and tokens partly outside are in the vector offset, which the range
  // check covers.
  const v4i rz = zero_rsrc();
  int g_krem = 0;
  auto load_part = [&](auto st, auto part) {
    constexpr int S = decltype(st)::value;
    constexpr int P = decltype(part)::value;
    if constexpr (P == 0) {
      g_live = __builtin_amdgcn_readfirstlane(ln < total ? 1 : 0);
      g_rb0 = __builtin_amdgcn_readfirstlane((lr0 >> 4) + RB * wave);
      g_soff = __builtin_amdgcn_readfirstlane(((lks + lkb) * (128 / EB) * ldx + lt0) * EB);
      g_krem = __builtin_amdgcn_readfirstlane((int)g.K - (lks + lkb) * (128 / EB));
    }
    if constexpr (P < RB) {
      const auto rv = rvv;
      const auto rm = rmm;
      const int blk = __builtin_amdgcn_readfirstlane(min(g_rb0 + P, nRB - 1) * nKB + lks + lkb);
      const int vo = voff_v + blk * C_B * 16;
#pragma unroll
      for (int c = 0; c < NVL; ++c) {
        const int rem = VB - 16 * c;
        if (rem >= 16) {
          const v4i x = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rv, vo + 16 * c, 0, 0));
          av[S][P][4 * c] = x[0]; av[S][P][4 * c + 1] = x[1];
          av[S][P][4 * c + 2] = x[2]; av[S][P][4 * c + 3] = x[3];
        } else if (rem == 12) {
          const auto x = __builtin_amdgcn_raw_buffer_load_b96(rv, vo + 16 * c, 0, 0);
          av[S][P][4 * c] = x[0]; av[S][P][4 * c + 1] = x[1]; av[S][P][4 * c + 2] = x[2];
        } else if (rem == 8) {
          const auto x = __builtin_amdgcn_raw_buffer_load_b64(rv, vo + 16 * c, 0, 0);
          av[S][P][4 * c] = x[0]; av[S][P][4 * c + 1] = x[1];
        } else {
          av[S][P][4 * c] = __builtin_amdgcn_raw_buffer_load_b32(rv, vo + 16 * c, 0, 0);
        }
      }
      if constexpr (MRB >= 8) {
        const auto m = __builtin_amdgcn_raw_buffer_load_b64(rm, voff_m + blk * MRB * 16, 0, 0);
        am[S][P] = ((uint64_t)m[1] << 32) | m[0];
      } else if constexpr (MRB == 4) {
        am[S][P] = __builtin_amdgcn_raw_buffer_load_b32(rm, voff_m + blk * MRB * 16, 0, 0);
      }
    } else if constexpr (P == RB || P == RB + 1) {
      uint8_t* sp = xstage(st);
      constexpr int H = DPW / 2, J0 = (P - RB) * H;
#pragma unroll
      for (int j = J0; j < J0 + H; ++j) {
        const int d = wave * DPW + j;
        // load d fills rows (8 or 4) d .. of the stage
        if ((I8 ? 8 : 4) * d < g_krem)
          lds_dma16(rx, lds_addr(sp + d * 1024), xoff(j) + g_soff, 0);
        else
          lds_dma16(rz, lds_addr(sp + d * 1024), 16 * lane, 0);
      }
    } else {
      if (g_live && lkb == 0) {
        uint8_t* bs = bsw + 512 * (lk & 3);
        const int row0 = __builtin_amdgcn_readfirstlane(lr0 + 32 * wave);
        const int boff = 4 * (row0 + lane);
        if (a.bias && row0 < (int)g.R)
          lds_dma4(rbias, lds_addr(bs), boff, 0);
        else
          lds_dma4(rz, lds_addr(bs), 4 * lane, 0);
        if (a.scale && row0 < (int)g.R)
          lds_dma4(rscale, lds_addr(bs + 256), boff, 0);
        else
          lds_dma4(rz, lds_addr(bs + 256), 4 * lane, 0);
      }
      ++ln;
      if (g_live && ++lkb == kbs) {
        lkb = 0;
        if (++lk < nmine) {
          tile_of(lk, lr0, lt0, lks);
          lks *= kbs;
        }
      }
    }
  };
  constexpr int NPART = RB + 3;
  static_assert(DPW % 2 == 0 && NPART < TN, "two X halves, one part per token tile");
  auto load_group = [&](auto st) {
    load_part(st, ic<0>()); load_part(st, ic<1>()); load_part(st, ic<2>()); load_part(st, ic<3>());
    load_part(st, ic<4>());
  };
  static_assert(RB == 2 && NPART == 5, "load parts are spelled out for two row blocks");
  auto group_size_extra = [&](int m) { return (m < total && m % kbs == 0) ? 2 : 0; };

  // ---- B transpose reads for token tile tt: lane (j, g) gets, for step s,
  // the dense k of its group's run: int8 rows 32 g + 16 s .. + 15 (tr8 reads
  // of rows 32 g + kq + i / 2, kq = 0, 8, 16, 24), fp16 rows 16 g + 8 s ..
  // + 7 (tr16 reads of rows 16 g + kq + e, kq = 0, 4, 8, 12).
  int xa, xb;
  if constexpr (I8) {
    const int base = 128 * (32 * lg + (li >> 1)) + 8 * (li & 1);
    xa = base | (16 * ((li >> 1) ^ (lg & 1)));
    xb = base | (16 * ((li >> 1) ^ (lg & 1) ^ 1));
  } else {
    const int e_s = li >> 2, q_s = li & 3;
    xa = (256 * (16 * lg + e_s) + 8 * q_s) | (32 * (e_s ^ (4 * (lg & 1))));
    xb = (256 * (16 * lg + 4 + e_s) + 8 * q_s) | (32 * (e_s ^ 4 ^ (4 * (lg & 1))));
  }
  auto bfrag = [&](const uint8_t* sb, int tt) -> v8i {
    if constexpr (I8) {
      int oa = xa ^ (16 * tt), ob = xb ^ (16 * tt);
      asm volatile("" : "+v"(oa), "+v"(ob));
      const v2i p0 = lds_tr8(sb + oa);
      const v2i p1 = lds_tr8(sb + oa + 8 * 128);
      const v2i p2 = lds_tr8(sb + ob + 16 * 128);
      const v2i p3 = lds_tr8(sb + ob + 24 * 128);
      return v8i{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    } else {
      int oa = xa ^ (32 * tt), ob = xb ^ (32 * tt);
      asm volatile("" : "+v"(oa), "+v"(ob));
      const v2i p0 = lds_tr16(sb + oa);
      const v2i p1 = lds_tr16(sb + ob);
      const v2i p2 = lds_tr16(sb + oa + 8 * 256);
      const v2i p3 = lds_tr16(sb + ob + 8 * 256);
      return v8i{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
  };

  Acc acc[RB][TN];
  auto compute = [&](auto st, auto ast, auto nxt) {
    constexpr int AS = decltype(ast)::value;
    const uint8_t* sb = xstage(st);
    // dense fragments of this block: both steps of both row blocks
    v4i da[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const uint64_t mb = W ? (am[AS][rb] >> mshift) : 0;
      da[rb][0] = expand_step<WT, NN, MM, 0>(av[AS][rb], mb);
      da[rb][1] = expand_step<WT, NN, MM, 1>(av[AS][rb], mb);
    }
    v8i bf[2];
    bf[0] = bfrag(sb, 0);
    bf[1] = bfrag(sb, 1);
    auto tile = [&](auto ttc) {
      constexpr int tt = decltype(ttc)::value;
      if constexpr (tt >= 1 && tt + 1 < TN) bf[(tt + 1) % 2] = bfrag(sb, tt + 1);
      const v8i b = bf[tt % 2];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        acc[rb][tt] = mfma_dense<WT>(da[rb][0], v4i{b[0], b[1], b[2], b[3]}, acc[rb][tt]);
        acc[rb][tt] = mfma_dense<WT>(da[rb][1], v4i{b[4], b[5], b[6], b[7]}, acc[rb][tt]);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (tt < NPART) load_part(nxt, ic<tt>());
      __builtin_amdgcn_sched_barrier(0);
    };
    tile(ic<0>()); tile(ic<1>()); tile(ic<2>()); tile(ic<3>());
    tile(ic<4>()); tile(ic<5>()); tile(ic<6>()); tile(ic<7>());
  };
  auto init_acc = [&](int k) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      Acc b;
      if constexpr (I8) b = bias_i(k, rb); else b = bias_f(k, rb);
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) acc[rb][tt] = b;
    }
  };

  // ---- epilogues.  Staging rows: position p = 8 g + 4 rb + v of a token
  // holds wave row 16 rb + 4 g + v; a lane's 8 rows of one token are one
  // chunk (8 bytes int8, 16 bytes 16-bit) at chunk position g ^ f(t).
  uint8_t* const os = ostage + ((OUT == NM_I8 || OUT16) ? wave * 2048 : 0);
  auto epilogue_i8 = [&](int k, int r0, int t0, auto actc) __attribute__((always_inline)) {
    constexpr bool ACT = decltype(actc)::value != 0;
    const float osc = a.out_scale;
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy), 0x00020000);
    const int oob = (int)(g.R * a.ldy);
    // token t (0..63 of the half) is a 32-byte row, f(t) = ((t >> 4) & 1) << 1;
    // reads: lane 16 G + 2 i + h reads token 16 G + 8 j + i, chunk (2 s + h)
    // ^ 2 (G & 1); output lane l then holds position 16 s + l, tokens 16 G +
    // 8 j .. + 7
    int wb = 32 * li + 8 * lg;
    int rbs = (32 * (16 * lg + (li >> 1))) | (8 * (((li & 1)) ^ (2 * (lg & 1))));
    asm volatile("" : "+v"(wb), "+v"(rbs));
    const int orow = 16 * ((li >> 2) & 1) + 4 * (li >> 3) + (li & 3);   // + 8 s
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int tt = 4 * h + u;
        int d[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const v4f sv = scale_vec(k, rb);
          float f[4];
#pragma unroll
          for (int v = 0; v < 4; ++v)
            f[v] = __builtin_amdgcn_fmed3f(i8_pre<ACT>(acc[rb][tt][v], sv[v], osc), -128.0f, 127.0f);
          d[rb] = (int)pack_rne_i8x4(f[0], f[1], f[2], f[3]);
        }
        // token 16 u + li: f = 2 (u & 1)
        *reinterpret_cast<v2i*>(os + ((512 * u + wb) ^ (16 * (u & 1)))) = v2i{d[0], d[1]};
      }
      // staging writes complete before the transpose reads
      __builtin_amdgcn_s_waitcnt(waitcnt(63, 0));
      const int tok = t0 + 64 * h + 16 * lg;
      const bool tok_ok = tok < a.T;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const v2i x0 = lds_tr8(os + (rbs ^ (16 * s)));
        const v2i x1 = lds_tr8(os + (rbs ^ (16 * s)) + 256);
        const int row = r0 + 32 * wave + orow + 8 * s;
        const int off = tok_ok ? row * (int)a.ldy + tok : oob;
        __builtin_amdgcn_raw_buffer_store_b128(v4i{x0[0], x0[1], x1[0], x1[1]}, ry, off, 0, kStreamStore);
      }
    }
  };
  auto epilogue_h = [&](int r0, int t0, auto actc) __attribute__((always_inline)) {
    constexpr bool ACT = decltype(actc)::value != 0;
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy * 2), 0x00020000);
    const int oob = (int)(g.R * a.ldy * 2);
    // token t (0..31 of the quarter) is a 64-byte row, f(t) = ((t >> 3) & 1)
    // << 1 over 16-byte chunks; reads: lane 16 G + 4 e + q reads token 8 G +
    // 4 j + e, chunk (2 s + q / 2) ^ f, byte 8 (q % 2); output lane l then
    // holds position 16 s + l, tokens 8 G + 4 j .. + 3
    const int e_s = li >> 2, q_s = li & 3;
    int wb = (64 * li) | (16 * (lg ^ (((li >> 3) & 1) << 1)));
    int rbs = (64 * (8 * lg + e_s) + 8 * (q_s & 1)) | (16 * ((q_s >> 1) ^ ((lg & 1) << 1)));
    asm volatile("" : "+v"(wb), "+v"(rbs));
    const int orow = 16 * ((li >> 2) & 1) + 4 * (li >> 3) + (li & 3);   // + 8 s
#pragma unroll
    for (int u4 = 0; u4 < 4; ++u4) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int tt = 2 * u4 + w;
        const uint32_t d0 = pack2<OUT>(fp_act<ACT>(acc[0][tt][0]), fp_act<ACT>(acc[0][tt][1]));
        const uint32_t d1 = pack2<OUT>(fp_act<ACT>(acc[0][tt][2]), fp_act<ACT>(acc[0][tt][3]));
        const uint32_t d2 = pack2<OUT>(fp_act<ACT>(acc[1][tt][0]), fp_act<ACT>(acc[1][tt][1]));
        const uint32_t d3 = pack2<OUT>(fp_act<ACT>(acc[1][tt][2]), fp_act<ACT>(acc[1][tt][3]));
        *reinterpret_cast<v4i*>(os + wb + 1024 * w) = v4i{(int)d0, (int)d1, (int)d2, (int)d3};
      }
      const int tok = t0 + 32 * u4 + 8 * lg;
      const bool tok_ok = tok < a.T;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint8_t* rp = os + (rbs ^ (32 * s));
        const v2i x0 = lds_tr16(rp);
        const v2i x1 = lds_tr16(rp + 256);
        const int row = r0 + 32 * wave + orow + 8 * s;
        const int off = tok_ok ? (row * (int)a.ldy + tok) * 2 : oob;
        __builtin_amdgcn_raw_buffer_store_b128(v4i{x0[0], x0[1], x1[0], x1[1]}, ry, off, 0, kStreamStore);
      }
    }
  };
  // int32 / fp32 output, or slice ks's partial sums under a K split
  auto store_direct = [&](int r0, int t0, int ks, auto actc) __attribute__((always_inline)) {
    constexpr bool ACT = decltype(actc)::value != 0 && !I8;
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<int32_t*>(a.Y) + ks * a.ys, 0, (int)(g.R * a.ldy * 4), 0x00020000);
    const int rw = r0 + 32 * wave + 4 * lg;
    const int oob = (int)(g.R * a.ldy * 4);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) {
        const int t = t0 + 16 * tt + li;
        // whole-vector cast (a bit cast of one element of a vector lvalue
        // reads element 0)
        Acc x = acc[rb][tt];
        if constexpr (ACT) {
#pragma unroll
          for (int v = 0; v < 4; ++v) x[v] = gelu_f32(x[v]);
        }
        const v4i ai4 = __builtin_bit_cast(v4i, x);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          __builtin_amdgcn_raw_buffer_store_b32(ai4[v], ry,
                                                t < a.T ? 4 * ((rw + 16 * rb + v) * (int)a.ldy + t) : oob, 0, kStreamStore);
      }
  };

  int n = 0, ck = 0, ckb = 0, cr0, ct0, cks;
  tile_of(0, cr0, ct0, cks);
  // Wait until the stage of the oldest outstanding group (and a tile's bias
  // rows) has landed.  Only direct-to-LDS loads are counted: they complete
  // in issue order among themselves, but the register loads of a later
  // group (A fragments hitting in L2) may complete before them, so a count
  // that included those could pass with the stage still in flight.  Every
  // group holds at least DPW of them, so at most DPW outstanding means every
  // direct-to-LDS load before the newest group is in; the compiler's own
  // waits cover the A registers.  One unconditional count keeps the wait a
  // single instruction on every path through the unrolled steps.
  auto wait_for_group = [&](int extra_after) {
    (void)extra_after;
    __builtin_amdgcn_s_waitcnt(waitcnt(DPW, 15));
  };

  load_group(ic<0>());
  load_group(ic<1>());
  wait_for_group(group_size_extra(1));
  init_acc(0);

  auto step = [&](auto st) {
    constexpr int ST = decltype(st)::value;
    constexpr int NX = (ST + 2) % 3;
    wait_for_group(group_size_extra(n + 1));
    barrier_nofence();
    compute(st, ic<ST>(), ic<NX>());
    ++n;
    if (++ckb < kbs) return;
    ckb = 0;
    if constexpr (OUT == NM_I8) {
      if (a.act)
        epilogue_i8(ck, cr0, ct0, ic<1>());
      else
        epilogue_i8(ck, cr0, ct0, ic<0>());
    } else if constexpr (OUT16) {
      if (a.act)
        epilogue_h(cr0, ct0, ic<1>());
      else
        epilogue_h(cr0, ct0, ic<0>());
    } else {
      if (a.act)
        store_direct(cr0, ct0, cks, ic<1>());
      else
        store_direct(cr0, ct0, cks, ic<0>());
    }
    ++ck;
    if (ck < nmine) {
      tile_of(ck, cr0, ct0, cks);
      wait_for_group(group_size_extra(n + 1));
      init_acc(ck);
    }
  };
  const int trips = total / 3, rest = total - 3 * trips;
  for (int it = 0; it < trips; ++it) {
    step(ic<0>());
    step(ic<1>());
    step(ic<2>());
  }
  if (rest > 0) step(ic<0>());
  if (rest > 1) step(ic<1>());
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
#endif
}

template <int WT, int NN, int MM, int OUT>
hipError_t launch_one(const SpmmArgs& a, hipStream_t s) {
  const int mtiles = (int)((a.g.R + BM - 1) / BM);
  const int ntiles = (int)((a.T + BN - 1) / BN);
  const int ntot = mtiles * ntiles * a.ksplit;
  const int per_xcd = (ntot + 7) / 8;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int nwg_xcd = cu_count(dev) / 8;                // one eight-wave workgroup per CU
  if (nwg_xcd > per_xcd) nwg_xcd = per_xcd;
  if (nwg_xcd < 1) nwg_xcd = 1;
  // operand bytes one row tile / one token tile brings per 128 columns
  const double eb = a.g.eb;
  const double wk = 256.0 * 128 * NN / MM * (eb + (NN == MM ? 0.0 : a.g.w / 8.0)), xk = 128.0 * BN * eb;
  const int gm = tile_group_rows(mtiles, ntiles, nwg_xcd, wk, xk, (double)(a.g.values_bytes() + a.g.meta_bytes()));
  hipLaunchKernelGGL((expand_kernel<WT, NN, MM, OUT>), dim3(8 * nwg_xcd), dim3(NW * 64), 0, s, a, mtiles, ntiles,
                     nwg_xcd, gm);
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

// one instantiation per weight dtype, each in its own translation unit
// (nm_spmm_expand_{i8,f16,bf16}.hip) so that they compile in parallel
hipError_t launch_spmm_expand_i8(const SpmmArgs& a, hipStream_t s);
hipError_t launch_spmm_expand_f16(const SpmmArgs& a, hipStream_t s);
hipError_t launch_spmm_expand_bf16(const SpmmArgs& a, hipStream_t s);

}  // namespace nm
