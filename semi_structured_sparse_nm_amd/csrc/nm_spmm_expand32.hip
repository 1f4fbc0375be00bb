// Persistent N:M sparse x dense product for every N:M the sparse matrix
// instructions do not take directly (1:4, 3:4, 1:8, 2:8, 4:8, N = M), int8
// and fp16 / bf16, on the gfx950 dense matrix cores with 32 x 32 fragments
// (v_mfma_i32_32x32x32_i8, v_mfma_f32_32x32x16_{f16,bf16}).
//
// This is the pages' micro-dense execution ("Realizable N:M Sparse
// Transformer Inference via Search-Kernel Co-Design", Sec. 4.2): the kept
// values of each window are placed at their positions inside dense
// fragments, so the matrix cores see only regular dense operands and the
// irregularity stays in load and decode.  The decode is done in registers,
// per lane (nm_expand.hpp): each kept value is shifted to its in-window
// position.  On gfx950 the 32 x 32 dense shapes deliver about 1.6 times the
// multiply-accumulates per cycle of the 16 x 16 ones (measured: 4.1 against
// 2.5 POPS int8, 2.1 against 1.2 PFLOPS fp16).
//
// k order: over the four MFMA steps of a packed block (128 int8 / 64 16-bit
// columns) lane group h (lanes 32 h ..) takes the dense columns
// [2 LR h, 2 LR (h + 1)), i.e. the packed runs 2 h and 2 h + 1 (LR = 32 int8
// / 16 fp16 columns a run): one contiguous piece of the packed row and two
// runs of meta bits.  Step s uses run 2 h + s / 2, half s % 2.  The B
// fragments (X) follow the same order.  A lane's 32 fragment rows span two
// packed 16-row blocks.
//
// Workgroups of eight waves (one per CU, two waves per SIMD), each wave 32
// rows x 128 tokens (4 accumulator fragments of 32 x 32), persistent over a
// per-XCD tile list; X in three LDS stages by direct-to-LDS loads; A in three
// register sets; exact vmcnt counts over loads only and one barrier per
// block.  Epilogues: int8 bias + requant, int32, fp16 / bf16 (LDS transpose,
// 16-byte row pieces), fp32 (direct); output streamed past L2.
#include "nm_common.hpp"
#include "nm_expand.hpp"

namespace nm {

namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

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
__device__ __forceinline__ v2i lds_tr16(const uint8_t* p) {
  return __builtin_bit_cast(
      v2i, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p)));
}

constexpr int NW = 8;              // waves per workgroup, stacked over rows
constexpr int BM = NW * 32;        // 256 rows per tile
constexpr int TB = 4;              // 32-token blocks per wave
constexpr int BN = TB * 32;        // 128 tokens per tile
constexpr int STAGE = 16384;       // bytes per X stage (128 B of dense k x 128 tokens)
constexpr int DPW = STAGE / 1024 / NW;

template <int WT, typename Acc>
__device__ __forceinline__ Acc mfma32(v4i a, v4i b, Acc c) {
  if constexpr (WT == NM_I8)
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  else if constexpr (WT == NM_F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0,
                                                   0, 0);
}

template <int OUT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (OUT == NM_F16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2h));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2bf));
}

template <int WT, int NN, int MM, int OUT>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
expand32_kernel(SpmmArgs a, int mtiles, int ntiles, int nwg_xcd) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr bool I8 = WT == NM_I8;
  typedef Run<WT, NN, MM> RG;
  constexpr int EB = RG::EB, VB = RG::VB, VD = RG::VD, W = RG::W, C_B = RG::C_B, MRB = RG::MRB;
  constexpr int AB = 2 * VB;                      // a lane's packed bytes per block (two runs)
  constexpr int NVL = (AB + 15) / 16;             // value loads per block
  constexpr int NML = W ? 2 : 0;                  // meta loads per block (one window per run)
  constexpr int NL = NVL + NML + DPW;             // loads per group (+2 on a tile's first block)
  constexpr bool OUT16 = OUT == NM_F16 || OUT == NM_BF16;
  typedef typename std::conditional<I8, v16i, v16f>::type Acc;

  __shared__ __attribute__((aligned(1024))) uint8_t xs0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs2[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ostage[(OUT == NM_I8 || OUT16) ? NW * 2048 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t bsbuf[NW * 4 * 512];

  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int j32 = lane & 31, h = lane >> 5;       // fragment row / column, lane group
  const int nKB = (int)g.nKB;
  const int ldx = (int)a.ldx;

  const int ntot = mtiles * ntiles;
  const int per_xcd = (ntot + 7) / 8;
  const int xcd = blockIdx.x % 8, jw = blockIdx.x / 8;
  const int lo = xcd * per_xcd;
  const int hi = min(lo + per_xcd, ntot);
  if (lo + jw >= hi) return;
  const int nmine = (hi - lo - jw + nwg_xcd - 1) / nwg_xcd;
  const int total = nmine * nKB;
  auto tile_of = [&](int k, int& r0, int& t0) {
    const int L = lo + jw + k * nwg_xcd;
    const int nt = L / mtiles;
    r0 = (L - nt * mtiles) * BM;
    t0 = nt * BN;
  };

  const v4i rx = make_rsrc(a.X, (int)(g.K * a.ldx * EB));
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values), 0, (int)g.values_bytes(), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.meta), 0, W ? (int)g.meta_bytes() : 0, 0x00020000);
  const v4i rbias = make_rsrc(a.bias, a.bias ? (int)(g.R * 4) : 0);
  const v4i rscale = make_rsrc(a.scale, a.scale ? (int)(g.R * 4) : 0);

  // ---- X stages: int8 128 rows (k) x 128 B, 16-byte chunk c of row r at
  // c ^ (r & 7); 16-bit 64 rows x 256 B, 32-byte chunk c of row r at
  // c ^ (r & 7).  Load d: int8 rows 8 d .. + 7 (lane l -> row 8 d + l / 8,
  // position l % 8); 16-bit rows 4 d .. + 3 (lane l -> row 4 d + l / 16,
  // position (l % 16) / 2, half l % 2).
  auto xoff = [&](int jj) {
    const int d = wave * DPW + jj;
    if constexpr (I8) {
      const int row = 8 * d + (lane >> 3);
      return row * ldx + 16 * ((lane & 7) ^ (row & 7));
    } else {
      const int row = 4 * d + (lane >> 4);
      return row * ldx * 2 + 32 * (((lane & 15) >> 1) ^ (row & 7)) + 16 * (lane & 1);
    }
  };
  auto xstage = [&](auto st) -> uint8_t* {
    constexpr int S = decltype(st)::value;
    return S == 0 ? xs0 : (S == 1 ? xs1 : xs2);
  };

  // ---- A: lane (i, h) holds fragment row i = the wave's row i: packed row
  // i % 16 of the wave's row block i / 16; its runs 2 h, 2 h + 1 are AB
  // contiguous bytes at offset 2 h VB of that packed row, its two meta
  // windows per Run::meta_window.  Offsets: the lane part here, the block
  // part (row block, column block) added per group.
  const int rbl = j32 >> 4;                       // the lane's row block within the wave
  const int lane_v = (j32 & 15) * C_B + 2 * h * VB + rbl * nKB * (int)g.vblk;
  int mdw0, msh0, mdw1, msh1;
  RG::meta_window(2 * h, mdw0, msh0);
  RG::meta_window(2 * h + 1, mdw1, msh1);
  const int lane_m0 = (j32 & 15) * MRB + 4 * mdw0 + rbl * nKB * (int)g.mblk;
  const int lane_m1 = (j32 & 15) * MRB + 4 * mdw1 + rbl * nKB * (int)g.mblk;
  constexpr int ADW = (AB + 3) / 4;
  uint32_t av[3][ADW];
  uint64_t am[3][2];

  // bias / scale of the wave's rows (64 from its first; rows past R read as
  // zero), one LDS slot per tile index mod 4
  uint8_t* const bsw = bsbuf + wave * 2048;

  int ln = 0, lk = 0, lkb = 0, lr0 = 0, lt0 = 0;
  tile_of(0, lr0, lt0);
  int g_live = 0, g_vb = 0, g_mb = 0, g_soff = 0;
  // group parts: 0: values; 1: meta; 2, 3: X halves; 4: bias / scale on a
  // tile's first block and the cursor.  Every offset that can leave its
  // buffer is in the vector offset (the range check covers it).
  auto load_part = [&](auto st, auto part) {
    constexpr int S = decltype(st)::value;
    constexpr int P = decltype(part)::value;
    if constexpr (P == 0) {
      g_live = __builtin_amdgcn_readfirstlane(ln < total ? 1 : 0);
      const int rb0 = (lr0 >> 4) + 2 * wave;
      const int blk = g_live ? rb0 * nKB + lkb : (int)(g.nRB * g.nKB);
      g_vb = __builtin_amdgcn_readfirstlane(blk * (int)g.vblk);
      g_mb = __builtin_amdgcn_readfirstlane(blk * (int)g.mblk);
      g_soff = __builtin_amdgcn_readfirstlane(g_live ? (lkb * (128 / EB) * ldx + lt0) * EB
                                                     : (int)(g.K * a.ldx * EB));
      const int vo = lane_v + g_vb;
#pragma unroll
      for (int c = 0; c < NVL; ++c) {
        const int rem = AB - 16 * c;
        if (rem >= 16) {
          const v4i x = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rv, vo + 16 * c, 0, 0));
          av[S][4 * c] = x[0]; av[S][4 * c + 1] = x[1]; av[S][4 * c + 2] = x[2]; av[S][4 * c + 3] = x[3];
        } else if (rem == 8) {
          const auto x = __builtin_amdgcn_raw_buffer_load_b64(rv, vo + 16 * c, 0, 0);
          av[S][4 * c] = x[0]; av[S][4 * c + 1] = x[1];
        } else {
          static_assert(AB % 8 == 0, "a lane's two runs are whole 8-byte pieces");
        }
      }
    } else if constexpr (P == 1) {
      if constexpr (MRB >= 8) {
        const auto m0 = __builtin_amdgcn_raw_buffer_load_b64(rm, lane_m0 + g_mb, 0, 0);
        const auto m1 = __builtin_amdgcn_raw_buffer_load_b64(rm, lane_m1 + g_mb, 0, 0);
        am[S][0] = ((uint64_t)m0[1] << 32) | m0[0];
        am[S][1] = ((uint64_t)m1[1] << 32) | m1[0];
      } else if constexpr (MRB == 4) {
        am[S][0] = __builtin_amdgcn_raw_buffer_load_b32(rm, lane_m0 + g_mb, 0, 0);
        am[S][1] = __builtin_amdgcn_raw_buffer_load_b32(rm, lane_m1 + g_mb, 0, 0);
      }
    } else if constexpr (P == 2 || P == 3) {
      uint8_t* sp = xstage(st);
      constexpr int J = P - 2;
      const int d = wave * DPW + J;
      lds_dma16(rx, lds_addr(sp + d * 1024), xoff(J) + g_soff, 0);
    } else {
      if (g_live && lkb == 0) {
        uint8_t* bs = bsw + 512 * (lk & 3);
        const int boff = 4 * (lr0 + 32 * wave + lane);
        lds_dma4(rbias, lds_addr(bs), boff, 0);
        lds_dma4(rscale, lds_addr(bs + 256), boff, 0);
      }
      ++ln;
      if (g_live && ++lkb == nKB) {
        lkb = 0;
        if (++lk < nmine) tile_of(lk, lr0, lt0);
      }
    }
  };
  static_assert(DPW == 2, "two X halves");
  auto load_group = [&](auto st) {
    load_part(st, ic<0>()); load_part(st, ic<1>()); load_part(st, ic<2>()); load_part(st, ic<3>());
    load_part(st, ic<4>());
  };
  auto group_size_extra = [&](int m) { return (m < total && m % nKB == 0) ? 2 : 0; };

  // ---- B fragments of step s, token block tb: two transpose reads of the
  // rows k0 .. k0 + 7 (int8: k0 = 64 h + 16 s + 8 q) or k0 .. k0 + 3 (16-bit:
  // k0 = 32 h + 8 s + 4 q), tokens 32 tb + 16 (G % 2) + .. (G = lane / 16)
  int xb0, xb1;
  if constexpr (I8) {
    const int i8r = li >> 1, hh = li & 1;
    xb0 = (128 * (64 * (lg >> 1) + i8r) + 8 * hh) | (16 * ((lg & 1) ^ i8r));
    xb1 = xb0;
  } else {
    const int e = li >> 2, qq = li & 3;
    xb0 = (256 * (32 * (lg >> 1) + e) + 8 * qq) | (32 * ((lg & 1) ^ e));
    xb1 = (256 * (32 * (lg >> 1) + 4 + e) + 8 * qq) | (32 * ((lg & 1) ^ (4 + e)));
  }
  auto bfrag = [&](const uint8_t* sb, int s, int tb) -> v4i {
    if constexpr (I8) {
      int o = xb0 ^ (32 * tb);
      asm volatile("" : "+v"(o));
      const v2i p0 = lds_tr8(sb + o + 128 * 16 * s);
      const v2i p1 = lds_tr8(sb + o + 128 * (16 * s + 8));
      return v4i{p0[0], p0[1], p1[0], p1[1]};
    } else {
      int o0 = xb0 ^ (64 * tb), o1 = xb1 ^ (64 * tb);
      asm volatile("" : "+v"(o0), "+v"(o1));
      const v2i p0 = lds_tr16(sb + o0 + 256 * 8 * s);
      const v2i p1 = lds_tr16(sb + o1 + 256 * 8 * s);
      return v4i{p0[0], p0[1], p1[0], p1[1]};
    }
  };

  Acc acc[TB];
  auto compute = [&](auto st, auto ast, auto nxt) {
    constexpr int AS = decltype(ast)::value;
    const uint8_t* sb = xstage(st);
    const uint64_t mb0 = W ? (am[AS][0] >> msh0) : 0;
    const uint64_t mb1 = W ? (am[AS][1] >> msh1) : 0;
    v4i bf[2][TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) bf[0][tb] = bfrag(sb, 0, tb);
    auto step = [&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if constexpr (s + 1 < 4) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) bf[(s + 1) % 2][tb] = bfrag(sb, s + 1, tb);
      }
      const v4i da = (s < 2) ? expand_step<WT, NN, MM, s % 2>(av[AS], mb0)
                             : expand_step<WT, NN, MM, s % 2>(av[AS] + VD, mb1);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) acc[tb] = mfma32<WT>(da, bf[s % 2][tb], acc[tb]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (s == 0) { load_part(nxt, ic<0>()); load_part(nxt, ic<1>()); }
      if constexpr (s == 1) load_part(nxt, ic<2>());
      if constexpr (s == 2) { load_part(nxt, ic<3>()); load_part(nxt, ic<4>()); }
      __builtin_amdgcn_sched_barrier(0);
    };
    step(ic<0>()); step(ic<1>()); step(ic<2>()); step(ic<3>());
  };
  // fragment register v of lane (j, h) holds row 8 (v / 4) + 4 h + v % 4
  auto init_acc = [&](int k) {
    const uint8_t* bs = bsw + 512 * (k & 3);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // whole-vector bit cast (a bit cast of one element of a vector lvalue
      // reads element 0)
      const v4i b = *reinterpret_cast<const v4i*>(bs + 4 * (8 * m + 4 * h));
      const v4f bf = __builtin_bit_cast(v4f, b);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (I8)
            acc[tb][4 * m + r] = b[r];
          else
            acc[tb][4 * m + r] = bf[r];
        }
    }
  };

  // ---- epilogues.  Staging positions of a token: p = 16 h + 4 m + r holds
  // wave row 8 m + 4 h + r (a lane's 16 rows of a token are contiguous);
  // a read that returns position 16 s + l then holds row
  // 8 (l >> 2) + 4 s + (l & 3).
  uint8_t* const os = ostage + ((OUT == NM_I8 || OUT16) ? wave * 2048 : 0);
  const int orow = 8 * (li >> 2) + (li & 3);      // + 4 s
  auto epilogue_i8 = [&](int k, int r0, int t0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy), 0x00020000);
    const int oob = (int)(g.R * a.ldy);
    const uint8_t* bs = bsw + 512 * (k & 3) + 256;
    // token t (0..63 of the half) is a 32-byte row, f(t) = ((t >> 4) & 1) << 1
    // over 8-byte chunks; reads: lane 16 G + 2 i + hh reads token 16 G + 8 jj
    // + i, chunk (2 s + hh) ^ 2 (G & 1); output lane l then holds position
    // 16 s + l, tokens 16 G + 8 jj .. + 7
    int wb = (32 * j32) | (16 * (h ^ ((j32 >> 4) & 1)));
    int rbs = (32 * (16 * lg + (li >> 1))) | (8 * ((li & 1) ^ (2 * (lg & 1))));
    asm volatile("" : "+v"(wb), "+v"(rbs));
#pragma unroll
    for (int H = 0; H < 2; ++H) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int tb = 2 * H + u;
        int d[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const v4f sv = *reinterpret_cast<const v4f*>(bs + 4 * (8 * m + 4 * h));
          uint32_t bb[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float f = __fmul_rn((float)acc[tb][4 * m + r], sv[r]);
            f = __builtin_amdgcn_fmed3f(f, -128.0f, 127.0f);
            bb[r] = __builtin_bit_cast(uint32_t, f + 12582912.0f);
          }
          d[m] = (int)(__builtin_amdgcn_perm(bb[1], bb[0], 0x0c0c0400u) |
                       __builtin_amdgcn_perm(bb[3], bb[2], 0x04000c0cu));
        }
        *reinterpret_cast<v4i*>(os + 1024 * u + wb) = v4i{d[0], d[1], d[2], d[3]};
      }
      const int tok = t0 + 64 * H + 16 * lg;
      const bool tok_ok = tok < a.T;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const v2i x0 = lds_tr8(os + (rbs ^ (16 * s)));
        const v2i x1 = lds_tr8(os + (rbs ^ (16 * s)) + 256);
        const int row = r0 + 32 * wave + orow + 4 * s;
        const int off = tok_ok ? row * (int)a.ldy + tok : oob;
        __builtin_amdgcn_raw_buffer_store_b128(v4i{x0[0], x0[1], x1[0], x1[1]}, ry, off, 0, kStreamStore);
      }
    }
  };
  auto epilogue_h = [&](int r0, int t0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy * 2), 0x00020000);
    const int oob = (int)(g.R * a.ldy * 2);
    // token t (0..31 of the block) is a 64-byte row, f(t) = ((t >> 3) & 1) << 1
    // over 16-byte chunks; reads: lane 16 G + 4 e + q reads token 8 G + 4 jj +
    // e, chunk (2 s + q / 2) ^ f, byte 8 (q % 2); output lane l then holds
    // position 16 s + l, tokens 8 G + 4 jj .. + 3
    const int e_s = li >> 2, q_s = li & 3;
    int wb = (64 * j32) | (32 * (h ^ ((j32 >> 3) & 1)));
    int rbs = (64 * (8 * lg + e_s) + 8 * (q_s & 1)) | (16 * ((q_s >> 1) ^ ((lg & 1) << 1)));
    asm volatile("" : "+v"(wb), "+v"(rbs));
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      uint32_t d[8];
#pragma unroll
      for (int k2 = 0; k2 < 8; ++k2) d[k2] = pack2<OUT>(acc[tb][2 * k2], acc[tb][2 * k2 + 1]);
      *reinterpret_cast<v4i*>(os + wb) = v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
      *reinterpret_cast<v4i*>(os + wb + 16) = v4i{(int)d[4], (int)d[5], (int)d[6], (int)d[7]};
      const int tok = t0 + 32 * tb + 8 * lg;
      const bool tok_ok = tok < a.T;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint8_t* rp = os + (rbs ^ (32 * s));
        const v2i x0 = lds_tr16(rp);
        const v2i x1 = lds_tr16(rp + 256);
        const int row = r0 + 32 * wave + orow + 4 * s;
        const int off = tok_ok ? (row * (int)a.ldy + tok) * 2 : oob;
        __builtin_amdgcn_raw_buffer_store_b128(v4i{x0[0], x0[1], x1[0], x1[1]}, ry, off, 0, kStreamStore);
      }
    }
  };
  auto store_direct = [&](int r0, int t0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy * 4), 0x00020000);
    const int oob = (int)(g.R * a.ldy * 4);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int t = t0 + 32 * tb + j32;
      // whole-vector cast (a bit cast of one element of a vector lvalue
      // reads element 0)
      const v16i ai = __builtin_bit_cast(v16i, acc[tb]);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = r0 + 32 * wave + 8 * (v >> 2) + 4 * h + (v & 3);
        __builtin_amdgcn_raw_buffer_store_b32(ai[v], ry, t < a.T ? 4 * (row * (int)a.ldy + t) : oob, 0,
                                              kStreamStore);
      }
    }
  };

  int n = 0, ck = 0, ckb = 0, cr0, ct0;
  tile_of(0, cr0, ct0);
  // a step waits until only the loads issued after its group are
  // outstanding (loads complete in order; stores are never counted)
  // Wait until the oldest outstanding group has landed: every group holds
  // at least NL loads and loads complete in order, so at most NL
  // outstanding means everything before the newest group is in.  One
  // unconditional count (not NL plus the next group's extra loads) keeps the
  // wait a single instruction on every path through the unrolled steps.
  auto wait_for_group = [&](int extra_after) {
    (void)extra_after;
    __builtin_amdgcn_s_waitcnt(waitcnt(NL, 15));
  };

  load_group(ic<0>());
  load_group(ic<1>());
  wait_for_group(group_size_extra(1));
  init_acc(0);

  auto block = [&](auto st) {
    constexpr int ST = decltype(st)::value;
    constexpr int NX = (ST + 2) % 3;
    wait_for_group(group_size_extra(n + 1));
    barrier_nofence();
    compute(st, ic<ST>(), ic<NX>());
    ++n;
    if (++ckb < nKB) return;
    ckb = 0;
    if constexpr (OUT == NM_I8)
      epilogue_i8(ck, cr0, ct0);
    else if constexpr (OUT16)
      epilogue_h(cr0, ct0);
    else
      store_direct(cr0, ct0);
    ++ck;
    if (ck < nmine) {
      tile_of(ck, cr0, ct0);
      wait_for_group(group_size_extra(n + 1));
      init_acc(ck);
    }
  };
  const int trips = total / 3, rest = total - 3 * trips;
  for (int it = 0; it < trips; ++it) {
    block(ic<0>());
    block(ic<1>());
    block(ic<2>());
  }
  if (rest > 0) block(ic<0>());
  if (rest > 1) block(ic<1>());
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

template <int WT, int NN, int MM, int OUT>
hipError_t launch_one(const SpmmArgs& a, hipStream_t s) {
  const int mtiles = (int)((a.g.R + BM - 1) / BM);
  const int ntiles = (int)((a.T + BN - 1) / BN);
  const int ntot = mtiles * ntiles;
  const int per_xcd = (ntot + 7) / 8;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int nwg_xcd = cu_count(dev) / 8;                // one eight-wave workgroup per CU
  if (nwg_xcd > per_xcd) nwg_xcd = per_xcd;
  if (nwg_xcd < 1) nwg_xcd = 1;
  hipLaunchKernelGGL((expand32_kernel<WT, NN, MM, OUT>), dim3(8 * nwg_xcd), dim3(NW * 64), 0, s, a, mtiles, ntiles,
                     nwg_xcd);
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
    if (N == 3) return launch_nm<WT, 3, 4>(a, s);
    if (N == 4) return launch_nm<WT, 4, 4>(a, s);
    return hipErrorInvalidValue;   // 2:4 has its sparse-MFMA kernels
  }
  if (N == 1) return launch_nm<WT, 1, 8>(a, s);
  if (N == 2) return launch_nm<WT, 2, 8>(a, s);
  if (N == 4) return launch_nm<WT, 4, 8>(a, s);
  if (N == 8) return launch_nm<WT, 8, 8>(a, s);
  return hipErrorInvalidValue;   // N:M not instantiated (the caller checks)
}

}  // namespace

bool expand32_supported(int N, int M) {
  return (M == 4 && N != 2) || (M == 8 && (N == 1 || N == 2 || N == 4 || N == 8));
}

hipError_t launch_spmm_expand32(const SpmmArgs& a, hipStream_t s) {
  if (a.wdt == NM_I8) return launch_wt<NM_I8>(a, s);
  if (a.wdt == NM_F16) return launch_wt<NM_F16>(a, s);
  return launch_wt<NM_BF16>(a, s);
}

}  // namespace nm
