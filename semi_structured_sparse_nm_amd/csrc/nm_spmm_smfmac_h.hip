// Persistent fp16 / bf16 2:4 sparse x dense product on the gfx950 sparse
// matrix cores (v_smfmac_f32_16x16x64_{f16,bf16}), fp32 accumulation, bias
// and output rounding fused.
//
// The operation is the N:M sparse product of "Realizable N:M Sparse
// Transformer Inference via Search-Kernel Co-Design" (Sec. 2.1 constraint,
// Sec. 4.2 packed windows); the pages' LLM and Swin workloads run it in half
// precision.  The structure follows the int8 persistent kernel: workgroups
// stay resident and walk a per-XCD tile list, X streams into three LDS stages
// by direct-to-LDS loads, the packed weights go straight to registers, one
// barrier per 64-column block, exact vmcnt counts.
//
// Operand mapping (measured on the GPU with one-hot inputs): for lane
// (row i, group g), A slot c (0..7) multiplies B element 8 (g / 2) +
// 4 ((c % 4) / 2) + pos of lane group 2 (g % 2) + c / 4, pos = index bits
// [2c, 2c + 1].  Reading B lane group h's elements 0..7 as k = 8 h .. 8 h + 7
// and elements 8..15 as k = 32 + 8 h .. + 7 makes A slot c cover dense k
// 16 g + 4 (c / 2) + pos: the lane's 8 slots are the 16-byte run 16 g .. of
// its packed row (64 dense columns per block, 32 kept halves per row) and its
// 16 index bits are bits 16 g .. 16 g + 15 of the row's meta.
//
// X stage: 64 rows (k) of 256 bytes (128 tokens); the 32-byte chunk of
// tokens 16 c .. + 15 of row r sits at position c ^ h(r), h(r) = (r & 7) ^
// 4 ((r >> 3) & 1).  B fragments come from ds_read_b64_tr_b16, which gives
// lane l of a 16-lane group half e = the half at (address of lane 4 e +
// l / 4) + 2 (l % 4): four k-rows of one token per read.
//
// Epilogue (fp16 / bf16 output), per quarter tile (32 tokens): the rows a
// lane holds for one token are rounded to the output type and written
// token-major to a per-wave LDS area (16-byte chunk c of token t at
// c ^ f(t), f(t) = (t & 2) | ((t >> 1) & 4)), read back with
// ds_read_b64_tr_b16 (four tokens of one row per read) and stored as
// 16-byte pieces (8 tokens of one row); fp32 output: direct stores.
#include "nm_common.hpp"

namespace nm {

namespace {

typedef _Float16 v16h __attribute__((ext_vector_type(16)));
typedef __bf16 v16bf __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int TN = 8;              // token tiles (16 tokens) per wave
constexpr int BN = TN * 16;        // 128 tokens per tile
constexpr int STAGE = 64 * 256;    // bytes per X stage: 64 k x 128 tokens x 2 B

template <int WT>
__device__ __forceinline__ v4f smfmac(v4i a, v8i b, v4f c, int idx) {
  if constexpr (WT == NM_F16)
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v16h, b), c,
                                                    idx, 0, 0);
  else
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v16bf, b), c,
                                                     idx, 0, 0);
}

// two fp32 -> packed fp16 / bf16, round to nearest even (v_cvt_pk_f16_f32 /
// v_cvt_pk_bf16_f32)
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
template <int OUT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (OUT == NM_F16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2h));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2bf));
}

// ACT: the fused activation, a template parameter so that the plain
// epilogue's kernel is unchanged by it (as a runtime branch its registers
// made the main loop spill)
template <int NW, int WT, int OUT, bool ACT = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
smfmac_h_kernel(SpmmArgs a, int mtiles, int ntiles, int nwg_xcd, int gm) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr bool OUT16 = OUT != NM_F32;
  // row blocks (16 rows) per wave: 4 with 4-wave workgroups (two per CU),
  // 2 with 8-wave workgroups (one per CU); the tile is 256 x 128 either way
  constexpr int RB = 16 / NW;
  constexpr int BM = NW * RB * 16;
  constexpr int DPW = STAGE / 1024 / NW;     // 1 KB direct-to-LDS loads per wave per block

  __shared__ __attribute__((aligned(1024))) uint8_t xs0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs2[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ostage[OUT16 ? NW * 4096 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t bsbuf[NW * 4 * 256];

  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int nKB = (int)g.nKB;
  const int ldx = (int)a.ldx;
  const int nRB = (int)g.nRB;

  // work items: (tile, K slice); the tiles of one slice are contiguous, in
  // groups of gm row tiles, row tile fastest inside a group, then the next
  // token tile: the workgroups of an XCD running at the same time cover
  // about gm row tiles x (their number / gm) token tiles, so both operands'
  // blocks are shared through its L2 (gm = all row tiles: one token strip at
  // a time, for weights small enough to stay in L2)
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

  const v4i rx = make_rsrc(a.X, (int)(g.K * a.ldx * 2));
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values), 0, (int)g.values_bytes(), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.meta), 0, (int)g.meta_bytes(), 0x00020000);
  const v4i rbias = make_rsrc(a.bias, a.bias ? (int)(g.R * 4) : 0);

  // ---- X block loads: load d (wave w issues d = w DPW + j) fills rows
  // 4 d .. 4 d + 3: lane l -> row 4 d + l / 16, 16-byte piece l % 16, i.e.
  // position p = (l % 16) / 2, half l % 2 of a 32-byte chunk; the chunk at
  // position p holds tokens 16 (p ^ h(row)) ..
  auto xoff = [&](int j) {
    const int d = wave * DPW + j;
    const int row = 4 * d + (lane >> 4);
    const int p = (lane & 15) >> 1;
    const int c = p ^ (row & 7) ^ (((row >> 3) & 1) << 2);
    return row * ldx * 2 + 32 * c + 16 * (lane & 1);
  };
  auto xstage = [&](auto st) -> uint8_t* {
    constexpr int S = decltype(st)::value;
    return S == 0 ? xs0 : (S == 1 ? xs1 : xs2);
  };

  // ---- A fragments: 16 bytes at row i, offset 16 g of a block (64 bytes per
  // row); index word: the row's meta dword g / 2, its half g % 2 moved to the
  // low 16 bits (the instruction reads the low half)
  const int voff_v = li * 64 + lg * 16;
  const int voff_m = li * 8 + (lg >> 1) * 4;
  const int ishift = 16 * (lg & 1);
  v4i av[3][RB];
  int ai[3][RB];

  // bias rows of a tile (4 bytes per lane: this wave's 64 rows), one slot per
  // tile index mod 4; absent bias reads as zero
  uint8_t* const bsw = bsbuf + wave * 1024;
  auto bias_vec = [&](int k, int rb) {
    return *reinterpret_cast<const v4f*>(bsw + 256 * (k & 3) + 4 * (16 * rb + 4 * lg));
  };

  int ln = 0, lk = 0, lkb = 0, lr0 = 0, lt0 = 0, lks = 0;
  tile_of(0, lr0, lt0, lks);
  lks *= kbs;                                // first column block of the slice
  int g_live = 0, g_rb0 = 0, g_soff = 0;
  // No load has all its lanes outside its operand (such a load returns at
  // once, ahead of older loads; see nm_zero_page): row blocks past R and
  // groups past the end read valid blocks (data nobody uses), X rows
  // entirely past K and absent bias rows read the zero page.
  const v4i rz = zero_rsrc();
  int g_krem = 0;
  auto load_part = [&](auto st, auto part) {
    constexpr int S = decltype(st)::value;
    constexpr int P = decltype(part)::value;
    if constexpr (P == 0) {
      g_live = __builtin_amdgcn_readfirstlane(ln < total ? 1 : 0);
      g_rb0 = __builtin_amdgcn_readfirstlane((lr0 >> 4) + RB * wave);
      g_soff = __builtin_amdgcn_readfirstlane(((lks + lkb) * 64 * ldx + lt0) * 2);
      g_krem = __builtin_amdgcn_readfirstlane((int)g.K - (lks + lkb) * 64);   // rows of this block inside K
    }
    if constexpr (P < RB) {
      const int blk = __builtin_amdgcn_readfirstlane(min(g_rb0 + P, nRB - 1) * nKB + lks + lkb);
      av[S][P] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v, blk * 1024, 0));
      ai[S][P] = (int)__builtin_amdgcn_raw_buffer_load_b32(rm, voff_m, blk * 128, 0);
    } else if constexpr (P == RB || P == RB + 1) {
      uint8_t* sp = xstage(st);
      constexpr int H = DPW / 2, J0 = (P - RB) * H;
#pragma unroll
      for (int j = J0; j < J0 + H; ++j) {
        const int d = wave * DPW + j;
        // load d fills rows 4 d .. 4 d + 3 of the stage
        if (4 * d < g_krem)
          lds_dma16(rx, lds_addr(sp + d * 1024), xoff(j), g_soff);
        else
          lds_dma16(rz, lds_addr(sp + d * 1024), 16 * lane, 0);
      }
    } else {
      if (g_live && lkb == 0) {
        const int row0 = __builtin_amdgcn_readfirstlane(lr0 + 16 * RB * wave);
        if (a.bias && row0 < (int)g.R)
          lds_dma4(rbias, lds_addr(bsw + 256 * (lk & 3)), 4 * lane, 4 * row0);
        else
          lds_dma4(rz, lds_addr(bsw + 256 * (lk & 3)), 4 * lane, 0);
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
  auto load_group = [&](auto st) {
    load_part(st, ic<0>()); load_part(st, ic<1>()); load_part(st, ic<2>()); load_part(st, ic<3>());
    load_part(st, ic<4>());
    if constexpr (NPART > 5) load_part(st, ic<5>());
    if constexpr (NPART > 6) load_part(st, ic<6>());
  };
  static_assert(NPART >= 5 && NPART <= 7, "load parts are spelled out for two or four row blocks");
  auto group_size_extra = [&](int m) { return (m < total && m % kbs == 0) ? 1 : 0; };

  v4f acc[RB][TN];
  // transpose reads of token tile tt, read i (k rows 8 g + 4 (i & 1) +
  // 32 (i >> 1) + e): source lane 4 e + q (of each 16-lane group) reads row
  // r = that + e, tokens 16 tt + 4 q .. + 3, at chunk position tt ^ h(r)
  // = tt ^ e ^ 4 ((i & 1) ^ (g & 1)).  The base has no bits 5..7, so the
  // address is base ^ 32 tt once the position term is or-ed in.
  const int e_s = li >> 2, q_s = li & 3;
  const int base0 = (8 * lg + e_s) * 256 + 8 * q_s;
  const int xa = base0 | (32 * (e_s ^ (4 * (lg & 1))));
  const int xb = (base0 + 4 * 256) | (32 * (e_s ^ (4 * ((lg & 1) ^ 1))));
  auto bfrag = [&](const uint8_t* sb, int tt) -> v8i {
    int oa = xa ^ (32 * tt), ob = xb ^ (32 * tt);
    asm volatile("" : "+v"(oa), "+v"(ob));
    const v2i p0 = lds_tr16(sb + oa);
    const v2i p1 = lds_tr16(sb + ob);
    const v2i p2 = lds_tr16(sb + oa + 32 * 256);
    const v2i p3 = lds_tr16(sb + ob + 32 * 256);
    return v8i{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  };

  auto compute = [&](auto st, auto ast, auto nxt) {
    constexpr int AS = decltype(ast)::value;
    const uint8_t* sb = xstage(st);
    // lane group g's 16 index bits, moved to the low half: the lanes of
    // groups 1 and 3 shift their meta word in place (registers are scarce)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) ai[AS][rb] = (int)((uint32_t)ai[AS][rb] >> ishift);
    // B fragments one token tile ahead (the 16-bit index shift and the
    // second read base leave no registers for a deeper ring)
    v8i bf[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) bf[tt] = bfrag(sb, tt);
    auto tile = [&](auto ttc) {
      constexpr int tt = decltype(ttc)::value;
      if constexpr (tt >= 1 && tt + 1 < TN) bf[(tt + 1) % 2] = bfrag(sb, tt + 1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb][tt] = smfmac<WT>(av[AS][rb], bf[tt % 2], acc[rb][tt], ai[AS][rb]);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (tt < NPART) load_part(nxt, ic<tt>());
      __builtin_amdgcn_sched_barrier(0);
    };
    static_assert(TN == 8 && NPART < TN, "token tiles are spelled out");
    tile(ic<0>()); tile(ic<1>()); tile(ic<2>()); tile(ic<3>());
    tile(ic<4>()); tile(ic<5>()); tile(ic<6>()); tile(ic<7>());
  };
  auto init_acc = [&](int k) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const v4f b = bias_vec(k, rb);
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) acc[rb][tt] = b;
    }
  };

  uint8_t* const os = ostage + (OUT16 ? wave * 4096 : 0);
  // 16-bit epilogue, per quarter (tokens 32 u4 .. + 31 of the tile).
  // Staging: token t (0..31) is a 128-byte row of 64 positions (2 bytes);
  // position 16 g + 4 rb + v holds row 16 rb + 4 g + v of the wave; 16-byte
  // chunk c of token t is stored at c ^ f(t).
  auto epilogue_h = [&](int r0, int t0, auto actc) __attribute__((always_inline)) {
    constexpr bool EACT = decltype(actc)::value != 0;
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy * 2), 0x00020000);
    const int oob = (int)(g.R * a.ldy * 2);
    // reads: lane 16 G + 4 e + q reads token 8 G + 4 j + e, positions
    // 16 s + 4 q .. + 3 (chunk 2 s + q / 2, byte 8 (q % 2)); output lane l
    // of group G then holds position 16 s + l = row 16 (l >> 2) + 4 s +
    // (l & 3), tokens 8 G + 4 j .. + 3
    // Both address families are one per-lane base xor-ed with a constant:
    // writes of staged token 16 w + li: f = (li & 2) | ((li >> 1) & 4) for
    // both w, chunk 2 g + b at 16 ((2 g) ^ f) + 16 b; reads of token 8 G +
    // 4 j + e: f = (e & 2) | 4 (G & 1), chunk (2 s + q / 2) ^ f at
    // 32 (s ^ f / 2) + 16 (q / 2).  The empty asm keeps the compiler from
    // hoisting a register per address out of the main loop.
    int wbase = 128 * li + 16 * ((2 * lg) ^ ((li & 2) | ((li >> 1) & 4)));
    int rbase = (1024 * lg + 128 * e_s + 8 * q_s) | (32 * (((e_s & 2) >> 1) | ((lg & 1) << 1)));
    int orow = 16 * (li >> 2) + (li & 3);
    asm volatile("" : "+v"(wbase), "+v"(rbase), "+v"(orow));
#pragma unroll
    for (int u4 = 0; u4 < 4; ++u4) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int tt = 2 * u4 + w;
        uint32_t d[8];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          d[2 * rb] = pack2<OUT>(fp_act<EACT>(acc[rb][tt][0]), fp_act<EACT>(acc[rb][tt][1]));
          d[2 * rb + 1] = pack2<OUT>(fp_act<EACT>(acc[rb][tt][2]), fp_act<EACT>(acc[rb][tt][3]));
        }
        *reinterpret_cast<v4i*>(os + wbase + 2048 * w) = v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
        if constexpr (RB > 2)
          *reinterpret_cast<v4i*>(os + wbase + 2048 * w + 16) = v4i{(int)d[4], (int)d[5], (int)d[6], (int)d[7]};
      }
      // the staging writes complete before the transpose reads are issued
      // (one wave's LDS operations are ordered; this wait does not rely on
      // that for the transpose reads, at the cost of one LDS round trip per
      // quarter)
      __builtin_amdgcn_s_waitcnt(waitcnt(63, 0));
      const int tok = t0 + 32 * u4 + 8 * lg;
      const bool tok_ok = tok < a.T;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint8_t* rp = os + (rbase ^ (32 * s));
        const v2i x0 = lds_tr16(rp);
        const v2i x1 = lds_tr16(rp + 512);
        // with two row blocks a wave owns rows 0..31 of the staging layout's
        // 64; the lanes that read rows 32..63 store nothing
        const int row = r0 + 16 * RB * wave + orow + 4 * s;
        const int off = (tok_ok && orow + 4 * s < 16 * RB) ? (row * (int)a.ldy + tok) * 2 : oob;
        __builtin_amdgcn_raw_buffer_store_b128(v4i{x0[0], x0[1], x1[0], x1[1]}, ry, off, 0, kStreamStore);
      }
    }
  };
  // fp32 output, or slice ks's partial sums under a K split
  auto store_f32 = [&](int r0, int t0, int ks, auto actc) __attribute__((always_inline)) {
    constexpr bool EACT = decltype(actc)::value != 0;
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<float*>(a.Y) + ks * a.ys, 0, (int)(g.R * a.ldy * 4), 0x00020000);
    const int rw = r0 + 16 * RB * wave + 4 * lg;
    const int oob = (int)(g.R * a.ldy * 4);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) {
        const int t = t0 + 16 * tt + li;
        // whole-vector cast: a bit cast of one element of a vector lvalue
        // reads element 0 (observed miscompile)
        const v4f x = acc[rb][tt];
        const v4i ai4 = __builtin_bit_cast(v4i, v4f{fp_act<EACT>(x[0]), fp_act<EACT>(x[1]), fp_act<EACT>(x[2]),
                                                    fp_act<EACT>(x[3])});
#pragma unroll
        for (int v = 0; v < 4; ++v)
          __builtin_amdgcn_raw_buffer_store_b32(
              ai4[v], ry,
              t0 + 16 * tt < a.T ? 4 * ((rw + 16 * rb + v) * (int)a.ldy + t) : oob, 0, kStreamStore);
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
    if constexpr (OUT16)
      epilogue_h(cr0, ct0, ic<ACT ? 1 : 0>());
    else
      store_f32(cr0, ct0, cks, ic<ACT ? 1 : 0>());
    ++ck;
    if (ck < nmine) {
      tile_of(ck, cr0, ct0, cks);
      // the next tile's bias rows arrive with its first group, L(n); only
      // the group after it (and the epilogue's stores) may still be in flight
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

template <int NW, int WT>
hipError_t launch_nw(const SpmmArgs& a, hipStream_t s) {
  constexpr int BM = 256;
  const int mtiles = (int)((a.g.R + BM - 1) / BM);
  const int ntiles = (int)((a.T + BN - 1) / BN);
  const int ntot = mtiles * ntiles * a.ksplit;
  const int per_xcd = (ntot + 7) / 8;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int nwg_xcd = cu_count(dev) * (8 / NW) / 8;
  if (nwg_xcd > per_xcd) nwg_xcd = per_xcd;
  if (nwg_xcd < 1) nwg_xcd = 1;
  const int grid = 8 * nwg_xcd;
  // operand bytes one row tile / one token tile brings per 128-column step
  const double wk = 256.0 * (64 * 2 + 16), xk = 128.0 * BN * 2;
  const int gm = tile_group_rows(mtiles, ntiles, nwg_xcd, wk, xk, (double)(a.g.values_bytes() + a.g.meta_bytes()));
  if (a.act) {
    if (a.ydt == NM_F32)
      hipLaunchKernelGGL((smfmac_h_kernel<NW, WT, NM_F32, true>), dim3(grid), dim3(NW * 64), 0, s, a, mtiles, ntiles,
                         nwg_xcd, gm);
    else if (WT == NM_F16)
      hipLaunchKernelGGL((smfmac_h_kernel<NW, WT, NM_F16, true>), dim3(grid), dim3(NW * 64), 0, s, a, mtiles, ntiles,
                         nwg_xcd, gm);
    else
      hipLaunchKernelGGL((smfmac_h_kernel<NW, WT, NM_BF16, true>), dim3(grid), dim3(NW * 64), 0, s, a, mtiles, ntiles,
                         nwg_xcd, gm);
  } else if (a.ydt == NM_F32) {
    hipLaunchKernelGGL((smfmac_h_kernel<NW, WT, NM_F32>), dim3(grid), dim3(NW * 64), 0, s, a, mtiles, ntiles, nwg_xcd, gm);
  } else if (WT == NM_F16) {
    hipLaunchKernelGGL((smfmac_h_kernel<NW, WT, NM_F16>), dim3(grid), dim3(NW * 64), 0, s, a, mtiles, ntiles, nwg_xcd, gm);
  } else {
    hipLaunchKernelGGL((smfmac_h_kernel<NW, WT, NM_BF16>), dim3(grid), dim3(NW * 64), 0, s, a, mtiles, ntiles, nwg_xcd, gm);
  }
  return hipGetLastError();
}

}  // namespace

// fp16 / bf16 2:4, 4-wave workgroups (256 x 128 tiles, two per CU)
hipError_t launch_spmm_smfmac_h(const SpmmArgs& a, hipStream_t s) {
  return a.wdt == NM_F16 ? launch_nw<4, NM_F16>(a, s) : launch_nw<4, NM_BF16>(a, s);
}

}  // namespace nm
