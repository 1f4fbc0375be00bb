// Persistent int8 2:4 sparse x dense product in the PyTorch-linear layout:
// Yt [T][R] = epilogue(Xt [T][K] . (mask (.) W)^T), so a linear layer's
// input and output need no transposes (the operand layout a Transformer
// keeps its activations in; "Realizable N:M Sparse Transformer Inference via
// Search-Kernel Co-Design", Sec. 1: the linear layers of each block are
// where the time goes).
//
// Structure, pipeline, waits, tile walk and the A operand as the [K][T]
// persistent kernel (nm_spmm_smfmac_i8p.hip): the packed 16 x 128 block is the
// v_smfmac_i32_16x16x128_i8 A operand byte for byte, X streams into three
// LDS stages by direct-to-LDS loads two blocks ahead, one barrier per block.
// What the layout changes:
//
// X stage: 128 tokens x 128 k bytes, token-major (a token's k run is one
// 128-byte LDS row); 16-byte chunk c of token t sits at position c ^ (t & 7).
// Load d of a block fills tokens 8 d .. 8 d + 7: lane l -> token 8 d + l / 8,
// position l % 8, source chunk (l % 8) ^ (l / 8).
//
// B operand: lane (token j, group g) needs k = 16 g .. 16 g + 15 and
// 64 + 16 g .. 64 + 16 g + 15 of token j, in k order: chunks g and 4 + g of
// token j's row, two plain 16-byte reads (the [K][T] kernel needs four
// transpose reads).  For a fixed g the eight tokens of a half lane group sit
// at eight distinct positions, so the reads are conflict-free.
//
// K tail: a token row's bytes past K (its padding, or the next token) meet
// packed values that are zero past K, so they add nothing (int8 products
// are exact).
//
// Epilogue (int8 output): the four rows a lane holds for one token (16 rb +
// 4 g + v) are requantised and packed into a dword per row block, written to
// a per-wave LDS area as token rows of 64 row bytes (the dword of row block
// rb at 16 (rb ^ ((t >> 2) & 3)) + 4 g, which keeps the writes conflict-free),
// then read back 16 bytes at a time, so each lane stores 16 consecutive rows
// of one token; R a multiple of 16 keeps every piece inside its token's row.
// int32 output: a lane's four rows of a token are 16 contiguous bytes,
// stored directly.
#include "nm_common.hpp"

namespace nm {

namespace {

constexpr int RB = 4;              // row blocks (16 rows) per wave
constexpr int TN = 8;              // token tiles (16 tokens) per wave
constexpr int BN = TN * 16;        // 128 tokens per tile
constexpr int STAGE = 128 * BN;    // bytes per X stage (16 KB)

// ACT: the fused activation, a template parameter so that the plain
// epilogue's kernel is unchanged by it
template <int NW, bool OUT_I8, bool ACT = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
smfmac_i8tk_kernel(SpmmArgs a, int mtiles, int ntiles, int nwg_xcd) {
  // device pass only (device-only types and builtins)
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = NW * RB * 16;           // rows per tile
  constexpr int DPW = STAGE / 1024 / NW;     // 1 KB direct-to-LDS loads per wave per block
  // one group of loads per block and wave: A values + meta, X (+ bias and
  // scale on a tile's first block)

  __shared__ __attribute__((aligned(1024))) uint8_t xs0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs2[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ostage[OUT_I8 ? NW * 4096 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t bsbuf[NW * 4 * 512];

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
  const int total = nmine * nKB;              // blocks this workgroup computes
  auto tile_of = [&](int k, int& r0, int& t0) {
    const int L = lo + jw + k * nwg_xcd;
    const int nt = L / mtiles;
    r0 = (L - nt * mtiles) * BM;
    t0 = nt * BN;
  };

  // ---- buffer resources (hardware range checks replace bounds tests)
  const v4i rx = make_rsrc(a.X, (int)(a.T * a.ldx));
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values), 0, (int)g.values_bytes(), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.meta), 0, (int)g.meta_bytes(), 0x00020000);
  const v4i rbias = make_rsrc(a.bias, a.bias ? (int)(g.R * 4) : 0);
  const v4i rscale = make_rsrc(a.scale, a.scale ? (int)(g.R * 4) : 0);

  // ---- X block loads.  An X stage is 128 rows (k) of 128 bytes (tokens);
  // the 16-byte chunk of tokens 16 c .. + 15 of row r sits at position
  // c ^ f(r), f(r) = (r & 7) ^ ((r >> 4) & 1), which makes the transpose
  // reads below conflict-free.  Load d of a block (wave w issues d = w DPW
  // + j) fills rows 8 d .. 8 d + 7: lane l -> row 8 d + l / 8, position
  // l % 8, so every load reads eight whole 128-byte row segments.  The
  // tile's first token and the block's first row go into the scalar offset.
  auto xoff = [&](int j) {
    const int d = wave * DPW + j;
    const int tok = 8 * d + (lane >> 3);
    const int c = (lane & 7) ^ (lane >> 3);
    return tok * ldx + 16 * c;
  };
  auto xstage = [&](auto st) -> uint8_t* {
    constexpr int S = decltype(st)::value;
    return S == 0 ? xs0 : (S == 1 ? xs1 : xs2);
  };

  // ---- A fragments (lane (i, g): 16 bytes at row i, offset 16 g of a block,
  // meta dword g of row i) of this wave's row blocks
  const int voff_v = li * 64 + lg * 16;
  const int voff_m = li * 16 + lg * 4;
  v4i av[3][RB];
  int ai[3][RB];

  // bias and scale of a tile's rows (4 bytes per lane: this wave's 64 rows),
  // loaded with the tile's first block into one LDS slot per tile index mod
  // 4, so a slot is rewritten only after its tile's epilogue; rows past R
  // and absent vectors read as zero.
  uint8_t* const bsw = bsbuf + wave * 2048;
  // the same slot area as an LDS address (integer offsets from the array)
  const uint32_t bs_lds = lds_addr(bsbuf) + wave * 2048;
  auto bias_vec = [&](int k, int rb) {
    return *reinterpret_cast<const v4i*>(bsw + 512 * (k & 3) + 4 * (16 * rb + 4 * lg));
  };
  auto scale_vec = [&](int k, int rb) {
    return *reinterpret_cast<const v4f*>(bsw + 512 * (k & 3) + 256 + 4 * (16 * rb + 4 * lg));
  };

  // ---- load cursor: tile lk (rows lr0, tokens lt0), block lkb; ln groups
  // issued.  A group is issued in parts between the token tiles of a block:
  // part rb < RB the A fragment of row block rb, then the X loads in two
  // halves, then (first block of a tile) bias and scale.  Groups past the
  // end (at most two) still issue their A and X loads, reading nothing but
  // zeros into a stage and register set nobody reads again, so every group
  // but a tile's first has the same size.
  int ln = 0, lk = 0, lkb = 0, lr0 = 0, lt0 = 0;
  tile_of(0, lr0, lt0);
  // No load has all its lanes outside its operand (such a load returns at
  // once, ahead of older loads; see nm_zero_page): row blocks past R and
  // groups past the end read valid blocks (data nobody uses), X tokens
  // entirely past T and absent bias / scale rows read the zero page.
  int g_live = 0, g_rb0 = 0, g_soff = 0, g_trem = 0;
  const v4i rz = zero_rsrc();
  auto load_part = [&](auto st, auto part) {
    constexpr int S = decltype(st)::value;
    constexpr int P = decltype(part)::value;
    if constexpr (P == 0) {
      g_live = __builtin_amdgcn_readfirstlane(ln < total ? 1 : 0);
      g_rb0 = __builtin_amdgcn_readfirstlane((lr0 >> 4) + RB * wave);
      g_soff = __builtin_amdgcn_readfirstlane(lt0 * ldx + lkb * 128);
      g_trem = __builtin_amdgcn_readfirstlane((int)a.T - lt0);   // tokens of this tile inside T
    }
    if constexpr (P < RB) {
      // A first: the compiler's waits for these registers may then hold
      // back at most later A loads, never an X stage.
      const int blk = __builtin_amdgcn_readfirstlane(min(g_rb0 + P, nRB - 1) * nKB + lkb);
      av[S][P] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v, blk * 1024, 0));
      ai[S][P] = (int)__builtin_amdgcn_raw_buffer_load_b32(rm, voff_m, blk * 256, 0);
    } else if constexpr (P == RB || P == RB + 1) {
      uint8_t* sp = xstage(st);
      constexpr int H = DPW / 2, J0 = (P - RB) * H;
#pragma unroll
      for (int j = J0; j < J0 + H; ++j) {
        const int d = wave * DPW + j;
        // load d fills tokens 8 d .. 8 d + 7 of the tile
        if (8 * d < g_trem)
          lds_dma16(rx, lds_addr(sp + d * 1024), xoff(j), g_soff);
        else
          lds_dma16(rz, lds_addr(sp + d * 1024), 16 * lane, 0);
      }
    } else {
      if (g_live && lkb == 0) {
        const uint32_t bs = bs_lds + 512 * (lk & 3);
        const int row0 = __builtin_amdgcn_readfirstlane(lr0 + 64 * wave);
        const int boff = 4 * row0;
        if (a.bias && row0 < (int)g.R)
          lds_dma4(rbias, bs, 4 * lane, boff);
        else
          lds_dma4(rz, bs, 4 * lane, 0);
        if (a.scale && row0 < (int)g.R)
          lds_dma4(rscale, bs + 256, 4 * lane, boff);
        else
          lds_dma4(rz, bs + 256, 4 * lane, 0);
      }
      ++ln;
      if (g_live && ++lkb == nKB) {
        lkb = 0;
        if (++lk < nmine) tile_of(lk, lr0, lt0);
      }
    }
  };
  constexpr int NPART = RB + 3;
  auto load_group = [&](auto st) {
    load_part(st, ic<0>()); load_part(st, ic<1>()); load_part(st, ic<2>()); load_part(st, ic<3>());
    load_part(st, ic<4>()); load_part(st, ic<5>()); load_part(st, ic<6>());
  };
  static_assert(RB == 4 && NPART == 7, "load parts are spelled out for four row blocks");
  // direct-to-LDS loads per group: DPW (plus 2 on a live tile's first block)
  auto group_size_extra = [&](int m) { return (m < total && m % nKB == 0) ? 2 : 0; };

  v4i acc[RB][TN];
  // B fragment of token tile tt: chunks lg and 4 + lg of token 16 tt + li
  // (positions chunk ^ (li & 7)); 16 tt rows are a 2048-byte immediate step
  const int xb0 = 128 * li + 16 * (lg ^ (li & 7));
  const int xb1 = 128 * li + 16 * ((4 + lg) ^ (li & 7));
  auto bfrag = [&](const uint8_t* sb, int tt) -> v8i {
    const v4i c0 = *reinterpret_cast<const v4i*>(sb + xb0 + 2048 * tt);
    const v4i c1 = *reinterpret_cast<const v4i*>(sb + xb1 + 2048 * tt);
    return v8i{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
  };

  // acc += A x B over one block (acc starts a tile at the tile's bias).  B
  // fragments are read two token tiles ahead of their products; the next
  // load group is issued right after the first token tile's products (see
  // the header on waits).  One code path for every block: a second variant
  // for a tile's first block would give the compiler's load-wait bookkeeping
  // merged paths on which the A registers look freshly loaded, and it then
  // waits for every load in flight.
  auto compute = [&](auto st, auto ast, auto nxt) {
    constexpr int AS = decltype(ast)::value;
    const uint8_t* sb = xstage(st);
    v8i bf[3];
#pragma unroll
    for (int tt = 0; tt < 3; ++tt) bf[tt] = bfrag(sb, tt);
    auto tile = [&](auto ttc) {
      constexpr int tt = decltype(ttc)::value;
      if constexpr (tt >= 1 && tt + 2 < TN) bf[(tt + 2) % 3] = bfrag(sb, tt + 2);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][tt] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(av[AS][rb], bf[tt % 3], acc[rb][tt], ai[AS][rb], 0, 0);
      // one part of the next load group after each token tile but the last
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (tt < NPART) load_part(nxt, ic<tt>());
      __builtin_amdgcn_sched_barrier(0);
    };
    static_assert(TN == 8 && NPART < TN, "token tiles are spelled out");
    tile(ic<0>()); tile(ic<1>()); tile(ic<2>()); tile(ic<3>());
    tile(ic<4>()); tile(ic<5>()); tile(ic<6>()); tile(ic<7>());
  };
  // acc = bias of tile k (this wave's own bias rows, loaded with the tile's
  // first group; the caller has waited for that group)
  auto init_acc = [&](int k) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const v4i b = bias_vec(k, rb);
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) acc[rb][tt] = b;
    }
  };

  // ---- int8 epilogue staging: this wave's 4 KB, four token tiles of 16
  // token rows x 64 row bytes; row 16 rb + 4 g + v of token t at byte
  // 16 (rb ^ ((t >> 2) & 3)) + 4 g + v of its row.
  uint8_t* const os = ostage + (OUT_I8 ? wave * 4096 : 0);
  auto epilogue_i8 = [&](int k, int r0, int t0) __attribute__((always_inline)) {
    const float osc = a.out_scale;
    const int sw = (li >> 2) & 3;
    const int wr = 64 * li + 4 * lg;                 // + 16 (rb ^ sw): this lane's dwords
    const int rd = 64 * li + 16 * (lg ^ sw);         // this lane's 16-byte piece: rows 16 lg ..
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(a.T * a.ldy), 0x00020000);
    const int oob = (int)(a.T * a.ldy);
    const int row = r0 + 64 * wave + 16 * lg;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int tt = 4 * h + u;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const v4f sv = scale_vec(k, rb);
          float f[4];
#pragma unroll
          for (int v = 0; v < 4; ++v)
            f[v] = __builtin_amdgcn_fmed3f(i8_pre<ACT>(acc[rb][tt][v], sv[v], osc), -128.0f, 127.0f);
          *reinterpret_cast<uint32_t*>(os + 1024 * u + wr + 16 * (rb ^ sw)) = pack_rne_i8x4(f[0], f[1], f[2], f[3]);
        }
      }
      // the wave reads back only what it wrote (LDS operations of one wave
      // complete in order); every lane stores (fixed operation count for the
      // waits); tokens past T and rows past R go to an offset past the
      // buffer's end, which the range check drops
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v4i piece = *reinterpret_cast<const v4i*>(os + 1024 * u + rd);
        const int tok = t0 + 16 * (4 * h + u) + li;
        const int off = (tok < a.T && row < g.R) ? tok * (int)a.ldy + row : oob;
        __builtin_amdgcn_raw_buffer_store_b128(piece, ry, off, 0, kStreamStore);
      }
    }
  };
  // int32 output: a lane's four rows of one token are 16 contiguous bytes
  auto store_i32 = [&](int r0, int t0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(a.T * a.ldy * 4), 0x00020000);
    const int rw = r0 + 64 * wave + 4 * lg;
    const int oob = (int)(a.T * a.ldy * 4);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) {
        const int t = t0 + 16 * tt + li;
        const int row = rw + 16 * rb;
        __builtin_amdgcn_raw_buffer_store_b128(acc[rb][tt], ry, (t < a.T && row < g.R) ? 4 * (t * (int)a.ldy + row) : oob,
                                               0, kStreamStore);
      }
  };

  // ---- compute cursor: tile ck (rows cr0, tokens ct0), block ckb; block n
  int n = 0, ck = 0, ckb = 0, cr0, ct0;
  tile_of(0, cr0, ct0);

  // wait until the stage of L(m) (and a tile's bias / scale rows) has
  // landed, given the group issued after it.  Only direct-to-LDS loads are
  // counted: they complete in issue order among themselves, but register
  // loads of a later group (A fragments hitting in L2) may complete before
  // them, so a count that included those could pass with the stage still in
  // flight.  The group after holds DPW of them, plus 2 when it starts a
  // live tile; the compiler's own waits cover the A registers.
  auto wait_for_group = [&](int extra_after) {
    if (extra_after)
      __builtin_amdgcn_s_waitcnt(waitcnt(DPW + 2, 15));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt(DPW, 15));
  };

  load_group(ic<0>());
  load_group(ic<1>());
  // tile 0's bias (group 0) has landed once group 1 is all that is left
  wait_for_group(group_size_extra(1));
  init_acc(0);

  // One block: stage / register set ST = n % 3; its loads were issued two
  // steps ago (or in the prologue).
  auto step = [&](auto st) {
    constexpr int ST = decltype(st)::value;
    constexpr int NX = (ST + 2) % 3;
    // groups past the end are issued too (see load_group), so L(n + 1) is
    // always in flight behind L(n)
    wait_for_group(group_size_extra(n + 1));
    barrier_nofence();
    compute(st, ic<ST>(), ic<NX>());
    ++n;
    if (++ckb < nKB) return;
    ckb = 0;
    if constexpr (OUT_I8)
      epilogue_i8(ck, cr0, ct0);
    else
      store_i32(cr0, ct0);
    ++ck;
    if (ck < nmine) {
      tile_of(ck, cr0, ct0);
      // the next tile's bias rows arrive with its first group, L(n); the
      // group after it and the epilogue's stores may still be in flight
      wait_for_group(group_size_extra(n + 1));
      init_acc(ck);
    }
  };
  // The trip count is known up front, so every exit is a plain counter
  // test: no path from a step's end leads back to the loop head except the
  // real back edge (the compiler's own load-wait bookkeeping merges the
  // states of every edge into the head).
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

template <int NW>
hipError_t launch_nw(const SpmmArgs& a, hipStream_t s) {
  constexpr int BM = NW * RB * 16;
  const int mtiles = (int)((a.g.R + BM - 1) / BM);
  const int ntiles = (int)((a.T + BN - 1) / BN);
  const int ntot = mtiles * ntiles;
  const int per_xcd = (ntot + 7) / 8;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  // two waves per SIMD: 8 / NW workgroups per CU
  int nwg_xcd = cu_count(dev) * (8 / NW) / 8;
  if (nwg_xcd > per_xcd) nwg_xcd = per_xcd;
  if (nwg_xcd < 1) nwg_xcd = 1;
  const int grid = 8 * nwg_xcd;
  if (a.ydt == NM_I8 && a.act)
    hipLaunchKernelGGL((smfmac_i8tk_kernel<NW, true, true>), dim3(grid), dim3(NW * 64), 0, s, a, mtiles, ntiles,
                       nwg_xcd);
  else if (a.ydt == NM_I8)
    hipLaunchKernelGGL((smfmac_i8tk_kernel<NW, true>), dim3(grid), dim3(NW * 64), 0, s, a, mtiles, ntiles, nwg_xcd);
  else
    hipLaunchKernelGGL((smfmac_i8tk_kernel<NW, false>), dim3(grid), dim3(NW * 64), 0, s, a, mtiles, ntiles, nwg_xcd);
  return hipGetLastError();
}

}  // namespace

// 4-wave workgroups (256 x 128 tiles, two per CU)
hipError_t launch_spmm_smfmac_i8tk(const SpmmArgs& a, hipStream_t s) { return launch_nw<4>(a, s); }

}  // namespace nm
