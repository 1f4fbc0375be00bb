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
// launch level): NW-wave workgroups stay resident (two waves per SIMD) and
// walk a list of (64 NW) x 128 output tiles.  Their loads form one continuous
// stream over (tile, 128-column block) pairs, two blocks ahead of the compute
// (three X stages in LDS, three register sets of A fragments), so the next
// tile's first blocks are in flight while the current tile is multiplied and
// requantised; no tile starts cold.
//
// Waits.  One vmcnt counter covers loads and stores; loads complete in issue
// order among themselves, but a store may complete before loads issued
// ahead of it, so a wait never counts stores.  Block n's loads L(n) are a
// fixed group: A fragments (8 register loads) first, then the X stage and
// the tile's bias / scale rows (direct-to-LDS).  Step n waits until at most
// |L(n+1)| operations are outstanding: whatever else is outstanding then
// (a stage of L(n+1), an epilogue's stores) leaves no load of L(n) pending,
// so L(n) has landed; then a barrier publishes every wave's part of the
// stage.  A tile's stores are waited for (at the latest) by the next step's
// wait, a block after they were issued.  L(n+2) is issued
// after the first token tile of block n is multiplied: by then the compiler's
// own waits for the A(n) registers are placed, and they count only the
// register loads it can see (A(n+1) and the stores), so they hold back at
// most A(n+1), issued a whole block earlier -- never an X stage.
//
// Tile order: each XCD (dispatch is round-robin over 8 XCDs) owns a
// contiguous range of tiles, row tile fastest; its workgroups sweep that
// range together, so the row tiles of one 128-token strip of X run at about
// the same time on one XCD and the strip comes from HBM once into its L2.
//
// Epilogue (int8 output), per half tile (64 tokens): f32(acc) * scale[r] (a
// separately rounded product; the bias is the accumulator's start value),
// clamp to [-128, 127], add 1.5 * 2^23 so the low byte is the round-half-even
// int8, written straight into its byte of the packed dword (SDWA); the four
// rows a lane holds for one token are packed into a dword, the
// four row blocks' dwords of one token into 16 bytes, written token-major to
// a per-wave LDS area (16-byte chunk c of token t stored at c ^ f(t), which
// keeps the 16-byte writes and the transpose reads conflict-free), then read
// back with ds_read_b64_tr_b8 so each lane holds 16 consecutive tokens of one
// row and stores them as one 16-byte piece; the four lane groups of a store
// cover 64 consecutive bytes of the same 16 rows.  int32 output: acc (bias
// included) stored directly.
#include "nm_common.hpp"

namespace nm {

namespace {

constexpr int RB = 4;              // row blocks (16 rows) per wave
constexpr int TN = 8;              // token tiles (16 tokens) per wave
constexpr int BN = TN * 16;        // 128 tokens per tile
constexpr int STAGE = 128 * BN;    // bytes per X stage (16 KB)

// X stages in LDS: three with 4-wave workgroups (two per CU), six with
// 8-wave ones (one per CU), whose activation then arrives PX = stages - 1
// blocks ahead of its products while the A fragments stay two ahead (three
// register sets).  Shapes with a large activation per weight (ViT-B FC2:
// K 3072, 38.7 MB of X) stream it from HBM, where two blocks of lead time
// leave the waves waiting on memory.
template <int NW> constexpr int x_stages() { return NW == 8 ? 6 : 3; }

// ACT: the fused activation, a template parameter so that the plain
// epilogue's kernel is unchanged by it
template <int NW, bool OUT_I8, bool ACT = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
smfmac_i8p_kernel(SpmmArgs a, int mtiles, int ntiles, int nwg_xcd) {
  // device pass only (device-only types and builtins)
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int BM = NW * RB * 16;           // rows per tile
  constexpr int DPW = STAGE / 1024 / NW;     // 1 KB direct-to-LDS loads per wave per block
  constexpr int XS = x_stages<NW>();
  constexpr int PX = XS - 1;                 // blocks the X loads run ahead
  // per block and wave: an A group (A values + meta, and the bias and scale
  // rows on a tile's first block) two blocks ahead, an X group PX ahead

  __shared__ __attribute__((aligned(1024))) uint8_t xsb[XS][STAGE];
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
  const v4i rx = make_rsrc(a.X, (int)(g.K * a.ldx));
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
    const int row = 8 * d + (lane >> 3);
    const int c = (lane & 7) ^ (row & 7) ^ ((row >> 4) & 1);
    return row * ldx + 16 * c;
  };
  auto xstage = [&](auto st) -> uint8_t* { return xsb[decltype(st)::value]; };

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

  // ---- load cursors: the A cursor (tile ak, rows ar0, block akb; an
  // groups issued) and the X cursor (tile xk, tokens xt0, block xkb; xn
  // groups issued).  The loads of a block are issued in parts between the
  // token tiles of an earlier block: parts rb < RB the A fragment of row
  // block rb (A cursor), part RB (first block of a tile) the tile's bias and
  // scale rows, then the A cursor moves on; parts RB + 1 and RB + 2 the X
  // loads in two halves (X cursor), then the X cursor moves on.  Groups past
  // the end still issue their A and X loads, at the last block's addresses,
  // into a stage and register set nobody reads again, so every X group has
  // the same number of direct-to-LDS loads.  No load has all its lanes
  // outside its operand (such a load returns at once, ahead of older loads;
  // see nm_zero_page): row blocks past R read the last row block, X rows
  // entirely past K read the zero page, absent bias / scale rows too.
  int an = 0, ak = 0, akb = 0, ar0 = 0, at0 = 0;
  int xn = 0, xk = 0, xkb = 0, xr0 = 0, xt0 = 0;
  tile_of(0, ar0, at0);
  tile_of(0, xr0, xt0);
  int g_live = 0, g_rb0 = 0, g_soff = 0, g_krem = 0;
  const v4i rz = zero_rsrc();
  auto load_part = [&](auto ast, auto xst, auto part) {
    constexpr int AS = decltype(ast)::value;
    constexpr int P = decltype(part)::value;
    if constexpr (P == 0) {
      g_live = __builtin_amdgcn_readfirstlane(an < total ? 1 : 0);
      g_rb0 = __builtin_amdgcn_readfirstlane((ar0 >> 4) + RB * wave);
    }
    if constexpr (P < RB) {
      // A first: the compiler's waits for these registers may then hold
      // back at most later A loads, never an X stage.
      const int blk = __builtin_amdgcn_readfirstlane(min(g_rb0 + P, nRB - 1) * nKB + akb);
      av[AS][P] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v, blk * 1024, 0));
      ai[AS][P] = (int)__builtin_amdgcn_raw_buffer_load_b32(rm, voff_m, blk * 256, 0);
    } else if constexpr (P == RB) {
      if (g_live && akb == 0) {
        const uint32_t bs = bs_lds + 512 * (ak & 3);
        const int row0 = __builtin_amdgcn_readfirstlane(ar0 + 64 * wave);
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
      ++an;
      if (g_live && ++akb == nKB) {
        akb = 0;
        if (++ak < nmine) tile_of(ak, ar0, at0);
      }
    } else {
      if constexpr (P == RB + 1) {
        g_soff = __builtin_amdgcn_readfirstlane(xkb * 128 * ldx + xt0);
        g_krem = __builtin_amdgcn_readfirstlane((int)g.K - xkb * 128);   // rows of this block inside K
      }
      uint8_t* sp = xstage(xst);
      constexpr int H = DPW / 2, J0 = (P - RB - 1) * H;
#pragma unroll
      for (int j = J0; j < J0 + H; ++j) {
        const int d = wave * DPW + j;
        // load d fills rows 8 d .. 8 d + 7 of the stage
        if (8 * d < g_krem)
          lds_dma16(rx, lds_addr(sp + d * 1024), xoff(j), g_soff);
        else
          lds_dma16(rz, lds_addr(sp + d * 1024), 16 * lane, 0);
      }
      if constexpr (P == RB + 2) {
        const int live = __builtin_amdgcn_readfirstlane(xn < total ? 1 : 0);
        ++xn;
        if (live && ++xkb == nKB) {
          xkb = 0;
          if (++xk < nmine) tile_of(xk, xr0, xt0);
        }
      }
    }
  };
  constexpr int NPART = RB + 3;
  static_assert(RB == 4 && NPART == 7, "load parts are spelled out for four row blocks");
  auto load_a_group = [&](auto ast) {
    load_part(ast, ic<0>(), ic<0>()); load_part(ast, ic<0>(), ic<1>()); load_part(ast, ic<0>(), ic<2>());
    load_part(ast, ic<0>(), ic<3>()); load_part(ast, ic<0>(), ic<4>());
  };
  auto load_x_group = [&](auto xst) {
    load_part(ic<0>(), xst, ic<5>()); load_part(ic<0>(), xst, ic<6>());
  };
  // bias and scale loads issued with block m's A group: 2 on a live tile's
  // first block
  auto group_size_extra = [&](int m) { return (m < total && m % nKB == 0) ? 2 : 0; };

  v4i acc[RB][TN];
  // transpose reads of token tile tt: lane (i, g) reads row r = kq + 16 g +
  // i / 2 (kq = 0, 8, 64, 72), tokens 16 tt + 8 (i & 1) .. + 7, i.e. chunk tt
  // at position tt ^ f(r) = tt ^ (i / 2) ^ (g & 1).  Of the two lane groups
  // served together, one reads positions of one parity on even rows and the
  // other the opposite parity, so the 32 lanes cover all 64 banks once.
  const int rbase = 128 * (16 * lg + (li >> 1)) + 8 * (li & 1);
  const int tsw = (li >> 1) ^ (lg & 1);
  // rbase has no bits 4..6, so rbase + 16 (tt ^ tsw) = xb ^ 16 tt; the
  // empty asm keeps the compiler from hoisting eight per-tile addresses
  // (registers are scarce in the main loop)
  const int xb = rbase | (16 * tsw);
  auto bfrag = [&](const uint8_t* sb, int tt) -> v8i {
    int o = xb ^ (16 * tt);
    asm volatile("" : "+v"(o));
    const uint8_t* p = sb + o;
    const v2i p0 = lds_tr8(p);
    const v2i p1 = lds_tr8(p + 8 * 128);
    const v2i p2 = lds_tr8(p + 64 * 128);
    const v2i p3 = lds_tr8(p + 72 * 128);
    return v8i{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  };

  // acc += A x B over one block (acc starts a tile at the tile's bias).  B
  // fragments are read two token tiles ahead of their products; the loads
  // of later blocks (A set nas, X stage nxs) are issued in parts after the
  // token tiles' products (see the header on waits).  One code path for every block: a second variant
  // for a tile's first block would give the compiler's load-wait bookkeeping
  // merged paths on which the A registers look freshly loaded, and it then
  // waits for every load in flight.
  auto compute = [&](auto st, auto ast, auto nas, auto nxs, bool live) {
    constexpr int AS = decltype(ast)::value;
    const uint8_t* sb = xstage(st);
    v8i bf[3];
    if (live) {
#pragma unroll
      for (int tt = 0; tt < 3; ++tt) bf[tt] = bfrag(sb, tt);
    }
    auto tile = [&](auto ttc) {
      constexpr int tt = decltype(ttc)::value;
      if (live) {
        if constexpr (tt >= 1 && tt + 2 < TN) bf[(tt + 2) % 3] = bfrag(sb, tt + 2);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb][tt] =
              __builtin_amdgcn_smfmac_i32_16x16x128_i8(av[AS][rb], bf[tt % 3], acc[rb][tt], ai[AS][rb], 0, 0);
      }
      // one part of the next load group after each token tile but the last
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (tt < NPART) load_part(nas, nxs, ic<tt>());
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

  // ---- int8 epilogue staging: this wave's 4 KB, 64 tokens x 64 row
  // positions; row 16 rb + 4 g + v of the wave is position 16 g + 4 rb + v,
  // so one lane's four row blocks of one token are 16 contiguous bytes.
  // Chunk c (positions 16 c .. + 15) of token t sits at c ^ f(t),
  // f(t) = bit 2 of t | (bit 4 of t) << 1.
  uint8_t* const os = ostage + (OUT_I8 ? wave * 4096 : 0);
  auto epilogue_i8 = [&](int k, int r0, int t0) __attribute__((always_inline)) {
    const float osc = a.out_scale;
    // writes: token 16 u + li (u = 0..3), chunk lg
    int wb[2];
  #pragma unroll
    for (int par = 0; par < 2; ++par) wb[par] = 64 * li + 16 * (lg ^ ((li >> 2) & 1) ^ (par << 1));
    // transpose reads: lane 16 G + 2 i + h reads token 16 G + 8 e + i, chunk
    // q ^ f, byte 8 h; output lane l of group G then holds position 16 q + l,
    // i.e. row 16 (l >> 2) + 4 q + (l & 3), tokens 16 G + 8 e .. + 7
    int rq[4];
    {
      const int i = (li >> 1) & 7, h = li & 1;
      const int f = ((i >> 2) & 1) | ((lg & 1) << 1);
  #pragma unroll
      for (int q = 0; q < 4; ++q) rq[q] = 1024 * lg + 64 * i + 16 * (q ^ f) + 8 * h;
    }
    const int orow = 16 * (li >> 2) + (li & 3);   // + 4 q: this lane's output row in the wave
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy), 0x00020000);
    const int oob = (int)(g.R * a.ldy);
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
        *reinterpret_cast<v4i*>(os + 1024 * u + wb[u & 1]) = v4i{d[0], d[1], d[2], d[3]};
      }
      // the wave reads back only what it wrote, after its staging writes
      // have completed (no reliance on the order of LDS writes and
      // transpose reads)
      __builtin_amdgcn_s_waitcnt(waitcnt(63, 0));
      // every lane stores (fixed operation count for the waits); pieces past
      // T go to an offset past the buffer's end, which the range check drops
      const int tok = t0 + 64 * h + 16 * lg;
      const bool tok_ok = tok < a.T;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v2i x0 = lds_tr8(os + rq[q]);
        const v2i x1 = lds_tr8(os + rq[q] + 512);
        const int row = r0 + 64 * wave + orow + 4 * q;
        const int off = tok_ok ? row * (int)a.ldy + tok : oob;
        __builtin_amdgcn_raw_buffer_store_b128(v4i{x0[0], x0[1], x1[0], x1[1]}, ry, off, 0, kStreamStore);
      }
    }
  };
  // int32 output: acc (bias included) stored directly
  auto store_i32 = [&](int r0, int t0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy * 4), 0x00020000);
    const int rw = r0 + 64 * wave + 4 * lg;
    const int oob = (int)(g.R * a.ldy * 4);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) {
        const int t = t0 + 16 * tt + li;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          __builtin_amdgcn_raw_buffer_store_b32(
              acc[rb][tt][v], ry, t0 + 16 * tt < a.T ? 4 * ((rw + 16 * rb + v) * (int)a.ldy + t) : oob, 0, kStreamStore);
      }
  };

  // ---- compute cursor: tile ck (rows cr0, tokens ct0), block ckb; block n
  int n = 0, ck = 0, ckb = 0, cr0, ct0;
  tile_of(0, cr0, ct0);

  // Waits count only direct-to-LDS loads: they complete in issue order
  // among themselves, but register loads (A fragments hitting in L2) may
  // complete before older ones, so a count that included those could pass
  // with a stage still in flight; extra loads outstanding only make a wait
  // stricter.  The compiler's own waits cover the A registers.
  // - Block n's stage.  With PX = 2 the loads issued after X(n) are block
  //   n + 1's bias and scale (2 on a live tile's first block) and X(n + 1)
  //   (DPW); with PX > 2 at least the X groups n + 1 .. n + PX - 1.
  // - A tile's bias and scale rows (issued with its first block's A group,
  //   two blocks ahead, before that block's X group): with PX = 2 the same
  //   count; with PX > 2 at least the next two X groups follow them.
  auto wait_stage = [&](int m) {
    if constexpr (PX == 2) {
      if (group_size_extra(m + 1))
        __builtin_amdgcn_s_waitcnt(waitcnt(DPW + 2, 15));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt(DPW, 15));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt((PX - 1) * DPW, 15));
    }
  };
  auto wait_bias = [&](int m) {
    if constexpr (PX == 2)
      wait_stage(m);
    else
      __builtin_amdgcn_s_waitcnt(waitcnt(2 * DPW, 15));
  };

  // prologue: A groups 0 and 1 (with the bias rows) and X groups 0 .. PX-1
  load_a_group(ic<0>());
  load_x_group(ic<0>());
  load_a_group(ic<1>());
  load_x_group(ic<1>());
  if constexpr (PX > 2) {
    load_x_group(ic<2 % XS>());
    load_x_group(ic<3 % XS>());
    load_x_group(ic<4 % XS>());
    static_assert(PX == 2 || PX == 5, "prologue X groups are spelled out for 3 or 6 stages");
    // one drain at the start
    __builtin_amdgcn_s_waitcnt(waitcnt(0, 15));
  } else {
    // tile 0's bias (group 0) has landed once group 1 is all that is left
    wait_stage(0);
  }
  init_acc(0);

  // One block: X stage ST = n % XS, A register set ST % 3; its loads were
  // issued PX and two blocks ago (or in the prologue).
  auto step = [&](auto st) {
    constexpr int ST = decltype(st)::value;
    constexpr int AS = ST % 3;
    constexpr int NA = (AS + 2) % 3;
    constexpr int NXS = (ST + PX) % XS;
    // groups past the end are issued too, so the counted loads are always
    // in flight behind block n's
    wait_stage(n);
    barrier_nofence();
    // a wave whose 64 rows of the tile lie past R (the last row tile of a
    // shape that is not a multiple of BM) skips its products and epilogue;
    // it still issues its share of the workgroup's loads and barriers
    const bool live = __builtin_amdgcn_readfirstlane(cr0 + 64 * wave < (int)g.R ? 1 : 0) != 0;
    compute(st, ic<AS>(), ic<NA>(), ic<NXS>(), live);
    ++n;
    if (++ckb < nKB) return;
    ckb = 0;
    if (live) {
      if constexpr (OUT_I8)
        epilogue_i8(ck, cr0, ct0);
      else
        store_i32(cr0, ct0);
    }
    ++ck;
    if (ck < nmine) {
      tile_of(ck, cr0, ct0);
      // the next tile's bias rows arrived with block n's A group; later
      // groups and the epilogue's stores may still be in flight
      wait_bias(n);
      init_acc(ck);
    }
  };
  // The trip count is known up front, so every exit is a plain counter
  // test: no path from a step's end leads back to the loop head except the
  // real back edge (the compiler's own load-wait bookkeeping merges the
  // states of every edge into the head).
  const int trips = total / XS, rest = total - XS * trips;
  for (int it = 0; it < trips; ++it) {
    step(ic<0>());
    step(ic<1>());
    step(ic<2>());
    if constexpr (XS == 6) {
      step(ic<3 % XS>());
      step(ic<4 % XS>());
      step(ic<5 % XS>());
    }
  }
  if (rest > 0) step(ic<0>());
  if (rest > 1) step(ic<1>());
  if constexpr (XS == 6) {
    if (rest > 2) step(ic<2>());
    if (rest > 3) step(ic<3 % XS>());
    if (rest > 4) step(ic<4 % XS>());
  }
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
    hipLaunchKernelGGL((smfmac_i8p_kernel<NW, true, true>), dim3(grid), dim3(NW * 64), 0, s, a, mtiles, ntiles,
                       nwg_xcd);
  else if (a.ydt == NM_I8)
    hipLaunchKernelGGL((smfmac_i8p_kernel<NW, true>), dim3(grid), dim3(NW * 64), 0, s, a, mtiles, ntiles, nwg_xcd);
  else
    hipLaunchKernelGGL((smfmac_i8p_kernel<NW, false>), dim3(grid), dim3(NW * 64), 0, s, a, mtiles, ntiles, nwg_xcd);
  return hipGetLastError();
}

}  // namespace

// cfg 0: 4-wave workgroups (256 x 128 tiles, two per CU); cfg 1: 8-wave
// workgroups (512 x 128 tiles, one per CU)
hipError_t launch_spmm_smfmac_i8p(const SpmmArgs& a, int cfg, hipStream_t s) {
  return cfg == 1 ? launch_nw<8>(a, s) : launch_nw<4>(a, s);
}

}  // namespace nm
