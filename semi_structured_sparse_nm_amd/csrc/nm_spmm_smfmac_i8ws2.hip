// Weight-stationary int8 product for K <= 768 over a weight split into two
// 2:4 layers (launch_split24): any N:M pattern (3:4, 4:4, 4:8, 8:8, ...) on
// the gfx950 sparse matrix cores, two v_smfmac_i32_16x16x128_i8 per B
// fragment and row block instead of expanded dense products.  Fused bias +
// requantisation epilogue.
//
// "Realizable N:M Sparse Transformer Inference via Search-Kernel
// Co-Design", Sec. 4.1-4.2: the kernel multiplies only what the packed
// windows hold, arranged for the matrix instructions of the target.  On
// gfx950 a 2:4 sparse product covers 128 columns in one instruction; a
// group of four columns of any N:M weight holds at most four kept members,
// i.e. two 2:4 slots in each of two layers, so the weight is the exact sum
// of two 2:4 layers.  The dense int8 MFMA covers 64 columns per instruction
// at a lower measured rate, so two sparse products per 128 columns replace
// two dense ones and the per-lane expansion of the packed windows.
//
// Arrangement (the 2:4 weight-stationary kernel's, halved in rows):
// * One 8-wave workgroup per CU (two waves per SIMD) owns a 256-row tile,
//   32 rows (two row blocks) per wave, and a contiguous run of 64-token
//   steps.  Each wave holds both layers' packed values and index words of
//   its rows for all of K (six 128-column blocks, 120 registers); per step
//   only the activations move.
// * Work split: the G workgroups are spread over the row tiles as evenly as
//   whole workgroups allow (G / mtiles or one more per row tile), and a
//   row tile's workgroups split its steps evenly.  Work items are numbered
//   step range first (k, then row tile) and handed to the XCDs in
//   contiguous bands of G / 8, so the workgroups of one XCD cover the same
//   stretch of tokens for every row tile and share that activation strip
//   through the XCD's L2.
// * Activations of one step (K x 64 bytes, 48 KB) arrive by direct-to-LDS
//   loads into one of two stages while the other is multiplied; each B
//   fragment read (ds_read_b64_tr_b8) feeds four sparse products (two row
//   blocks x two layers).  A fragment's second-layer products are issued
//   after the next fragment's first-layer ones, so no product waits on the
//   accumulator the previous instruction writes.
// * Waits are whole drains (vmcnt 0): once per step after the products and
//   once in the prologue; a barrier per step publishes a stage and frees the
//   other.  No count depends on the order in which loads complete.
//
// Dense weights (N = M: 8:8, 4:4) need no split copy: every group of four
// holds its four columns, so the first layer is columns 0 and 1 of each
// group and the second columns 2 and 3, with the same index word for every
// lane (positions (0, 1) and (2, 3)).  The kernel loads the dense packed rows
// (32 bytes per lane and block) and sorts the bytes into the two layers with
// byte permutes in the first step, just before each block's first products.
//
// The PyTorch-linear layout (TK: X [T][K] with K contiguous, Y [T][R]) takes
// the stages, B-fragment reads and epilogue of the [T][K] weight-stationary
// kernel (nm_spmm_smfmac_i8wstk.hip): per block 64 tokens of 128 k bytes,
// token-major (chunk c of token t at c ^ (t & 7)), B fragments as two plain
// 16-byte reads, and token rows of the wave's 32 output rows staged so each
// lane stores 16 consecutive rows of one token (R a multiple of 16).
//
// Epilogue (int8 output): f32(acc) * scale[r] (one rounded product; the bias
// is the first layer's accumulator start), clamp, add 1.5 * 2^23 so the low
// byte is the round-half-even int8; the wave's two row blocks of one token
// are 8 contiguous staging bytes, read back transposed so each lane stores
// 16 consecutive tokens of one row.  int32 output: acc stored as is.
#include "nm_common.hpp"

namespace nm {

namespace {

constexpr int NW = 8;                  // waves per workgroup, two per SIMD
constexpr int RB = 2;                  // row blocks (16 rows) per wave
[[maybe_unused]] constexpr int NL = 2;                // 2:4 layers
constexpr int TN = 4;                  // 16-token tiles per step
constexpr int BM = NW * RB * 16;       // 256 rows per row tile
constexpr int BN = TN * 16;            // 64 tokens per step
constexpr int NKB = 6;                 // 128-column blocks held in registers (K <= 768)
constexpr int BLK = 128 * BN;          // bytes of one column block of a stage (8 KB)
[[maybe_unused]] constexpr int STAGE = NKB * BLK;   // 48 KB
[[maybe_unused]] constexpr int OST = 64 * RB * 16;    // int8 staging bytes per wave: 64 tokens x 32 rows

template <bool TK, bool DENSE, bool OUT_I8, bool ACT>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
smfmac_i8ws2_kernel(SpmmArgs a, int mtiles, int nsteps) {
  // device pass only (device-only types and builtins)
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) uint8_t xs0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ostage[OUT_I8 ? NW * OST : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t bsbuf[NW * 512];

  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int ldx = (int)a.ldx;
  const int nRB = (int)g.nRB;

  // ---- my work item: n in XCD-major order (dispatch is round-robin over
  // the 8 XCDs, so XCD x runs items x G / 8 .. (x + 1) G / 8 - 1); item n is
  // (step range k, row tile rt) in k-major order; row tile rt has cr
  // workgroups, range k of them covers steps k S / cr .. (k + 1) S / cr - 1
  const int G = (int)gridDim.x;
  const int n = (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8);
  const int base = G / mtiles, extra = G % mtiles;
  int rt, k;
  if (n < base * mtiles) {
    k = n / mtiles;
    rt = n % mtiles;
  } else {
    k = base;
    rt = n - base * mtiles;
  }
  const int cr = base + (rt < extra ? 1 : 0);
  const int sa = k * nsteps / cr, sb = (k + 1) * nsteps / cr;
  if (sa >= sb) return;
  const int r0 = rt * BM;
  const int rb0 = __builtin_amdgcn_readfirstlane(r0 / 16 + RB * wave);

  // ---- buffer resources (hardware range checks replace bounds tests)
  const v4i rx = make_rsrc(a.X, (int)((TK ? a.T : g.K) * a.ldx));
  const v4i rz = zero_rsrc();
  const __amdgpu_buffer_rsrc_t rv0 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values), 0, (int)g.values_bytes(), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm0 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.meta), 0, (int)g.meta_bytes(), 0x00020000);
  // (dense: the N = M packing, 2048 bytes per block; the meta resources unused)
  const __amdgpu_buffer_rsrc_t rv1 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(DENSE ? a.values : a.values2), 0, (int)g.values_bytes(), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm1 =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(DENSE ? a.meta : a.meta2), 0, DENSE ? 0 : (int)g.meta_bytes(), 0x00020000);
  const v4i rbias = make_rsrc(a.bias, a.bias ? (int)(g.R * 4) : 0);
  const v4i rscale = make_rsrc(a.scale, a.scale ? (int)(g.R * 4) : 0);

  // ---- activation stage loads: block kb of step s holds X rows
  // 128 kb .. + 127, tokens 64 s .. + 63.  Wave w's load of a block fills
  // rows 16 w .. 16 w + 15: lane l -> row 16 w + l / 4, position l % 4, the
  // source chunk whose swizzled position that is.  Rows past K lie past the
  // resource's range and read as zero (every wait is a full drain).
  // (TK: wave w's load of a block fills tokens 8 w .. 8 w + 7: lane l ->
  // token 8 w + l / 8, position l % 8, source chunk (l % 8) ^ (l / 8);
  // tokens past T read as zero)
  int xv;
  if constexpr (TK) {
    const int tok = 8 * wave + (lane >> 3);
    const int c = (lane & 7) ^ (lane >> 3);
    xv = tok * ldx + 16 * c;
  } else {
    const int row = 16 * wave + (lane >> 2);
    const int c = (lane & 3) ^ (((row >> 2) & 1) | ((row >> 3) & 2));
    xv = row * ldx + 16 * c;
  }
  auto issue_xb = [&](int step, uint8_t* sp, int kb) __attribute__((always_inline)) {
    lds_dma16(rx, lds_addr(sp + kb * BLK + wave * 1024), xv,
              TK ? step * BN * ldx + kb * 128 : kb * 128 * ldx + step * BN);
  };

  // ---- the wave's packed rows of both layers (lane (i, g): 16 bytes at row
  // i, offset 16 g of a block, index dword g of row i; row blocks past R
  // re-read the last one).  Column block 0 comes with the prologue, the
  // others in the first step after its next-stage loads.
  const int voff_v = li * 64 + lg * 16;
  const int voff_m = li * 16 + lg * 4;
  v4i av[NKB][NL][RB];
  int ai[NKB][NL][RB];
  auto load_a = [&](int kb, int l, int rb) __attribute__((always_inline)) {
    const int blk = __builtin_amdgcn_readfirstlane(min(rb0 + rb, nRB - 1) * NKB + kb);
    if constexpr (DENSE) {
      // lane (i, g): the 32 dense bytes of columns 32 g .. 32 g + 31 of row
      // i, the first 16 in the first layer's registers, the rest in the
      // second's, until dense_sort arranges them
      av[kb][l][rb] = __builtin_bit_cast(
          v4i, __builtin_amdgcn_raw_buffer_load_b128(rv0, li * 128 + lg * 32 + 16 * l, blk * 2048, 0));
      ai[kb][l][rb] = l ? (int)0xEEEEEEEE : 0x44444444;   // positions (2, 3) / (0, 1) in every group
    } else {
      av[kb][l][rb] =
          __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(l ? rv1 : rv0, voff_v, blk * 1024, 0));
      ai[kb][l][rb] = (int)__builtin_amdgcn_raw_buffer_load_b32(l ? rm1 : rm0, voff_m, blk * 256, 0);
    }
  };
  // dense: dword j of the 32 bytes is group j's four columns; the first
  // layer takes bytes 0 and 1 of each group, the second bytes 2 and 3
  auto dense_sort = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const v4i lo = av[kb][0][rb], hi = av[kb][1][rb];
      const uint32_t d[8] = {(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)lo[2], (uint32_t)lo[3],
                             (uint32_t)hi[0], (uint32_t)hi[1], (uint32_t)hi[2], (uint32_t)hi[3]};
      v4i f, sc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[j] = (int)__builtin_amdgcn_perm(d[2 * j + 1], d[2 * j], 0x05040100u);
        sc[j] = (int)__builtin_amdgcn_perm(d[2 * j + 1], d[2 * j], 0x07060302u);
      }
      av[kb][0][rb] = f;
      av[kb][1][rb] = sc;
    }
  };
#pragma unroll
  for (int l = 0; l < NL; ++l)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) load_a(0, l, rb);
  // bias and scale rows of the wave (64-row loads, the first 32 used; zeros
  // past R or when absent)
  uint8_t* const bsw = bsbuf + wave * 512;      // bias 256 B, then scale 256 B
  {
    const uint32_t bs = lds_addr(bsw);
    const int row0 = __builtin_amdgcn_readfirstlane(r0 + 16 * RB * wave);
    if (a.bias && row0 < (int)g.R)
      lds_dma4(rbias, bs, 4 * lane, 4 * row0);
    else
      lds_dma4(rz, bs, 4 * lane, 0);
    if (a.scale && row0 < (int)g.R)
      lds_dma4(rscale, bs + 256, 4 * lane, 4 * row0);
    else
      lds_dma4(rz, bs + 256, 4 * lane, 0);
  }
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) issue_xb(sa, xs0, kb);
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 15));
  auto bias_vec = [&](int rb) { return *reinterpret_cast<const v4i*>(bsw + 4 * (16 * rb + 4 * lg)); };
  auto scale_vec = [&](int rb) { return *reinterpret_cast<const v4f*>(bsw + 256 + 4 * (16 * rb + 4 * lg)); };

  // ---- B fragments: lane (i, g) of token tile tt reads rows kq + 16 g +
  // i / 2 (kq = 0, 8, 64, 72) of a block, tokens 16 tt + 8 (i & 1) .. + 7,
  // i.e. chunk tt at position tt ^ f(row) = tt ^ (i / 8) ^ 2 (g & 1)
  // (TK: chunks lg and 4 + lg of token 16 tt + li, positions chunk ^ (li &
  // 7); 16 tokens are 2048 bytes)
  const int rbase = 64 * (16 * lg + (li >> 1)) + 8 * (li & 1);
  const int fsw = ((li >> 3) & 1) | ((lg & 1) << 1);
  const int xb0 = 128 * li + 16 * (lg ^ (li & 7));
  const int xb1 = 128 * li + 16 * ((4 + lg) ^ (li & 7));
  auto bfrag = [&](const uint8_t* sp, int kb, int tt) __attribute__((always_inline)) -> v8i {
    if constexpr (TK) {
      const uint8_t* p = sp + kb * BLK + 2048 * tt;
      const v4i c0 = *reinterpret_cast<const v4i*>(p + xb0);
      const v4i c1 = *reinterpret_cast<const v4i*>(p + xb1);
      return v8i{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    } else {
      const uint8_t* p = sp + kb * BLK + rbase + 16 * (tt ^ fsw);
      const v2i p0 = lds_tr8(p);
      const v2i p1 = lds_tr8(p + 8 * 64);
      const v2i p2 = lds_tr8(p + 64 * 64);
      const v2i p3 = lds_tr8(p + 72 * 64);
      return v8i{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
    }
  };

  // acc = bias + A0 x B + A1 x B over the stage: the 24 (block, token tile)
  // fragments in order, each read one fragment ahead; fragment f's
  // first-layer products, then fragment f - 1's second-layer ones.  The
  // first-layer products of block 0 take the bias rows as their accumulator
  // input.  The wave's loads of the next stage (step nx into stage np, when
  // nx < sb) go between the products of the first six fragments.
  typedef v4i Acc[RB][TN];
  auto compute = [&](Acc& acc, const uint8_t* sp, int nx, uint8_t* np, bool spread, bool first) __attribute__((always_inline)) {
    constexpr int NF = NKB * TN;
    constexpr int NB = 3;              // fragments f + 1, f, f - 1
    v8i bf[NB];
    bf[0] = bfrag(sp, 0, 0);
    auto second = [&](int f) __attribute__((always_inline)) {
      const int kb = f / TN, tt = f % TN;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][tt] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(av[kb][1][rb], bf[f % NB], acc[rb][tt],
                                                              ai[kb][1][rb], 0, 0);
    };
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f + 1 < NF) bf[(f + 1) % NB] = bfrag(sp, (f + 1) / TN, (f + 1) % TN);
      const int kb = f / TN, tt = f % TN;
      if (DENSE && first && tt == 0) dense_sort(kb);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][tt] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(av[kb][0][rb], bf[f % NB],
                                                              kb == 0 ? bias_vec(rb) : acc[rb][tt], ai[kb][0][rb], 0, 0);
      if (f > 0) second(f - 1);
      if (f < NKB && nx < sb && spread) issue_xb(nx, np, f);
    }
    second(NF - 1);
  };

  // ---- int8 epilogue, in the wave's 2 KB staging area: 64 tokens x 32 row
  // positions; row 16 rb + 4 g + v of the wave is position 8 g + 4 rb + v,
  // so one lane's two row blocks of one token are 8 contiguous bytes; the
  // 16-byte chunk c of token t sits at c ^ f(t), f(t) = (bit 3 ^ bit 4) of
  // t, so that the 32 lanes served together touch distinct banks.
  uint8_t* const oh = ostage + (OUT_I8 ? wave * OST : 0);
  // TK: token rows of the wave's 32 rows (32 bytes each, 16 tokens per
  // token tile): the dword of rows 16 rb + 4 g .. + 3 of token t at byte
  // 16 (rb ^ f(t)) + 4 g, f(t) = bit 3 of t; each lane then reads one
  // 16-byte half (16 consecutive rows of one token) and stores it.
  auto epilogue_i8_tk = [&](Acc& acc, int t0) __attribute__((always_inline)) {
    const float osc = a.out_scale;
    const int sw = (li >> 3) & 1;
#pragma unroll
    for (int u = 0; u < TN; ++u) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const v4f sv = scale_vec(rb);
        float f[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          f[v] = __builtin_amdgcn_fmed3f(i8_pre<ACT>(acc[rb][u][v], sv[v], osc), -128.0f, 127.0f);
        *reinterpret_cast<uint32_t*>(oh + 512 * u + 32 * li + 16 * (rb ^ sw) + 4 * lg) =
            pack_rne_i8x4(f[0], f[1], f[2], f[3]);
      }
    }
    // the wave reads back only what it wrote, after its staging writes have
    // completed; the area's next writes (a step later) come after these
    // reads have returned (the stores consume them)
    __builtin_amdgcn_s_waitcnt(waitcnt(63, 0));
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(a.T * a.ldy), 0x00020000);
    const int oob = (int)(a.T * a.ldy);
    const int tl = (lane >> 1) & 15, h = lane & 1;   // token of the tile, half (rows 16 h ..)
    const int row = r0 + 16 * RB * wave + 16 * h;
#pragma unroll
    for (int q = 0; q < TN / 2; ++q) {
      const int u = 2 * q + (lane >> 5);
      const v4i piece = *reinterpret_cast<const v4i*>(oh + 512 * u + 32 * tl + 16 * (h ^ ((tl >> 3) & 1)));
      const int tok = t0 + 16 * u + tl;
      const int off = (tok < a.T && row < (int)g.R) ? tok * (int)a.ldy + row : oob;
      __builtin_amdgcn_raw_buffer_store_b128(piece, ry, off, 0, kStreamStore);
    }
  };
  // TK, int32 output: a lane's four rows of one token are 16 contiguous bytes
  auto store_i32_tk = [&](Acc& acc, int t0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(a.T * a.ldy * 4), 0x00020000);
    const int rw = r0 + 16 * RB * wave + 4 * lg;
    const int oob = (int)(a.T * a.ldy * 4);
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) {
        const int t = t0 + 16 * tt + li;
        const int row = rw + 16 * rr;
        __builtin_amdgcn_raw_buffer_store_b128(acc[rr][tt], ry,
                                               (t < a.T && row < (int)g.R) ? 4 * (t * (int)a.ldy + row) : oob, 0,
                                               kStreamStore);
      }
  };
  auto epilogue_i8 = [&](Acc& acc, int t0) __attribute__((always_inline)) {
    const float osc = a.out_scale;
    const float magic = 12582912.0f;          // 1.5 * 2^23
#pragma unroll
    for (int u = 0; u < TN; ++u) {
      uint32_t d[RB];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        const v4f sv = scale_vec(rr);
        float f[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          f[v] = __builtin_amdgcn_fmed3f(i8_pre<ACT>(acc[rr][u][v], sv[v], osc), -128.0f, 127.0f);
        rne_i8_byte<0>(d[rr], f[0], magic);
        rne_i8_byte<1>(d[rr], f[1], magic);
        rne_i8_byte<2>(d[rr], f[2], magic);
        rne_i8_byte<3>(d[rr], f[3], magic);
      }
      // token 16 u + li: chunk lg / 2, half lg & 1
      const int wb = 512 * u + 32 * li + 16 * ((lg >> 1) ^ (((li >> 3) ^ u) & 1)) + 8 * (lg & 1);
      *reinterpret_cast<v2i*>(oh + wb) = v2i{(int)d[0], (int)d[1]};
    }
    // the wave reads back only what it wrote, after its staging writes have
    // completed; the area's next writes (a step later) come after these
    // reads have returned (the stores consume them).  Transpose reads: lane
    // 16 G + 2 i + h reads token 16 G + 8 e + i, chunk q ^ f, byte 8 h;
    // output lane l of group G then holds position 16 q + l, i.e. row
    // 16 ((l >> 2) & 1) + 8 q + 4 (l >> 3) + (l & 3), tokens 16 G + 8 e .. + 7
    __builtin_amdgcn_s_waitcnt(waitcnt(63, 0));
    const int i = (li >> 1) & 7, hb = li & 1;
    const int orow = 16 * ((li >> 2) & 1) + 4 * (li >> 3) + (li & 3);
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy), 0x00020000);
    const int tok = t0 + 16 * lg;
    const bool tok_ok = tok < a.T;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      v2i x[2];
#pragma unroll
      for (int e = 0; e < 2; ++e)
        x[e] = lds_tr8(oh + 512 * lg + 256 * e + 32 * i + 16 * (q ^ ((e ^ lg) & 1)) + 8 * hb);
      const int row = r0 + 16 * RB * wave + orow + 8 * q;
      const int off = tok_ok ? row * (int)a.ldy + tok : (int)(g.R * a.ldy);
      __builtin_amdgcn_raw_buffer_store_b128(v4i{x[0][0], x[0][1], x[1][0], x[1][1]}, ry, off, 0, kStreamStore);
    }
  };
  // int32 output: acc (bias included) stored directly
  auto store_i32 = [&](Acc& acc, int t0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy * 4), 0x00020000);
    const int rw = r0 + 16 * RB * wave + 4 * lg;
    const int oob = (int)(g.R * a.ldy * 4);
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int tt = 0; tt < TN; ++tt) {
        const int t = t0 + 16 * tt + li;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          __builtin_amdgcn_raw_buffer_store_b32(
              acc[rr][tt][v], ry, t0 + 16 * tt < a.T ? 4 * ((rw + 16 * rr + v) * (int)a.ldy + t) : oob, 0,
              kStreamStore);
      }
  };
  auto finish = [&](Acc& acc, int t0) __attribute__((always_inline)) {
    if constexpr (TK && OUT_I8)
      epilogue_i8_tk(acc, t0);
    else if constexpr (TK)
      store_i32_tk(acc, t0);
    else if constexpr (OUT_I8)
      epilogue_i8(acc, t0);
    else
      store_i32(acc, t0);
  };

  // ---- steps.  Entering step s: this wave's part of its stage has landed
  // (the drain before the previous epilogue, or the prologue's); the barrier
  // makes every wave's part visible and guarantees that no wave still reads
  // the other stage, which this step's loads then fill.
  auto run_step = [&](auto stc, int s) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
    barrier_nofence();
    if constexpr (ST == 2) {
      // the first step: its next-stage loads, then the rest of the rows
      if (s + 1 < sb) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) issue_xb(s + 1, xs1, kb);
      }
#pragma unroll
      for (int kb = 1; kb < NKB; ++kb)
#pragma unroll
        for (int l = 0; l < NL; ++l)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) load_a(kb, l, rb);
    }
    Acc acc;
    compute(acc, ST == 1 ? xs1 : xs0, s + 1, ST == 1 ? xs0 : xs1, ST != 2, ST == 2);
    // the next stage (issued this step) and the previous step's stores:
    // nothing else is outstanding
    __builtin_amdgcn_s_waitcnt(waitcnt(0, 15));
    finish(acc, s * BN);
  };
  // stage of step s: xs0 for s - sa even, xs1 for odd (ic<2>: the first
  // step, in xs0)
  run_step(ic<2>(), sa);
  int s = sa + 1;
  for (; s + 1 < sb; s += 2) {
    run_step(ic<1>(), s);
    run_step(ic<0>(), s + 1);
  }
  if (s < sb) run_step(ic<1>(), s);
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
#endif
}

template <bool TK, bool DENSE, bool OUT_I8, bool ACT>
hipError_t launch_cfg(const SpmmArgs& a, int mtiles, int nsteps, int G, hipStream_t s) {
  hipLaunchKernelGGL((smfmac_i8ws2_kernel<TK, DENSE, OUT_I8, ACT>), dim3(G), dim3(NW * 64), 0, s, a, mtiles, nsteps);
  return hipGetLastError();
}

template <bool TK, bool DENSE>
hipError_t launch_out(const SpmmArgs& a, int mtiles, int nsteps, int G, hipStream_t s) {
  if (a.ydt == NM_I8 && a.act) return launch_cfg<TK, DENSE, true, true>(a, mtiles, nsteps, G, s);
  if (a.ydt == NM_I8) return launch_cfg<TK, DENSE, true, false>(a, mtiles, nsteps, G, s);
  return launch_cfg<TK, DENSE, false, false>(a, mtiles, nsteps, G, s);
}

template <bool DENSE>
hipError_t launch_dt(const SpmmArgs& a, int mtiles, int nsteps, int G, hipStream_t s) {
  // the [T][K] epilogue stores 16-row pieces: R a multiple of 16
  if (a.layout == NM_LAYOUT_TK)
    return a.g.R % 16 ? hipErrorInvalidValue : launch_out<true, DENSE>(a, mtiles, nsteps, G, s);
  return launch_out<false, DENSE>(a, mtiles, nsteps, G, s);
}

}  // namespace

// K in (640, 768] (six column blocks); one workgroup per CU (G of them, a
// multiple of 8), at most G row tiles of 256 rows.
hipError_t launch_spmm_smfmac_i8ws2(const SpmmArgs& a, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const int mtiles = (int)((a.g.R + BM - 1) / BM);
  const int nsteps = (int)((a.T + BN - 1) / BN);
  const int G = cu_count(dev) / 8 * 8;
  if (a.g.nKB != NKB || a.g.N != 2 || a.g.M != 4 || !a.values2 || !a.meta2 || G < 8 || mtiles > G)
    return hipErrorInvalidValue;
  return launch_dt<false>(a, mtiles, nsteps, G, s);
}

// a dense int8 weight (N = M) in its own packing, split in registers
hipError_t launch_spmm_smfmac_i8ws2_dense(const SpmmArgs& a, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const int mtiles = (int)((a.g.R + BM - 1) / BM);
  const int nsteps = (int)((a.T + BN - 1) / BN);
  const int G = cu_count(dev) / 8 * 8;
  if (a.wdt != NM_I8 || a.g.N != a.g.M || a.g.nKB != NKB || a.g.vblk != 2048 || G < 8 || mtiles > G)
    return hipErrorInvalidValue;
  return launch_dt<true>(a, mtiles, nsteps, G, s);
}

}  // namespace nm
