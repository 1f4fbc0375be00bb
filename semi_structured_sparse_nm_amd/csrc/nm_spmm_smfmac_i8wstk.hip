// Weight-stationary int8 2:4 sparse x dense product for K <= 768 in the
// PyTorch-linear layout: Yt [T][R] = epilogue(Xt [T][K] . (mask (.) W)^T),
// on the gfx950 sparse matrix cores (v_smfmac_i32_16x16x128_i8), fused
// bias + requantisation epilogue.
//
// The [K][T] weight-stationary kernel (nm_spmm_smfmac_i8ws.hip) in the
// operand layout a Transformer keeps its activations in ("Realizable N:M
// Sparse Transformer Inference via Search-Kernel Co-Design", Sec. 1: the
// linear layers of each block are where the time goes; Sec. 4.1: micro-dense
// execution with inference-aware parallelism).  Workgroups, row tiles, token
// steps, the packed rows held in registers, the two activation stages, the
// waits and the barriers are that kernel's.  What the layout changes:
//
// * Activation stage, per 128-column block: 64 tokens of 128 k bytes,
//   token-major (a token's k run is one 128-byte LDS row); the 16-byte chunk
//   c of token t sits at position c ^ (t & 7).  Wave w's load of a block
//   fills tokens 8 w .. 8 w + 7: lane l -> token 8 w + l / 8, position l % 8,
//   source chunk (l % 8) ^ (l / 8).  Tokens past T lie past the resource's
//   range and read as zero; a token row's bytes past K meet packed values
//   that are zero past K.
// * B operand: lane (token j, group g) takes k = 16 g .. 16 g + 15 and
//   64 + 16 g .. 64 + 16 g + 15 of token j, chunks g and 4 + g of its row:
//   two plain 16-byte reads instead of four transpose reads.  For a fixed g
//   the eight tokens of a half lane group sit at eight distinct positions,
//   so the reads are conflict-free.
// * Epilogue (int8 output): the four rows a lane holds for one token
//   (16 rb + 4 g + v) are requantised and packed into a dword per row block,
//   written to the wave's LDS area as token rows of 64 row bytes (the dword
//   of row block rb at 16 (rb ^ ((t >> 2) & 3)) + 4 g), then read back 16
//   bytes at a time, so each lane stores 16 consecutive rows of one token;
//   R a multiple of 16 keeps every piece inside its token's row, and pieces
//   of rows past R are dropped (in this layout they would land inside the
//   token's row).  int32 output: a lane's four rows of a token are 16
//   contiguous bytes, stored directly.
#include "nm_common.hpp"

namespace nm {

namespace {

constexpr int NW = 8;                  // waves per workgroup, two per SIMD
constexpr int RB = 4;                  // row blocks (16 rows) per wave
constexpr int TN = 4;                  // 16-token tiles per step
constexpr int BM = NW * RB * 16;       // 512 rows per row tile
constexpr int BN = TN * 16;            // 64 tokens per step
constexpr int NKB = 6;                 // 128-column blocks held in registers (K <= 768)
constexpr int BLK = 128 * BN;          // bytes of one column block of a stage (8 KB)
constexpr int STAGE = NKB * BLK;       // 48 KB

template <bool OUT_I8, bool ACT>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
smfmac_i8wstk_kernel(SpmmArgs a, int mtiles, int nsteps, int nwg_xcd) {
  // device pass only (device-only types and builtins)
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) uint8_t xs0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ostage[OUT_I8 ? NW * 4096 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t bsbuf[NW * 512];

  const Geometry& g = a.g;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int ldx = (int)a.ldx;
  const int nRB = (int)g.nRB;

  // ---- my row tile and token steps.  Workgroup j of XCD x takes row tile
  // j mod mtiles; the cr workgroups of that row tile on this XCD split the
  // XCD's steps evenly (the host guarantees nwg_xcd >= mtiles).
  const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
  const int rt = j % mtiles, ir = j / mtiles;
  const int cr = (nwg_xcd - rt + mtiles - 1) / mtiles;
  const int sx0 = xcd * nsteps / 8, nsx = (xcd + 1) * nsteps / 8 - sx0;
  const int sa = sx0 + ir * nsx / cr, sb = sx0 + (ir + 1) * nsx / cr;
  if (sa >= sb) return;
  const int r0 = rt * BM;
  const int rb0 = __builtin_amdgcn_readfirstlane(r0 / 16 + RB * wave);

  // ---- buffer resources (hardware range checks replace bounds tests)
  const v4i rx = make_rsrc(a.X, (int)(a.T * a.ldx));
  const v4i rz = zero_rsrc();
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values), 0, (int)g.values_bytes(), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.meta), 0, (int)g.meta_bytes(), 0x00020000);
  const v4i rbias = make_rsrc(a.bias, a.bias ? (int)(g.R * 4) : 0);
  const v4i rscale = make_rsrc(a.scale, a.scale ? (int)(g.R * 4) : 0);

  // ---- activation stage loads: block kb of step s holds tokens 64 s ..
  // + 63, k 128 kb .. + 127 (every wait here is a full drain, so loads past
  // T need no special path)
  int xv;
  {
    const int tok = 8 * wave + (lane >> 3);
    const int c = (lane & 7) ^ (lane >> 3);
    xv = tok * ldx + 16 * c;
  }
  // this wave's load of block kb
  auto issue_xb = [&](int step, uint8_t* sp, int kb) __attribute__((always_inline)) {
    lds_dma16(rx, lds_addr(sp + kb * BLK + wave * 1024), xv, step * BN * ldx + kb * 128);
  };

  // ---- the wave's packed rows (lane (i, g): 16 bytes at row i, offset
  // 16 g of a block, meta dword g of row i; row blocks past R re-read the
  // last one).  Column block 0 comes with the prologue; the first step
  // issues its next-stage loads and then the other blocks' rows, so each
  // block's products wait only for that block (the compiler counts the
  // register loads issued after it, and the earlier direct-to-LDS loads
  // can only make such a wait stricter).
  const int voff_v = li * 64 + lg * 16;
  const int voff_m = li * 16 + lg * 4;
  v4i av[NKB][RB];
  int ai[NKB][RB];
  auto load_a = [&](int kb, int rb) __attribute__((always_inline)) {
    const int blk = __builtin_amdgcn_readfirstlane(min(rb0 + rb, nRB - 1) * NKB + kb);
    av[kb][rb] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rv, voff_v, blk * 1024, 0));
    ai[kb][rb] = (int)__builtin_amdgcn_raw_buffer_load_b32(rm, voff_m, blk * 256, 0);
  };
  // prologue: block 0 of the rows, the bias and scale rows (zeros past R or
  // when absent) and the first stage
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) load_a(0, rb);
  uint8_t* const bsw = bsbuf + wave * 512;      // bias 256 B, then scale 256 B
  {
    const uint32_t bs = lds_addr(bsw);
    const int row0 = __builtin_amdgcn_readfirstlane(r0 + 64 * wave);
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

  // ---- B fragments: token tile tt, block kb: chunks lg and 4 + lg of
  // token 16 tt + li (positions chunk ^ (li & 7)); 16 tokens are 2048 bytes
  const int xb0 = 128 * li + 16 * (lg ^ (li & 7));
  const int xb1 = 128 * li + 16 * ((4 + lg) ^ (li & 7));
  auto bfrag = [&](const uint8_t* sp, int kb, int tt) __attribute__((always_inline)) -> v8i {
    const uint8_t* p = sp + kb * BLK + 2048 * tt;
    const v4i c0 = *reinterpret_cast<const v4i*>(p + xb0);
    const v4i c1 = *reinterpret_cast<const v4i*>(p + xb1);
    return v8i{c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
  };

  // acc = bias + A x B over the stage: the 24 (block, token tile) fragments
  // in order, each read PF fragments ahead of its products; the products of
  // block 0 take the bias rows as their accumulator input.  The wave's loads
  // of the next stage (step nx into stage np, when nx < sb) are issued
  // between the products of the first six fragments, one each.
  typedef v4i Acc[RB][TN];
  auto compute = [&](Acc& acc, const uint8_t* sp, int nx, uint8_t* np, bool spread) __attribute__((always_inline)) {
    constexpr int NF = NKB * TN;
    constexpr int PF = 1;
    v8i bf[PF + 1];
#pragma unroll
    for (int f = 0; f < PF; ++f) bf[f] = bfrag(sp, f / TN, f % TN);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f + PF < NF) bf[(f + PF) % (PF + 1)] = bfrag(sp, (f + PF) / TN, (f + PF) % TN);
      const int kb = f / TN, tt = f % TN;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        acc[rb][tt] = __builtin_amdgcn_smfmac_i32_16x16x128_i8(av[kb][rb], bf[f % (PF + 1)],
                                                              kb == 0 ? bias_vec(rb) : acc[rb][tt], ai[kb][rb], 0, 0);
      if (f < NKB && nx < sb && spread) issue_xb(nx, np, f);
    }
  };

  // ---- int8 epilogue, in the wave's 4 KB staging area: four token tiles
  // of 16 token rows x 64 row bytes; row 16 rb + 4 g + v of token t at byte
  // 16 (rb ^ ((t >> 2) & 3)) + 4 g + v of its row.
  uint8_t* const oh = ostage + (OUT_I8 ? wave * 4096 : 0);
  auto epilogue_i8 = [&](Acc& acc, int t0) __attribute__((always_inline)) {
    const float osc = a.out_scale;
    const int sw = (li >> 2) & 3;
    const int wr = 64 * li + 4 * lg;                 // + 16 (rb ^ sw): this lane's dwords
    const int rd = 64 * li + 16 * (lg ^ sw);         // this lane's 16-byte piece: rows 16 lg ..
#pragma unroll
    for (int u = 0; u < TN; ++u) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const v4f sv = scale_vec(rb);
        float f[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
          f[v] = __builtin_amdgcn_fmed3f(i8_pre<ACT>(acc[rb][u][v], sv[v], osc), -128.0f, 127.0f);
        *reinterpret_cast<uint32_t*>(oh + 1024 * u + wr + 16 * (rb ^ sw)) = pack_rne_i8x4(f[0], f[1], f[2], f[3]);
      }
    }
    // the wave reads back only what it wrote, after its staging writes have
    // completed; the area's next writes (a step later) come after these
    // reads have returned (the stores consume them)
    __builtin_amdgcn_s_waitcnt(waitcnt(63, 0));
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(a.T * a.ldy), 0x00020000);
    const int oob = (int)(a.T * a.ldy);
    const int row = r0 + 64 * wave + 16 * lg;
#pragma unroll
    for (int u = 0; u < TN; ++u) {
      const v4i piece = *reinterpret_cast<const v4i*>(oh + 1024 * u + rd);
      const int tok = t0 + 16 * u + li;
      const int off = (tok < a.T && row < (int)g.R) ? tok * (int)a.ldy + row : oob;
      __builtin_amdgcn_raw_buffer_store_b128(piece, ry, off, 0, kStreamStore);
    }
  };
  // int32 output: a lane's four rows of one token are 16 contiguous bytes
  auto store_i32 = [&](Acc& acc, int t0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(a.T * a.ldy * 4), 0x00020000);
    const int rw = r0 + 64 * wave + 4 * lg;
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
  auto finish = [&](Acc& acc, int t0) __attribute__((always_inline)) {
    if constexpr (OUT_I8)
      epilogue_i8(acc, t0);
    else
      store_i32(acc, t0);
  };

  // ---- steps.  Entering step s (stage s & 1 relative to sa): this wave's
  // part of the stage has landed (the drain before the previous epilogue, or
  // the prologue's); the barrier makes every wave's part visible and
  // guarantees that no wave still reads the other stage, which the next
  // step's loads then fill.
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
        for (int rb = 0; rb < RB; ++rb) load_a(kb, rb);
    }
    Acc acc;
    compute(acc, ST == 1 ? xs1 : xs0, s + 1, ST == 1 ? xs0 : xs1, ST != 2);
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

template <bool OUT_I8, bool ACT>
hipError_t launch_cfg(const SpmmArgs& a, int mtiles, int nsteps, int nwg_xcd, hipStream_t s) {
  hipLaunchKernelGGL((smfmac_i8wstk_kernel<OUT_I8, ACT>), dim3(8 * nwg_xcd), dim3(NW * 64), 0, s, a, mtiles, nsteps,
                     nwg_xcd);
  return hipGetLastError();
}

}  // namespace

// K in (640, 768] (six column blocks); one workgroup per CU, so every XCD
// needs at least one per row tile (R <= 512 CUs / 8).
hipError_t launch_spmm_smfmac_i8wstk(const SpmmArgs& a, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const int mtiles = (int)((a.g.R + BM - 1) / BM);
  const int nsteps = (int)((a.T + BN - 1) / BN);
  const int nwg_xcd = cu_count(dev) / 8;
  if (a.g.nKB != NKB || mtiles > nwg_xcd || a.g.R % 16 != 0) return hipErrorInvalidValue;
  if (a.ydt == NM_I8 && a.act) return launch_cfg<true, true>(a, mtiles, nsteps, nwg_xcd, s);
  if (a.ydt == NM_I8) return launch_cfg<true, false>(a, mtiles, nsteps, nwg_xcd, s);
  return launch_cfg<false, false>(a, mtiles, nsteps, nwg_xcd, s);
}

}  // namespace nm
