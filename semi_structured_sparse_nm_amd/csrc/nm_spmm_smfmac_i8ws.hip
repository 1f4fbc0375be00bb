// Weight-stationary int8 2:4 sparse x dense product for K <= 768 on the
// gfx950 sparse matrix cores (v_smfmac_i32_16x16x128_i8), fused bias +
// requantisation epilogue.
//
// The kernel side of "Realizable N:M Sparse Transformer Inference via
// Search-Kernel Co-Design", Sec. 4.1 (micro-dense execution on the sparse
// matrix cores with inference-aware parallelism), arranged for MI355X:
//
// * One 8-wave workgroup per CU (two waves per SIMD, which hide each
//   other's LDS and dependency stalls).  A workgroup owns 512 rows (a row
//   tile, 64 rows per wave) and a contiguous run of 64-token steps.  Each
//   wave loads its rows' packed values and index words for all of K (six
//   128-column blocks, 120 registers) once and keeps them: per step only
//   the activations move.  That removes the weight re-reads that bound the
//   tile kernels (the same packed block read again for every token tile)
//   from the vector-memory path.
// * Activations of one step (K x 64 bytes, 48 KB) arrive by direct-to-LDS
//   loads into one of two stages while the other stage is multiplied; each
//   B fragment read (ds_read_b64_tr_b8) feeds four sparse products (the
//   wave's four row blocks).
// * Waits are whole drains (vmcnt 0) at two points per step: after the
//   step's products (the next stage, issued a whole step earlier, and the
//   previous step's output stores, issued a step earlier) and once in the
//   prologue; a barrier per step publishes every wave's part of a stage and
//   frees the other.  No count depends on the order in which loads complete.
// * Token steps: XCD x (dispatch is round-robin over 8 XCDs) covers steps
//   [x S / 8, (x + 1) S / 8) of every row tile, its workgroups split that
//   range per row tile, so an activation strip is read from HBM once per
//   XCD and shared by the row tiles through its L2.
//
// Operand mapping as in the tile kernels: the packed 16 x 128 block is the
// v_smfmac A operand byte for byte (16 kept values per lane, 2-bit positions
// in one index word).  A stage holds, per 128-column block, 128 rows (k) of
// 64 bytes (tokens); the 16-byte chunk c of row r sits at position
// c ^ f(r), f(r) = bit 2 of r | (bit 4 of r) << 1, which makes the transpose
// reads conflict-free: of the 32 lanes served together, the eight rows a
// lane group reads cover four rows mod 4 twice, at four distinct positions.
//
// Epilogue (int8 output): f32(acc) * scale[r] (one rounded product; the bias
// is the accumulator's start value), clamp to [-128, 127], add 1.5 * 2^23 so
// the low byte is the round-half-even int8; four rows per dword, staged
// token-major in the wave's LDS area and read back transposed so each lane
// stores 16 consecutive tokens of one row.  int32 output: acc stored as is.
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
smfmac_i8ws_kernel(SpmmArgs a, int mtiles, int nsteps, int nwg_xcd) {
  // device pass only (device-only types and builtins)
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ __attribute__((aligned(1024))) uint8_t xs0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ostage[OUT_I8 ? NW * 4096 : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t bsbuf[NW * 512];

  const Geometry& g = a.g;
  load_args_early(a);
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
  const v4i rx = make_rsrc(a.X, (int)(g.K * a.ldx));
  const v4i rz = zero_rsrc();
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values), 0, (int)g.values_bytes(), 0x00020000);
  const __amdgpu_buffer_rsrc_t rm =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.meta), 0, (int)g.meta_bytes(), 0x00020000);
  const v4i rbias = make_rsrc(a.bias, a.bias ? (int)(g.R * 4) : 0);
  const v4i rscale = make_rsrc(a.scale, a.scale ? (int)(g.R * 4) : 0);

  // ---- activation stage loads: block kb of step s holds X rows
  // 128 kb .. + 127, tokens 64 s .. + 63.  Load d (wave w issues d = w of
  // every block) fills rows 16 d .. 16 d + 15: lane l -> row 16 d + l / 4,
  // position l % 4, the source chunk whose swizzled position that is.  Rows
  // past K lie past the resource's range and read as zero (every wait here
  // is a full drain, so such loads need no special path).
  int xv;
  {
    const int row = 16 * wave + (lane >> 2);
    const int c = (lane & 3) ^ (((row >> 2) & 1) | ((row >> 3) & 2));
    xv = row * ldx + 16 * c;
  }
  // this wave's load of block kb
  auto issue_xb = [&](int step, uint8_t* sp, int kb) __attribute__((always_inline)) {
    lds_dma16(rx, lds_addr(sp + kb * BLK + wave * 1024), xv, kb * 128 * ldx + step * BN);
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

  // ---- B fragments: lane (i, g) of token tile tt reads rows kq + 16 g +
  // i / 2 (kq = 0, 8, 64, 72) of a block, tokens 16 tt + 8 (i & 1) .. + 7,
  // i.e. chunk tt at position tt ^ f(row) = tt ^ (i / 8) ^ 2 (g & 1)
  const int rbase = 64 * (16 * lg + (li >> 1)) + 8 * (li & 1);
  const int fsw = ((li >> 3) & 1) | ((lg & 1) << 1);
  auto bfrag = [&](const uint8_t* sp, int kb, int tt) __attribute__((always_inline)) -> v8i {
    const uint8_t* p = sp + kb * BLK + rbase + 16 * (tt ^ fsw);
    const v2i p0 = lds_tr8(p);
    const v2i p1 = lds_tr8(p + 8 * 64);
    const v2i p2 = lds_tr8(p + 64 * 64);
    const v2i p3 = lds_tr8(p + 72 * 64);
    return v8i{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
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

  // ---- int8 epilogue, in the wave's 4 KB staging area: 64 tokens x 64 row
  // positions; row 16 rb + 4 g + v of the wave is position 16 g + 4 rb + v,
  // so one lane's four row blocks of one token are 16 contiguous bytes;
  // chunk c of token t sits at c ^ f(t), f(t) = bit 2 of t | (bit 4 of t) << 1.
  uint8_t* const oh = ostage + (OUT_I8 ? wave * 4096 : 0);
  auto epilogue_i8 = [&](Acc& acc, int t0) __attribute__((always_inline)) {
    const float osc = a.out_scale;
    const float magic = 12582912.0f;          // 1.5 * 2^23
#pragma unroll
    for (int u = 0; u < TN; ++u) {
      uint32_t d[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
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
      const int wb = 64 * li + 16 * (lg ^ ((li >> 2) & 1) ^ ((u & 1) << 1));
      *reinterpret_cast<v4i*>(oh + 1024 * u + wb) = v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
    }
    // the wave reads back only what it wrote, after its staging writes have
    // completed; the area's next writes (a step later) come after these
    // reads have returned (the stores consume them).  Transpose reads: lane
    // 16 G + 2 i + h reads token 16 G + 8 e + i, chunk q ^ f, byte 8 h;
    // output lane l of group G then holds position 16 q + l, i.e. row
    // 16 (l >> 2) + 4 q + (l & 3), tokens 16 G + 8 e .. + 7
    __builtin_amdgcn_s_waitcnt(waitcnt(63, 0));
    const int i = (li >> 1) & 7, hb = li & 1;
    const int fq = ((i >> 2) & 1) | ((lg & 1) << 1);
    const int orow = 16 * (li >> 2) + (li & 3);
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy), 0x00020000);
    const int tok = t0 + 16 * lg;
    const bool tok_ok = tok < a.T;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rq = 1024 * lg + 64 * i + 16 * (q ^ fq) + 8 * hb;
      const v2i x0 = lds_tr8(oh + rq);
      const v2i x1 = lds_tr8(oh + rq + 512);
      const int row = r0 + 64 * wave + orow + 4 * q;
      const int off = tok_ok ? row * (int)a.ldy + tok : (int)(g.R * a.ldy);
      __builtin_amdgcn_raw_buffer_store_b128(v4i{x0[0], x0[1], x1[0], x1[1]}, ry, off, 0, kStreamStore);
    }
  };
  // int32 output: acc (bias included) stored directly
  auto store_i32 = [&](Acc& acc, int t0) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.Y, 0, (int)(g.R * a.ldy * 4), 0x00020000);
    const int rw = r0 + 64 * wave + 4 * lg;
    const int oob = (int)(g.R * a.ldy * 4);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
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
  hipLaunchKernelGGL((smfmac_i8ws_kernel<OUT_I8, ACT>), dim3(8 * nwg_xcd), dim3(NW * 64), 0, s, a, mtiles, nsteps,
                     nwg_xcd);
  return hipGetLastError();
}

}  // namespace

// K in (640, 768] (six column blocks); one workgroup per CU, so every XCD
// needs at least one per row tile (R <= 512 CUs / 8).
hipError_t launch_spmm_smfmac_i8ws(const SpmmArgs& a, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const int mtiles = (int)((a.g.R + BM - 1) / BM);
  const int nsteps = (int)((a.T + BN - 1) / BN);
  const int nwg_xcd = cu_count(dev) / 8;
  if (a.g.nKB != NKB || mtiles > nwg_xcd) return hipErrorInvalidValue;
  if (a.ydt == NM_I8 && a.act) return launch_cfg<true, true>(a, mtiles, nsteps, nwg_xcd, s);
  if (a.ydt == NM_I8) return launch_cfg<true, false>(a, mtiles, nsteps, nwg_xcd, s);
  return launch_cfg<false, false>(a, mtiles, nsteps, nwg_xcd, s);
}

}  // namespace nm
