// Product of a weight in the three-layer format (Sparse-TC 2:4 layer,
// Slot-Filling layer with 4-bit PDD distances, CSR residual; format at
// nm_hybrid in nm_sparse.h) with an fp16 / bf16 activation, for inference
// shapes with few tokens (page "Accelerating GPU Inference of Large Language
// Models with Moderately Unstructured Sparse Weight Matrices", Methodology 2:
// the vector units decode the PDD codes, the sparse matrix cores run the 2:4
// layer, the residual goes to a separate buffer added at the end, and loads
// overlap decode and product).
//
// Schedule.  A workgroup of four waves (one per SIMD) takes row blocks
// b, b + G, ... and walks K in chunks of four 512-column segments; the chunk's
// activation columns (16 tokens) sit in LDS, one segment per wave (staged and
// read by that wave only), in the layout the transposing reads want.  Work
// item of a wave = (row block, its segment of the chunk) = 64 fill units, one
// per lane: lane (row li, quad lg)
// holds exactly the A-operand part of its unit.  The item's Sparse-TC values,
// positions and codes are loaded to registers while the wave decodes and
// multiplies the previous item; the residual entries of the next item are
// staged the same way.
//
// Decode of a unit (per lane, no cross-lane traffic): empty slots are the
// position pairs a group with two nonzeros never has (equal: slot 1 empty;
// descending: both empty).  The unit's codes, read in order, give the local
// column of each slot-filled element; the k-th real point takes the value of
// the k-th empty slot (a per-lane 128-byte copy of the values in LDS, laid
// out without bank conflicts, gives random access to it; each slot read is
// cleared in the copy, which then reads back as the Sparse-TC operand with
// every empty slot zero).  The elements are scattered into a second 2:4
// operand of the same groups (value, position) in a zeroed LDS area and read
// back as registers.  Each 64-column block then takes two sparse matrix
// instructions on the same B fragment.  An element's group holds at most two surplus elements, so the
// second operand is a valid 2:4 operand; a single one sits in slot 0 with a
// zero partner at the same position.
//
// Residual: lane l takes row l / 4 and tokens 4 (l % 4) .. + 3 of the item,
// walks that row's CSR entries (staged in LDS, four at a time) and multiplies
// with the activation values already in LDS.
//
// Partial sums per (wave, row block): a 16 x 16 fp32 tile in LDS.  Each item
// adds its matrix products, then its residual sums (held apart in registers
// until then); at the end the four waves' tiles are added in wave order (a
// fixed order: results do not depend on timing).
#include "nm_hybrid.hpp"

namespace nm {

namespace {

typedef _Float16 v16h __attribute__((ext_vector_type(16)));
typedef __bf16 v16bf __attribute__((ext_vector_type(16)));

template <int WT>
__device__ __forceinline__ v4f smfmac(v4i a, v8i b, v4f c, int idx) {
  if constexpr (WT == NM_F16)
    return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v16h, b), c,
                                                    idx, 0, 0);
  else
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v16bf, b), c,
                                                     idx, 0, 0);
}

template <int WT>
__device__ __forceinline__ float to_f32(uint32_t h) {
  if constexpr (WT == NM_F16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  else
    return __builtin_bit_cast(float, h << 16);
}

constexpr int SEGB = 8;        // column blocks per segment
constexpr int RESCAP = 256;    // residual entries staged per item (more are read from memory)

// Waves, row blocks per workgroup and the LDS map (bytes).  The three-layer
// form: four waves (one per SIMD), with per-lane decode areas.  The plain
// 2:4 form needs none of those: eight waves (two per SIMD) and twice the
// activation chunk.
template <bool HY>
struct Lay {
  static constexpr int NW = kHybridWaves[HY];                    // waves = segments per chunk
  static constexpr int MAXRB = kHybridMaxRB[HY];
  static constexpr int XS_OFF = 0;                               // X chunk: NW segments x 8 blocks x 2 KB
  static constexpr int STG_OFF = XS_OFF + NW * SEGB * 2048;      // per lane 128 B: the Sparse-TC values
  static constexpr int STG2_OFF = STG_OFF + (HY ? NW * 64 * 128 : 0);   // per lane 128 B: second operand
  static constexpr int IDX_OFF = STG2_OFF + (HY ? NW * 64 * 128 : 0);   // per lane 32 B: its positions
  static constexpr int PART_OFF = IDX_OFF + (HY ? NW * 64 * 32 : 0);    // per wave, row block: 1 KB partials
  static constexpr int RES_OFF = PART_OFF + NW * MAXRB * 1024;   // per wave: RESCAP residual entries
  static constexpr int BYTES = RES_OFF + (HY ? NW * RESCAP * 4 : 0);
  static_assert(BYTES <= 160 * 1024, "LDS");
};

// One item's register-resident loads.
struct Item {
  v4i a[SEGB];      // Sparse-TC values of the lane's quad in each block
  int m[SEGB];      // the quad's 16-bit positions word (in the low half)
  int c0, c1;       // the unit's sixteen codes
};

__device__ __forceinline__ int ctz_u32(uint32_t x) { return __builtin_ctz(x); }

// The decode areas are written and read as 8-, 16- and 32-bit words; these
// types tell the compiler that such accesses alias (so it keeps their order).
typedef uint32_t __attribute__((may_alias)) u32a;
typedef uint16_t __attribute__((may_alias)) u16a;
typedef uint8_t __attribute__((may_alias)) u8a;

template <int WT, int OUT, bool HY>
__global__ void __launch_bounds__(Lay<HY>::NW * 64) hybrid_kernel(HybridArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef Lay<HY> L;
  constexpr int NW = L::NW, MAXRB = L::MAXRB;
  constexpr int XS_OFF = L::XS_OFF, STG_OFF = L::STG_OFF, STG2_OFF = L::STG2_OFF, IDX_OFF = L::IDX_OFF,
                PART_OFF = L::PART_OFF, RES_OFF = L::RES_OFF;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[L::BYTES];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int b = blockIdx.x;
  const int ty = blockIdx.y;                       // 16-token tile
  const int G = a.G;
  const int nKB = (int)a.nKB, nSeg = (int)a.nSeg;
  const int ni = __builtin_amdgcn_readfirstlane((int)((a.nRB - 1 - b) / G) + 1);   // row blocks of this workgroup
  const int nItems = ni * a.nChunk;
  const int ldx = (int)a.ldx;

  // The weight buffers are read with plain global loads: every offset below
  // lies inside its buffer by construction (blocks clamped to the last one,
  // items to the wave's last item, residual entries to the last entry), and
  // a buffer descriptor would hold four scalar registers each.
  const uint8_t* const gv = a.values;
  const uint8_t* const gm = a.meta;
  const uint8_t* const gc = a.codes;
  const int32_t* const gp = a.res_ptr;
  const uint32_t* const ge = a.res_ent;
  const v4i rx = make_rsrc(a.X, (int)(a.K * a.ldx * 2));

  // per-lane decode areas, interleaved by dword (lane l's dword d at
  // (64 d + l) * 4): a wave's accesses to them hit 64 distinct banks whatever
  // slot each lane addresses
  u32a* const stg = reinterpret_cast<u32a*>(lds + STG_OFF + w * 64 * 128) + lane;   // 32 dwords
  u32a* const stg2 = reinterpret_cast<u32a*>(lds + STG2_OFF + w * 64 * 128) + lane; // 32 dwords
  u32a* const idxs = reinterpret_cast<u32a*>(lds + IDX_OFF + w * 64 * 32) + lane;   // 8 dwords
  // byte b of a lane's interleaved area
  auto stg_b = [&](u32a* base, int b) { return reinterpret_cast<u8a*>(base + 64 * (b >> 2)) + (b & 3); };
  uint8_t* const xseg = lds + XS_OFF + w * SEGB * 2048;     // this wave's segment of the chunk
  uint8_t* const part = lds + PART_OFF + w * MAXRB * 1024;
  uint32_t* const rstage = reinterpret_cast<uint32_t*>(lds + RES_OFF + w * RESCAP * 4);

  // partial sums and the second operand's staging start at zero (the
  // staging is cleared again after each use)
  for (int i = lane; i < MAXRB * 256; i += 64) reinterpret_cast<float*>(part)[i] = 0.f;
  if constexpr (HY) {
#pragma unroll
    for (int d = 0; d < 4 * SEGB; ++d) stg2[64 * d] = 0u;
#pragma unroll
    for (int d = 0; d < SEGB; ++d) idxs[64 * d] = 0u;
  }

  // item j: chunk j / ni, row block b + (j % ni) G, segment 4 (j / ni) + w
  auto seg_of = [&](int j) { return NW * (j / ni) + w; };
  auto rb_of = [&](int j) { return b + (j % ni) * G; };

  auto load_item = [&](int j, Item& it) {
    const int s = seg_of(j), rb = rb_of(j);
#pragma unroll
    for (int bi = 0; bi < SEGB; ++bi) {
      const int kb = min(s * SEGB + bi, nKB - 1);            // past the segment: a valid block, unused
      const int blk = rb * nKB + kb;
      it.a[bi] = *reinterpret_cast<const v4i*>(gv + (uint32_t)(blk * 1024 + li * 64 + lg * 16));
      it.m[bi] = *reinterpret_cast<const int*>(gm + (uint32_t)(blk * 128 + li * 8 + (lg >> 1) * 4));
    }
    if constexpr (HY) {
      const v2i c = *reinterpret_cast<const v2i*>(gc + (uint32_t)((rb * nSeg + s) * 512 + lane * 8));
      it.c0 = c[0];
      it.c1 = c[1];
    }
  };
  // lane x <= 16 holds res_ptr[(rb nSeg + s) 16 + x]
  auto load_rp = [&](int j) -> int {
    const int s = seg_of(j), rb = rb_of(j);
    return gp[(uint32_t)((rb * nSeg + s) * 16 + min(lane, 16))];
  };
  // every load below is issued whatever the item (clamped to data inside
  // its buffer): the compiler's waits count loads in issue order, which
  // holds only if each path through the loop issues the same loads
  const int n_ent = (int)(a.res_ent_bytes / 4);
  // (entries past the item's own are loaded too and never read)
  auto load_ent = [&](int rpv, uint32_t (&e)[4]) {
    const int r0 = __builtin_amdgcn_readlane(rpv, 0);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      e[m] = ge[(uint32_t)min(r0 + lane + 64 * m, n_ent - 1)];
  };

  // activation chunk c: segment NW c + w's 8 blocks, rows 64 kb .. + 63 of
  // tokens 16 ty .. + 15, row r of a block at 32 r with its two 16-byte
  // halves swapped when (r >> 3) & 1 (the transposing reads' bank layout)
  int xoff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 32 * j + (lane >> 1);
    xoff[j] = r * ldx * 2 + 16 * ((lane & 1) ^ ((r >> 3) & 1));
  }
  auto load_x = [&](int c) {
    const int s = NW * c + w;
    if (s >= nSeg) return;
#pragma unroll
    for (int bi = 0; bi < SEGB; ++bi) {
      const int kb = s * SEGB + bi;
      if (kb >= nKB) break;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        lds_dma16(rx, lds_addr(xseg + bi * 2048 + 1024 * j), xoff[j], (kb * 64 * ldx + 16 * ty) * 2);
    }
  };

  // B fragment reads (as the fp16 decode kernel): source lane 4 e + q of
  // group g reads row 8 g + e (+4, +32, +36), tokens 4 q .. + 3
  const int e_s = li >> 2, q_s = li & 3;
  const int bbase = (8 * lg + e_s) * 32 + 16 * ((q_s >> 1) ^ (lg & 1)) + 8 * (q_s & 1);
  const int ishift = 16 * (lg & 1);

  // this wave's items with a segment: chunks c with NW c + w < nSeg
  const int nValid = w < nSeg ? ni * ((nSeg - 1 - w) / NW + 1) : 0;
  const int jlast = max(nValid - 1, 0);
  Item cur, nxt;
  uint32_t ent_cur[4] = {0u, 0u, 0u, 0u}, ent_nxt[4] = {0u, 0u, 0u, 0u};
  int rp_cur = 0, rp_n1 = 0, rp_n2 = 0;
  // a wave without a segment in any chunk has no work (the loop holds no
  // barrier): skipping the loop keeps every load inside it unconditional
  if (nValid > 0) {
  load_item(0, cur);
  if constexpr (HY) {
    rp_cur = load_rp(0);
    load_ent(rp_cur, ent_cur);
    rp_n1 = load_rp(min(1, jlast));
  }

  auto step = [&](int j, auto pf) {
    constexpr bool PF = decltype(pf)::value != 0;
    const int i = j % ni;
    const int s = seg_of(j);
    if (i == 0) {
      // a new chunk: each wave stages and reads only its own segment's
      // activation columns, so no barrier; the previous chunk's reads have
      // all returned (their results were consumed)
      load_x(j / ni);
      __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
      if (a.patch_last) {
        // the last activation element, alone: its 16-byte piece ends past X
        const int kk = (int)a.K - 1, tl = (int)a.T - 1;
        if (s == kk / (SEGB * 64) && ty == tl / 16 && lane == 0) {
          const uint16_t v = __builtin_amdgcn_raw_buffer_load_b16(
              __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.X), 0, (int)(a.K * a.ldx * 2), 0x00020000),
              0, (kk * ldx + tl) * 2, 0);
          const int r = kk & 63, bi = (kk >> 6) & (SEGB - 1), h = (tl & 15) >> 3;
          *reinterpret_cast<uint16_t*>(xseg + bi * 2048 + r * 32 + 16 * (h ^ ((r >> 3) & 1)) + 2 * (tl & 7)) = v;
        }
      }
    }
    // next item's loads overlap this one's decode and product (the last
    // item, run without them, issues none)
    if constexpr (PF) {
      load_item(j + 1, nxt);
      if constexpr (HY) {
        load_ent(rp_n1, ent_nxt);
        rp_n2 = load_rp(min(j + 2, jlast));
      }
    }

    {
      const int nb = min(SEGB, nKB - s * SEGB);
      v4i a1[SEGB], a2[SEGB];
      int i1[SEGB], i2[SEGB];
#pragma unroll
      for (int bi = 0; bi < SEGB; ++bi) {
        a1[bi] = cur.a[bi];
        i1[bi] = (int)(((uint32_t)cur.m[bi] >> ishift) & 0xFFFFu);
      }
      if constexpr (HY) {
        // empty slots: bit sigma = 8 bi + 2 t + j
        uint32_t e8[SEGB];
#pragma unroll
        for (int bi = 0; bi < SEGB; ++bi) {
          const uint32_t mm = (uint32_t)i1[bi];
          const uint32_t p0 = mm & 0x3333u, p1 = (mm >> 2) & 0x3333u;
          const uint32_t ge = (((p0 | 0x4444u) - p1) & 0x4444u) >> 2;   // bit 4t: i0 >= i1
          const uint32_t x = p0 ^ p1;
          const uint32_t gt = ge & (x | (x >> 1)) & 0x1111u;             // bit 4t: i0 > i1
          uint32_t e = gt | (ge << 1);
          e = (e & 0x3u) | ((e >> 2) & 0xCu) | ((e >> 4) & 0x30u) | ((e >> 6) & 0xC0u);
          e8[bi] = bi < nb ? e : 0u;
        }
        const uint32_t elo = e8[0] | (e8[1] << 8) | (e8[2] << 16) | (e8[3] << 24);
        const uint32_t ehi = e8[4] | (e8[5] << 8) | (e8[6] << 16) | (e8[7] << 24);
        // the values as loaded (slot-filled ones included), for random access
#pragma unroll
        for (int bi = 0; bi < SEGB; ++bi)
#pragma unroll
          for (int t = 0; t < 4; ++t) stg[64 * (4 * bi + t)] = (uint32_t)a1[bi][t];
        // PDD decode: the k-th real point takes the k-th empty slot's value;
        // that slot is then cleared in the copy (LDS runs a wave's accesses
        // in order, so the clear lands after the read)
        uint32_t lv[16];
        int lu[16];
        uint32_t clo = elo, chi = ehi;
        int pos = -1;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int code = ((k < 8 ? cur.c0 : cur.c1) >> (4 * (k & 7))) & 15;
          const bool real = code != 0;
          pos += real ? code : 15;
          const int sg = clo ? ctz_u32(clo) : 32 + ctz_u32(chi | 0x80000000u);
          const uint32_t clo2 = clo & (clo - 1u), chi2 = clo ? chi : (chi & (chi - 1u));
          clo = real ? clo2 : clo;
          chi = real ? chi2 : chi;
          u16a* const sp = reinterpret_cast<u16a*>(stg_b(stg, 2 * (sg & 63)));
          lv[k] = *sp;
          if (real) *sp = 0;
          lu[k] = (real && pos < 16 * nb) ? pos : -1;
        }
        // every empty slot is now zero or was zero: the Sparse-TC operand
        // without the slot-filled elements
#pragma unroll
        for (int bi = 0; bi < SEGB; ++bi)
#pragma unroll
          for (int t = 0; t < 4; ++t) a1[bi][t] = (int)stg[64 * (4 * bi + t)];
        // second operand: each element at (block, group, slot) of the zeroed staging
        int pg = -1, pp = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int u = lu[k];
          if (u >= 0) {
            const int g = u >> 2, p = u & 3;
            const bool second = g == pg;
            *reinterpret_cast<u16a*>(stg_b(stg2, 4 * g + 2 * (int)second)) = (uint16_t)lv[k];
            *stg_b(idxs, g) = (uint8_t)(second ? (pp | (p << 2)) : (p | (p << 2)));
            pg = g;
            pp = p;
          }
        }
#pragma unroll
        for (int bi = 0; bi < SEGB; ++bi)
#pragma unroll
          for (int t = 0; t < 4; ++t) a2[bi][t] = (int)stg2[64 * (4 * bi + t)];
#pragma unroll
        for (int bi = 0; bi < SEGB; ++bi) {
          const uint32_t d = idxs[64 * bi];
          i2[bi] = (int)((d & 0xFu) | ((d >> 4) & 0xF0u) | ((d >> 8) & 0xF00u) | ((d >> 12) & 0xF000u));
        }
        // cleared for the next item (after the reads above, in LDS order)
#pragma unroll
        for (int d = 0; d < 4 * SEGB; ++d) stg2[64 * d] = 0u;
#pragma unroll
        for (int d = 0; d < SEGB; ++d) idxs[64 * d] = 0u;
      }

      // products: every block of the segment on this wave's activation columns
      v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int bi = 0; bi < SEGB; ++bi) {
        if (bi < nb) {
          const uint8_t* xb = xseg + bi * 2048;
          const v2i p0 = lds_tr16(xb + bbase);
          const v2i p1 = lds_tr16(xb + bbase + 128);
          const v2i p2 = lds_tr16(xb + bbase + 1024);
          const v2i p3 = lds_tr16(xb + bbase + 1152);
          const v8i bf = v8i{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          acc = smfmac<WT>(a1[bi], bf, acc, i1[bi]);
          if constexpr (HY) acc = smfmac<WT>(a2[bi], bf, acc, i2[bi]);
        }
      }
      float* pt = reinterpret_cast<float*>(part + i * 1024);
#pragma unroll
      for (int v = 0; v < 4; ++v) pt[(4 * lg + v) * 16 + li] += acc[v];

      if constexpr (HY) {
        // residual: row rr, tokens 4 tq .. + 3
        const int rr = lane >> 2, tq = lane & 3;
        const int r0 = __builtin_amdgcn_readlane(rp_cur, 0);
        const int beg = __shfl(rp_cur, rr) - r0, end = __shfl(rp_cur, rr + 1) - r0;
#pragma unroll
        for (int m = 0; m < 4; ++m) rstage[lane + 64 * m] = ent_cur[m];
        // the residual's own sums (registers), added to the tile after the products
        float racc[4] = {0.f, 0.f, 0.f, 0.f};
        auto res_fma = [&](uint32_t ent, bool on) {
          const int col = (int)(ent >> 16), bi = col >> 6, r = col & 63;
          const float wv = on ? to_f32<WT>(ent & 0xFFFFu) : 0.f;
          const uint8_t* xp = xseg + bi * 2048 + r * 32 + 16 * ((tq >> 1) ^ ((r >> 3) & 1)) + 8 * (tq & 1);
          const v2i xv = *reinterpret_cast<const v2i*>(xp);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const uint32_t h = ((uint32_t)xv[x >> 1] >> (16 * (x & 1))) & 0xFFFFu;
            racc[x] = __builtin_fmaf(wv, to_f32<WT>(h), racc[x]);
          }
        };
        // four entries at a time, so their LDS reads overlap (padding
        // entries past the row's end count with weight 0)
        const int estg = min(end, RESCAP);
        for (int e = beg; e < estg; e += 4) {
          uint32_t en[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) en[q] = rstage[min(e + q, RESCAP - 1)];
#pragma unroll
          for (int q = 0; q < 4; ++q) res_fma(en[q], e + q < estg);
        }
        // entries past the staged ones (more than RESCAP in this item): read
        // from memory, in order, after everything else of the item
        if (__builtin_amdgcn_readlane(rp_cur, 16) - r0 > RESCAP)
          for (int e = max(beg, RESCAP); e < end; ++e)
            res_fma(ge[(uint32_t)(r0 + e)], true);
        float* rpt = reinterpret_cast<float*>(part + i * 1024) + rr * 16 + 4 * tq;
#pragma unroll
        for (int x = 0; x < 4; ++x) rpt[x] += racc[x];
      }
    }
    if constexpr (PF) {
      cur = nxt;
      if constexpr (HY) {
        rp_cur = rp_n1;
        rp_n1 = rp_n2;
#pragma unroll
        for (int m = 0; m < 4; ++m) ent_cur[m] = ent_nxt[m];
      }
    }
  };
  for (int j = 0; j < nValid - 1; ++j) step(j, ic<1>{});
  step(nValid - 1, ic<0>{});
  }

  // the waves' partial tiles, in wave order, then the epilogue
  __syncthreads();
  for (int o = threadIdx.x; o < ni * 256; o += NW * 64) {
    const int i = o >> 8, t = o & 255;
    const int row = t >> 4, tok = t & 15;
    float y = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) y += reinterpret_cast<const float*>(lds + PART_OFF + (v * MAXRB + i) * 1024)[t];
    const int64_t r = (int64_t)(b + i * G) * 16 + row;
    const int64_t tt = (int64_t)ty * 16 + tok;
    if (r < a.R && tt < a.T) {
      if (a.bias) y += a.bias[r];
      if (a.act) y = gelu_f32(y);
      const int64_t o = r * a.ldy + tt;
      if constexpr (OUT == NM_F32)
        static_cast<float*>(a.Y)[o] = y;
      else if constexpr (OUT == NM_F16)
        static_cast<uint16_t*>(a.Y)[o] = f32_to_f16_bits(y);
      else
        static_cast<uint16_t*>(a.Y)[o] = f32_to_bf16_bits(y);
    }
  }
#endif
}

template <int WT, bool HY>
hipError_t launch_wt(const HybridArgs& a, dim3 grid, hipStream_t s) {
  const dim3 block(Lay<HY>::NW * 64);
  if (a.ydt == NM_F32)
    hipLaunchKernelGGL((hybrid_kernel<WT, NM_F32, HY>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((hybrid_kernel<WT, WT, HY>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_spmm_hybrid(const HybridArgs& a, bool hy, hipStream_t s) {
  const dim3 grid((unsigned)a.G, (unsigned)((a.T + 15) / 16));
  if (a.wdt == NM_F16)
    return hy ? launch_wt<NM_F16, true>(a, grid, s) : launch_wt<NM_F16, false>(a, grid, s);
  return hy ? launch_wt<NM_BF16, true>(a, grid, s) : launch_wt<NM_BF16, false>(a, grid, s);
}

}  // namespace nm
