// Host packer of the three-layer format (page "Accelerating GPU Inference of
// Large Language Models with Moderately Unstructured Sparse Weight Matrices",
// Methodology 1): Sparse-TC 2:4 layer, Slot-Filling layer with 4-bit PDD
// distances and dummy points, CSR residual.  The byte image is described at
// nm_hybrid in nm_sparse.h.  Offline and host-only: it runs once per weight,
// before any product, and its greedy slot assignment is sequential within a
// fill unit; units are independent and go to worker threads by row block.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "nm_sparse.h"

namespace {

struct HyGeo {
  int64_t R, K, ldw, nRB, nKB, nSeg;
};

HyGeo hy_geo(int64_t R, int64_t K, int64_t ldw) {
  HyGeo g{R, K, ldw, (R + 15) / 16, (K + 63) / 64, 0};
  g.nSeg = (g.nKB + 7) / 8;
  return g;
}

// One fill unit's share of the image.
struct Unit {
  uint16_t val[64];   // slot sigma -> stored value
  uint8_t pos[64];    // slot sigma -> 2-bit position
  uint64_t codes;     // sixteen 4-bit codes, code i at bits 4 i
  int n_fill;
  int n_res;
  uint32_t res[64];   // (column in segment) << 16 | value bits
};

// Build unit (r, s, q).  w(c) = raw bits at column c of row r (0 outside).
template <typename F>
void build_unit(const HyGeo& g, int64_t s, int q, F w, Unit& u) {
  const int nb = (int)std::min<int64_t>(8, g.nKB - 8 * s);
  uint64_t empty = 0;                    // bit sigma: slot is empty
  int sur_u[64], ns = 0;                 // surplus local columns, ascending
  uint16_t sur_v[64];
  u.n_fill = u.n_res = 0;
  u.codes = 0;
  std::memset(u.val, 0, sizeof u.val);
  for (int sg = 0; sg < 64; ++sg) u.pos[sg] = (uint8_t)(1 - (sg & 1));  // empty pattern 1, 0
  for (int bi = 0; bi < nb; ++bi)
    for (int t = 0; t < 4; ++t) {
      const int64_t c0 = 64 * (8 * s + bi) + 16 * q + 4 * t;
      uint16_t v[4], key[4];
      int nzmask = 0;
      for (int p = 0; p < 4; ++p) {
        v[p] = w(c0 + p);
        key[p] = (uint16_t)(v[p] & 0x7FFF);  // sign-cleared bits order the magnitudes
        if (key[p]) nzmask |= 1 << p;
      }
      const int nz = __builtin_popcount(nzmask);
      const int sg = 8 * bi + 2 * t;
      if (nz >= 2) {
        // the best and second best: strictly larger key wins, ties to the lower p
        int a = -1, b = -1;
        for (int p = 0; p < 4; ++p) {
          if (!(nzmask >> p & 1)) continue;
          if (a < 0 || key[p] > key[a]) { b = a; a = p; }
          else if (b < 0 || key[p] > key[b]) b = p;
        }
        const int lo = std::min(a, b), hi = std::max(a, b);
        u.val[sg] = v[lo]; u.pos[sg] = (uint8_t)lo;
        u.val[sg + 1] = v[hi]; u.pos[sg + 1] = (uint8_t)hi;
        for (int p = 0; p < 4; ++p)
          if ((nzmask >> p & 1) && p != lo && p != hi) {
            sur_u[ns] = 16 * bi + 4 * t + p;
            sur_v[ns++] = v[p];
          }
      } else if (nz == 1) {
        const int p = __builtin_ctz(nzmask);
        u.val[sg] = v[p]; u.pos[sg] = (uint8_t)p;
        u.pos[sg + 1] = (uint8_t)p;
        empty |= 1ull << (sg + 1);
      } else {
        empty |= 3ull << sg;
      }
    }
  // slot filling: each surplus element, in column order, takes the next empty
  // slot and one distance code (after dummy codes for a gap over 15), or goes
  // to the residual once slots or codes run out
  int last = -1, ncode = 0;
  for (int i = 0; i < ns; ++i) {
    const int gap = sur_u[i] - last;
    const int dummies = (gap - 1) / 15;
    if (empty != 0 && ncode + dummies + 1 <= 16) {
      ncode += dummies;                              // dummy codes are 0
      u.codes |= (uint64_t)(gap - 15 * dummies) << (4 * ncode++);
      const int sg = __builtin_ctzll(empty);
      empty &= empty - 1;
      u.val[sg] = sur_v[i];
      ++u.n_fill;
      last = sur_u[i];
    } else {
      const int col = 64 * (sur_u[i] / 16) + 16 * q + sur_u[i] % 16;
      u.res[u.n_res++] = ((uint32_t)col << 16) | sur_v[i];
    }
  }
}

struct RowBlockOut {
  std::vector<uint32_t> res;        // residual entries, segment rows in order
  std::vector<int32_t> count;       // entries per segment row (nSeg * 16)
  int64_t n_fill = 0;
};

// Pack row blocks [rb0, rb1); write the layer-1/2 bytes when `values` is set.
void pack_rows(const uint16_t* W, const HyGeo& g, int64_t rb0, int64_t rb1, uint8_t* values,
               uint8_t* meta, uint8_t* codes, std::vector<RowBlockOut>& out) {
  Unit u;
  for (int64_t rb = rb0; rb < rb1; ++rb) {
    RowBlockOut& o = out[rb];
    o.count.assign(g.nSeg * 16, 0);
    for (int64_t s = 0; s < g.nSeg; ++s)
      for (int rr = 0; rr < 16; ++rr) {
        const int64_t r = rb * 16 + rr;
        auto w = [&](int64_t c) -> uint16_t { return (r < g.R && c < g.K) ? W[r * g.ldw + c] : (uint16_t)0; };
        uint32_t seg_res[256];
        int nres = 0;
        for (int q = 0; q < 4; ++q) {
          build_unit(g, s, q, w, u);
          o.n_fill += u.n_fill;
          for (int i = 0; i < u.n_res; ++i) seg_res[nres++] = u.res[i];
          if (!values) continue;
          const int nb = (int)std::min<int64_t>(8, g.nKB - 8 * s);
          for (int bi = 0; bi < nb; ++bi) {
            const int64_t blk = rb * g.nKB + 8 * s + bi;
            uint8_t* vrow = values + blk * 1024 + rr * 64 + 16 * q;   // quad q: slots 8q .. 8q+7
            std::memcpy(vrow, &u.val[8 * bi], 16);
            uint16_t m = 0;
            for (int k = 0; k < 8; ++k) m |= (uint16_t)(u.pos[8 * bi + k] << (2 * k));
            uint8_t* mrow = meta + blk * 128 + rr * 8 + 2 * q;        // 16 bits per quad
            mrow[0] = (uint8_t)m;
            mrow[1] = (uint8_t)(m >> 8);
          }
          std::memcpy(codes + ((rb * g.nSeg + s) * 64 + 16 * q + rr) * 8, &u.codes, 8);
        }
        // the four quads interleave in column order: sort the segment row
        std::sort(seg_res, seg_res + nres);
        o.count[s * 16 + rr] = nres;
        o.res.insert(o.res.end(), seg_res, seg_res + nres);
      }
  }
}

bool valid_args(const void* W, int64_t ldw, int64_t R, int64_t K, nm_status* st, int32_t dt) {
  if (!W || R < 1 || K < 4 || K % 4 || ldw < K) { *st = NM_EINVAL; return false; }
  if (dt != NM_F16 && dt != NM_BF16) { *st = NM_EUNSUPPORTED; return false; }
  return true;
}

// Run the packer over all row blocks on worker threads.
void run(const uint16_t* W, const HyGeo& g, uint8_t* values, uint8_t* meta, uint8_t* codes,
         std::vector<RowBlockOut>& out) {
  out.assign(g.nRB, RowBlockOut());
  const unsigned hw = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  const int64_t nth = std::min<int64_t>(hw, g.nRB);
  std::vector<std::thread> th;
  for (int64_t i = 0; i < nth; ++i) {
    const int64_t a = g.nRB * i / nth, b = g.nRB * (i + 1) / nth;
    th.emplace_back(pack_rows, W, std::cref(g), a, b, values, meta, codes, std::ref(out));
  }
  for (auto& t : th) t.join();
}

void sizes(const HyGeo& g, nm_hybrid* d, int64_t n_res) {
  d->values_bytes = (size_t)(g.nRB * g.nKB * 1024);
  d->meta_bytes = (size_t)(g.nRB * g.nKB * 128);
  d->codes_bytes = (size_t)(g.nRB * g.nSeg * 512);
  d->res_ptr_bytes = (size_t)((g.nRB * g.nSeg * 16 + 1) * 4);
  d->res_ent_bytes = (size_t)(n_res * 4);
}

}  // namespace

extern "C" {

nm_status nm_hybrid_pack_size(const void* W, int64_t ldw, int64_t rows, int64_t K, int32_t dtype,
                              nm_hybrid* desc) {
  nm_status st = NM_OK;
  if (!desc || !valid_args(W, ldw, rows, K, &st, dtype)) return desc ? st : NM_EINVAL;
  const HyGeo g = hy_geo(rows, K, ldw);
  std::vector<RowBlockOut> out;
  run(static_cast<const uint16_t*>(W), g, nullptr, nullptr, nullptr, out);
  int64_t n_res = 0, n_fill = 0;
  for (auto& o : out) { n_res += (int64_t)o.res.size(); n_fill += o.n_fill; }
  if (n_res > INT32_MAX) return NM_EINVAL;
  desc->rows = rows;
  desc->K = K;
  desc->dtype = dtype;
  desc->n_res = n_res;
  desc->n_fill = n_fill;
  sizes(g, desc, n_res);
  return NM_OK;
}

nm_status nm_hybrid_pack(const void* W, int64_t ldw, nm_hybrid* desc) {
  nm_status st = NM_OK;
  if (!desc) return NM_EINVAL;
  if (!valid_args(W, ldw, desc->rows, desc->K, &st, desc->dtype)) return st;
  const HyGeo g = hy_geo(desc->rows, desc->K, ldw);
  nm_hybrid want = *desc;
  sizes(g, &want, desc->n_res);
  if (!desc->values || !desc->meta || !desc->codes || !desc->res_ptr || (desc->n_res > 0 && !desc->res_ent) ||
      desc->values_bytes != want.values_bytes || desc->meta_bytes != want.meta_bytes ||
      desc->codes_bytes != want.codes_bytes || desc->res_ptr_bytes != want.res_ptr_bytes ||
      desc->res_ent_bytes != want.res_ent_bytes)
    return NM_EINVAL;
  std::vector<RowBlockOut> out;
  uint8_t* values = static_cast<uint8_t*>(desc->values);
  uint8_t* meta = static_cast<uint8_t*>(desc->meta);
  std::memset(values, 0, desc->values_bytes);
  std::memset(meta, 0, desc->meta_bytes);
  std::memset(desc->codes, 0, desc->codes_bytes);
  // rows past R and blocks of the last segment past nKB are never visited by
  // a unit: give them the empty pattern here (units overwrite the rest)
  for (int64_t i = 0; i < (int64_t)desc->meta_bytes; ++i) meta[i] = 0x11;
  run(static_cast<const uint16_t*>(W), g, values, meta, static_cast<uint8_t*>(desc->codes), out);
  int64_t n_res = 0;
  for (auto& o : out) n_res += (int64_t)o.res.size();
  if (n_res != desc->n_res) return NM_EINVAL;   // desc sized for another weight
  int32_t* ptr = static_cast<int32_t*>(desc->res_ptr);
  uint32_t* ent = static_cast<uint32_t*>(desc->res_ent);
  int64_t at = 0;
  ptr[0] = 0;
  for (int64_t rb = 0; rb < g.nRB; ++rb) {
    const RowBlockOut& o = out[rb];
    for (int64_t z = 0; z < g.nSeg * 16; ++z) {
      at += o.count[z];
      ptr[rb * g.nSeg * 16 + z + 1] = (int32_t)at;
    }
    if (!o.res.empty()) std::memcpy(ent + (at - (int64_t)o.res.size()), o.res.data(), o.res.size() * 4);
  }
  desc->format_version = NM_FORMAT_VERSION;
  return NM_OK;
}

}  // extern "C"
