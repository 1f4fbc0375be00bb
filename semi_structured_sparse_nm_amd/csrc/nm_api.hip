// C ABI of the library (include/nm_sparse.h): host-side validation, kernel
// variant choice per shape, launches.  Stateless and thread-safe.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nm_common.hpp"
#include "nm_hybrid.hpp"

using nm::Geometry;
using nm::SpmmArgs;

#include <atomic>
#include <mutex>

namespace nm {

int cu_count(int device) {
  static std::atomic<int> cache[64];
  if (device < 0 || device >= 64) return 256;
  int cus = cache[device].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0)
    cus = 256;
  cache[device].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace nm

namespace {

bool is_weight_dtype(int dt) { return dt == NM_I8 || dt == NM_F16 || dt == NM_BF16; }

nm_status check_shape(int64_t rows, int64_t K, int32_t N, int32_t M, int32_t dtype) {
  if (rows < 1 || K < 1 || N < 1 || M < 1 || N > M) return NM_EINVAL;
  if (M != 4 && M != 8) return NM_EUNSUPPORTED;
  if (K % M != 0) return NM_EINVAL;
  if (!is_weight_dtype(dtype)) return NM_EUNSUPPORTED;
  return NM_OK;
}

bool pair_supported(int wdt, int ydt) {
  switch (wdt) {
    case NM_I8: return ydt == NM_I32 || ydt == NM_I8;
    case NM_F16: return ydt == NM_F16 || ydt == NM_F32;
    case NM_BF16: return ydt == NM_BF16 || ydt == NM_F32;
    default: return false;
  }
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

nm_status check_desc(const nm_packed* w, Geometry* out) {
  if (!w) return NM_EINVAL;
  nm_status st = check_shape(w->rows, w->K, w->N, w->M, w->dtype);
  if (st != NM_OK) return st;
  Geometry g = Geometry::make(w->rows, w->K, w->N, w->M, nm::dtype_bytes(w->dtype));
  if (!w->values || w->values_bytes != g.values_bytes()) return NM_EINVAL;
  if (g.w != 0 && (!w->meta || w->meta_bytes != g.meta_bytes())) return NM_EINVAL;
  if (!aligned(w->values, 16) || (g.w != 0 && !aligned(w->meta, 16))) return NM_EUNSUPPORTED;
  *out = g;
  return NM_OK;
}

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  return nm::cu_count(dev);
}

// The one debug override: NM_SPMM_VARIANT=<variant>[:<S>] forces a variant
// where its requirements hold, and with ":<S>" also the number of K slices
// of the tile kernels that take a K split (tile and split sweeps); an empty
// variant name (":<S>") keeps the automatic choice and forces only S.
struct Forced {
  char name[96];
  int S;        // 0: not forced
};

Forced forced() {
  Forced f{};
  const char* e = getenv("NM_SPMM_VARIANT");
  if (!e) return f;
  const char* colon = strchr(e, ':');
  const size_t n = colon ? (size_t)(colon - e) : strlen(e);
  if (n < sizeof f.name) {
    memcpy(f.name, e, n);
    f.name[n] = 0;
  }
  if (colon) f.S = atoi(colon + 1);
  return f;
}

// Variant table (the paper's adaptive parallelism, Sec. 4.1: the kernel and
// its tiling follow the operator's shape).
enum Variant {
  V_INVALID = 0,
  V_GENERIC,
  V_SMFMAC_I8P,     // int8 2:4 sparse MFMA, persistent 256 x 128 tiles, cross-tile pipeline
  V_SMFMAC_I8P8,    // persistent, 8-wave workgroups (512 x 128 tiles, one per CU)
  V_SMFMAC_I8WS,    // int8 2:4, K <= 768: packed rows held in registers, activations streamed
  V_SMFMAC_I8SM,    // int8 2:4, any T and row alignment: one wave per 16 x 16 output tile
  V_SMFMAC_H,       // fp16 / bf16 2:4 sparse MFMA, persistent 256 x 128 tiles
  V_SMFMAC_HD,      // fp16 / bf16 2:4, decode shapes (T <= 16): K split across 8 waves
  V_EXPAND,         // any other N:M (int8, fp16, bf16): windows expanded in registers, dense MFMA
  V_EXPAND_DECODE,  // any N:M, decode shapes (T <= 16): K split across 8 waves, dense MFMA
  V_SMFMAC_I8TK,    // int8 2:4 persistent, [T][K] layout (X [T][K], Y [T][R])
  V_SMFMAC_I8WSTK,  // int8 2:4, K <= 768, [T][K] layout: packed rows held in registers
  V_STREAM24,       // fp16 / bf16 2:4, T <= 16 per token tile: one workgroup per CU walking row
                    // blocks, values straight to registers one 512-column segment ahead
  V_SPLIT24_I8WS,   // int8 N:M, K <= 768: the weight split into two 2:4 layers in the
                    // workspace, then a weight-stationary kernel over both
  V_DENSE24_I8WS,   // int8 N = M, K <= 768: the same kernel, the two layers taken in registers
  V_SPLIT24_I8WSTK, // the two-layer split in the [T][K] layout
  V_DENSE24_I8WSTK, // the dense form in the [T][K] layout
  V_COUNT
};

const char* variant_name(Variant v) {
  switch (v) {
    case V_GENERIC: return "generic_dense_expand";
    case V_SMFMAC_I8P: return "smfmac_i8_2of4_persistent";
    case V_SMFMAC_I8P8: return "smfmac_i8_2of4_persistent_w8";
    case V_SMFMAC_I8WS: return "smfmac_i8_2of4_stationary";
    case V_SMFMAC_I8SM: return "smfmac_i8_2of4_small";
    case V_SMFMAC_H: return "smfmac_h_2of4_persistent";
    case V_SMFMAC_HD: return "smfmac_h_2of4_decode";
    case V_EXPAND: return "expand_mfma_persistent";
    case V_EXPAND_DECODE: return "expand_mfma_decode";
    case V_SMFMAC_I8TK: return "smfmac_i8_2of4_tk";
    case V_SMFMAC_I8WSTK: return "smfmac_i8_2of4_stationary_tk";
    case V_STREAM24: return "smfmac_h_2of4_stream_decode";
    case V_SPLIT24_I8WS: return "split24_smfmac_i8_stationary";
    case V_DENSE24_I8WS: return "dense24_smfmac_i8_stationary";
    case V_SPLIT24_I8WSTK: return "split24_smfmac_i8_stationary_tk";
    case V_DENSE24_I8WSTK: return "dense24_smfmac_i8_stationary_tk";
    default: return "invalid";
  }
}

struct Call {
  const Geometry* g;
  int wdt, ydt;
  int64_t T, ldx, ldy;
  const void* X;
  const void* Y;
  int act;
  int layout;
};

bool eligible(Variant v, const Call& c);

// the 2:4 geometry of a weight's two-layer split (and of its 2:4 re-pack)
Geometry geometry24(const Geometry& g) { return Geometry::make(g.R, g.K, 2, 4, g.eb); }

bool eligible(Variant v, const Call& c) {
  // the [T][K] layout has kernels of its own (and the generic one)
  if ((c.layout == NM_LAYOUT_TK) !=
          (v == V_SMFMAC_I8TK || v == V_SMFMAC_I8WSTK || v == V_SPLIT24_I8WSTK || v == V_DENSE24_I8WSTK) &&
      v != V_GENERIC)
    return false;
  switch (v) {
    case V_GENERIC: return true;
    case V_SMFMAC_I8P:
    case V_SMFMAC_I8P8:
      // 2:4 int8; X rows in whole 16-byte chunks; 32-bit buffer offsets,
      // which must not wrap for the rows a tile reaches past K and R (up to
      // 128 k and 512 rows); int8 output stored as 16-byte row pieces
      return c.wdt == NM_I8 && c.g->N == 2 && c.g->M == 4 && c.T % 16 == 0 && c.ldx % 16 == 0 &&
             aligned(c.X, 16) && (c.g->K + 128) * c.ldx < (1ll << 31) &&
             c.g->values_bytes() < (1ull << 31) && (c.g->R + 512) * c.ldy * 4 < (1ll << 31) &&
             (c.ydt == NM_I32 || (c.ydt == NM_I8 && c.ldy % 16 == 0 && aligned(c.Y, 16)));
    case V_SMFMAC_I8SM:
      // 2:4 int8, int8 or int32 output, any T and row alignment (byte
      // gathers and byte / dword stores); 32-bit buffer offsets that do not
      // wrap for the rows a block reaches past K and R
      return c.wdt == NM_I8 && c.g->N == 2 && c.g->M == 4 && (c.ydt == NM_I8 || c.ydt == NM_I32) &&
             (c.g->K + 128) * c.ldx < (1ll << 31) && c.g->values_bytes() < (1ull << 31) &&
             (c.g->R + 16) * c.ldy * 4 < (1ll << 31);
    case V_SMFMAC_I8WS:
      // as the persistent kernels, and K in (640, 768] (six column blocks
      // held in registers) with every XCD's workgroups (one per CU)
      // covering the row tiles of 512 rows
      return eligible(V_SMFMAC_I8P, c) && c.g->nKB == 6 && (c.g->R + 511) / 512 <= device_cus() / 8;
    case V_SMFMAC_H:
      // fp16 / bf16 2:4; X rows in whole 16-byte pieces; 32-bit buffer
      // offsets that do not wrap for the rows a tile reaches past K and R;
      // 16-bit output stored as 16-byte row pieces
      return (c.wdt == NM_F16 || c.wdt == NM_BF16) && c.g->N == 2 && c.g->M == 4 && c.T % 16 == 0 &&
             c.ldx % 8 == 0 && aligned(c.X, 16) && (c.g->K + 64) * c.ldx * 2 < (1ll << 31) &&
             c.g->values_bytes() < (1ull << 31) && (c.g->R + 256) * c.ldy * 4 < (1ll << 31) &&
             (c.ydt == NM_F32 || (c.ldy % 8 == 0 && aligned(c.Y, 16)));
    case V_SMFMAC_HD:
      // fp16 / bf16 2:4 with at most 16 tokens; X rows in whole 16-byte
      // pieces; 32-bit buffer offsets that do not wrap past K
      return (c.wdt == NM_F16 || c.wdt == NM_BF16) && c.g->N == 2 && c.g->M == 4 && c.T <= 16 &&
             c.ldx % 8 == 0 && aligned(c.X, 16) && (c.g->K + 64) * c.ldx * 2 < (1ll << 31) &&
             c.g->values_bytes() < (1ull << 31);
    case V_EXPAND:
      // an instantiated N:M other than 2:4 (2:4 too with an activation, as
      // a fallback for it); whole 16-token tiles; X rows in
      // whole 16-byte pieces; 32-bit buffer offsets that do not wrap for the
      // rows a tile reaches past K and R (up to 128 k and 256 rows); 8- and
      // 16-bit output stored as 16-byte row pieces
      return nm::expand_supported(c.g->N, c.g->M) && !(c.g->N == 2 && c.g->M == 4 && c.act == NM_ACT_NONE) &&
             c.T % 16 == 0 &&
             c.ldx % (16 / c.g->eb) == 0 && aligned(c.X, 16) && (c.g->K + 128) * c.ldx * c.g->eb < (1ll << 31) &&
             c.g->values_bytes() + 1024 < (1ull << 31) && c.g->meta_bytes() + 1024 < (1ull << 31) &&
             (c.g->R + 256) * c.ldy * 4 < (1ll << 31) &&
             (c.ydt == NM_I32 || c.ydt == NM_F32 || (c.ldy % (16 / nm::dtype_bytes(c.ydt)) == 0 && aligned(c.Y, 16)));
    case V_EXPAND_DECODE:
      // any instantiated N:M with at most 16 tokens; X rows in whole 16-byte
      // pieces; 32-bit buffer offsets that do not wrap for the rows past K a
      // block reaches and the loads past the packed buffers' ends
      return nm::expand_supported(c.g->N, c.g->M) && c.T <= 16 && c.ldx % (16 / c.g->eb) == 0 &&
             aligned(c.X, 16) && (c.g->K + 128) * c.ldx * c.g->eb < (1ll << 31) &&
             c.g->values_bytes() + 2048 < (1ull << 31) && c.g->meta_bytes() + 1024 < (1ull << 31) &&
             c.g->R * c.ldy < (1ll << 40);
    case V_STREAM24:
      // fp16 / bf16 2:4 with at most 16 tokens; 32-bit buffer offsets
      return (c.wdt == NM_F16 || c.wdt == NM_BF16) && c.g->N == 2 && c.g->M == 4 && c.T <= 16 &&
             aligned(c.X, 2) && c.g->K * c.ldx * 2 < (1ll << 31) && c.g->values_bytes() < (1ull << 31);
    case V_SMFMAC_I8TK:
      // int8 2:4 in the [T][K] layout; token rows in whole 16-byte pieces;
      // 32-bit buffer offsets that do not wrap for the tokens a tile reaches
      // past T; R a multiple of 16, so a 16-row output piece never crosses
      // into the next token's row
      return c.wdt == NM_I8 && c.g->N == 2 && c.g->M == 4 && c.ldx % 16 == 0 && aligned(c.X, 16) &&
             (c.T + 128) * c.ldx < (1ll << 31) && c.g->values_bytes() < (1ull << 31) && c.g->R % 16 == 0 &&
             (c.T + 128) * c.ldy * 4 < (1ll << 31) && aligned(c.Y, 16) &&
             ((c.ydt == NM_I8 && c.ldy % 16 == 0) || (c.ydt == NM_I32 && c.ldy % 4 == 0));
    case V_SMFMAC_I8WSTK:
      // as the [T][K] persistent kernel, and K in (640, 768] with every
      // XCD's workgroups (one per CU) covering the row tiles of 512 rows
      return eligible(V_SMFMAC_I8TK, c) && c.g->nKB == 6 && (c.g->R + 511) / 512 <= device_cus() / 8;
    case V_SPLIT24_I8WS: {
      // int8, any N:M; the 2:4 layers' product as the persistent kernels
      // take it, K in (640, 768] (six column blocks held in registers), at
      // most one 256-row tile per workgroup (one per CU)
      if (c.wdt != NM_I8 || !nm::split24_supported(*c.g) || c.g->values_bytes() >= (1ull << 31)) return false;
      const Geometry g24 = geometry24(*c.g);
      Call c24 = c;
      c24.g = &g24;
      return eligible(V_SMFMAC_I8P, c24) && g24.nKB == 6 && (c.g->R + 255) / 256 <= device_cus() / 8 * 8;
    }
    case V_DENSE24_I8WS:
      // int8 N = M (dense rows of 2048-byte blocks), otherwise as the split
      return c.wdt == NM_I8 && c.g->N == c.g->M && c.g->values_bytes() < (1ull << 31) &&
             eligible(V_SPLIT24_I8WS, c);
    case V_SPLIT24_I8WSTK: {
      // as the split, with the 2:4 layers' product as the [T][K] int8 2:4
      // kernel takes it (R a multiple of 16)
      if (c.wdt != NM_I8 || !nm::split24_supported(*c.g) || c.g->values_bytes() >= (1ull << 31)) return false;
      const Geometry g24 = geometry24(*c.g);
      Call c24 = c;
      c24.g = &g24;
      return eligible(V_SMFMAC_I8TK, c24) && g24.nKB == 6 && (c.g->R + 255) / 256 <= device_cus() / 8 * 8;
    }
    case V_DENSE24_I8WSTK:
      return c.wdt == NM_I8 && c.g->N == c.g->M && c.g->values_bytes() < (1ull << 31) &&
             eligible(V_SPLIT24_I8WSTK, c);
    default: return false;
  }
}

Variant choose_auto(const Call& c, bool ws_ok = true);

// ws_ok: variants that need a workspace copy of the weight may be chosen
Variant choose(const Call& c, bool ws_ok = true) {
  const Forced f = forced();
  if (f.name[0]) {
    for (int v = V_GENERIC; v < V_COUNT; ++v)
      if (strcmp(f.name, variant_name((Variant)v)) == 0 && eligible((Variant)v, c) &&
          (ws_ok || (v != V_SPLIT24_I8WS && v != V_SPLIT24_I8WSTK)))
        return (Variant)v;
  }
  return choose_auto(c, ws_ok);
}

constexpr double kRepackMinWork = 2147483648.0;

Variant choose_auto(const Call& c, bool ws_ok) {
  // [T][K] layout, int8 2:4: the weight-stationary form under the same rule
  // as in [K][T] (below), else the persistent kernel.  Measured on MI355X at
  // T = 12608, rotated operands, one box (stationary / persistent us): FC1
  // R 3072 29.4 / 33.6, QKV R 2304 27.0 / 29.0
  if (eligible(V_SMFMAC_I8WSTK, c)) {
    const int64_t steps = ((c.g->R + 511) / 512) * ((c.T + 63) / 64);
    if (2 * steps >= 7 * (int64_t)device_cus()) return V_SMFMAC_I8WSTK;
  }
  if (eligible(V_SMFMAC_I8TK, c)) return V_SMFMAC_I8TK;
  // [T][K] layout, other int8 N:M with K in (640, 768]: the two-layer kernel
  // (dense weights: the layers in registers; else split in the workspace,
  // except 1:4, 1:8 and 2:8, which the 2:4 re-pack takes)
  {
    const double work = (double)c.g->R * (double)c.g->K * (double)c.T;
    if (eligible(V_DENSE24_I8WSTK, c) && work >= kRepackMinWork) return V_DENSE24_I8WSTK;
    if (ws_ok && eligible(V_SPLIT24_I8WSTK, c) && !(c.g->N == 2 && c.g->M == 4) &&
        !nm::repack24_supported(*c.g) && work >= kRepackMinWork)
      return V_SPLIT24_I8WSTK;
  }
  // decode shapes (few tokens), fp16 / bf16 2:4: with more 16-row blocks
  // than compute units, one workgroup per CU walking row blocks with its
  // loads a segment ahead; otherwise K split inside a workgroup per row
  // block.  Measured on MI355X, LLaMA-7B T = 16 (streaming / split us): up
  // (688 row blocks) 13.1 / 16.8, qkvo (256) 7.6 / 7.5, down (256) 15.4 / 15.1
  if (eligible(V_STREAM24, c) && c.g->nRB > device_cus()) return V_STREAM24;
  if (eligible(V_SMFMAC_HD, c)) return V_SMFMAC_HD;
  if (eligible(V_EXPAND_DECODE, c)) return V_EXPAND_DECODE;
  // int8 2:4, K in (640, 768]: the weight-stationary kernel when its
  // workgroups (one per CU) get at least 3.5 token steps of 64 each, so the
  // one-time load of their packed rows is spread over enough products.
  // Measured on MI355X at T = 12608, rotated operands (stationary /
  // persistent us): FC1 R 3072 (4.6 steps) 31.3 / 38.8 (4-wave); QKV R 2304
  // (3.8) 29.7 / 30.7 (8-wave); proj R 768 (1.5) 18.0 / 16.7 (8-wave).
  if (eligible(V_SMFMAC_I8WS, c)) {
    const int64_t steps = ((c.g->R + 511) / 512) * ((c.T + 63) / 64);
    if (2 * steps >= 7 * (int64_t)device_cus()) return V_SMFMAC_I8WS;
  }
  // int8 2:4 persistent: 8-wave workgroups (512 x 128 tiles, one per CU,
  // two waves per SIMD) unless the 256 x 128 tiles of the 4-wave kernel
  // (two workgroups per CU) number at least four per CU.  Measured on MI355X
  // at T = 12608 (4-wave tiles; 4-wave / 8-wave us): proj R 768 (297): 17.6
  // / 15.0; FC2 R 768, K 3072 (297): 43.3 / 36.5; QKV R 2304 (891): 30.2 /
  // 25.7; FC1 R 3072 (1188): 31.5 / 33.1.
  if (eligible(V_SMFMAC_I8P, c)) {
    const int64_t tiles4 = ((c.g->R + 255) / 256) * ((c.T + 127) / 128);
    if (tiles4 < 4 * (int64_t)device_cus() && eligible(V_SMFMAC_I8P8, c)) return V_SMFMAC_I8P8;
    return V_SMFMAC_I8P;
  }
  // int8 2:4 the tile kernels do not take (T not a multiple of 16, rows not
  // 16-byte aligned): one wave per output tile.  ViT-Tiny slice 192 x 192 x
  // 197: see the measured figure in the variant's documentation
  if (eligible(V_SMFMAC_I8SM, c)) return V_SMFMAC_I8SM;
  if (eligible(V_SMFMAC_H, c)) return V_SMFMAC_H;
  // int8 N:M with up to four kept members per group of four columns (3:4,
  // 3:8 .. 7:8), K in (640, 768], large enough for the extra launch:
  // the two-layer split and the weight-stationary kernel over both layers
  // (1:4, 1:8, 2:8 take the single-layer re-pack below instead)
  // (dense int8, N = M: the same kernel takes the two layers in registers,
  // no copy)
  const double work = (double)c.g->R * (double)c.g->K * (double)c.T;
  if (eligible(V_DENSE24_I8WS, c) && work >= kRepackMinWork) return V_DENSE24_I8WS;
  if (ws_ok && eligible(V_SPLIT24_I8WS, c) && !(c.g->N == 2 && c.g->M == 4) && !nm::repack24_supported(*c.g) &&
      work >= kRepackMinWork)
    return V_SPLIT24_I8WS;
  if (eligible(V_EXPAND, c)) return V_EXPAND;
  return V_GENERIC;
}

Call make_call(const Geometry& g, int wdt, int ydt, int64_t T, int64_t ldx, int64_t ldy, const void* X,
               const void* Y, int act = NM_ACT_NONE, int layout = NM_LAYOUT_KT) {
  Call c;
  c.g = &g; c.wdt = wdt; c.ydt = ydt; c.T = T; c.ldx = ldx; c.ldy = ldy; c.X = X; c.Y = Y; c.act = act;
  c.layout = layout;
  return c;
}


// K slices for the tile kernels that take a K split (the paper's adaptive
// parallelism, Sec. 4.1: enough work items in flight at inference-sized
// shapes, with the reduction's cost bounded).  Slices divide the column
// blocks evenly and keep at least kMinBlocks blocks each, so the load
// pipeline still fills.  Cost model: rounds of work items over the compute
// units times column blocks per item times the time of one block step, plus
// the partial sums' round trip (S R T 4 bytes written, then read by the
// reduction) and the reduction's launch.  One work item per CU per round:
// the fp16 kernel keeps two workgroups on a CU, but they share its matrix
// cores and LDS, so a second one does not double the rate.  The constants
// are fitted on MI355X (Swin-T and LLaMA-7B shapes, forced S = 1 .. 16): the
// model ranks the measured times and picks S = 4 for the Swin stage-4 MLP
// out-projection (37.7 -> 22.8 us) and no split where the partials' traffic
// outweighs the gain.  NM_SPMM_VARIANT=<variant>:<S> forces S where it
// divides the column blocks (1 turns the split off).
constexpr int kMinBlocks = 4;
constexpr double kStepUs = 0.8;          // one column-block step of a work item
constexpr double kPartialGBs = 5000.0;   // partial sums' effective write + read rate
constexpr double kReduceUs = 2.0;        // reduction launch and tail

int ksplit_for(Variant v, const Call& c) {
  if (v != V_SMFMAC_H && v != V_EXPAND) return 1;
  const Geometry& g = *c.g;
  const int nKB = (int)g.nKB;
  if (c.T % 4 != 0) return 1;
  // the partials' 32-bit element offsets within one slice
  if ((g.R + 256) * c.T * 4 >= (1ll << 31)) return 1;
  const int fS = forced().S;
  if (fS) return (fS >= 1 && fS <= nKB && nKB % fS == 0) ? fS : 1;
  const int64_t tiles = ((g.R + 255) / 256) * ((c.T + 127) / 128);
  const int64_t slots = device_cus();
  auto cost = [&](int S) {
    const double rounds = (double)((tiles * S + slots - 1) / slots);
    double us = rounds * (nKB / S) * kStepUs;
    if (S > 1) us += kReduceUs + (double)S * g.R * c.T * 4 * 2 / (kPartialGBs * 1e3);
    return us;
  };
  int best = 1;
  double best_us = cost(1);
  for (int S = 2; S <= 16 && nKB / S >= kMinBlocks; ++S) {
    if (nKB % S) continue;
    const double us = cost(S);
    if (us < best_us) { best = S; best_us = us; }
  }
  return best;
}

size_t workspace_for(Variant v, const Call& c) {
  const int S = ksplit_for(v, c);
  return S > 1 ? (size_t)S * c.g->R * c.T * 4 : 0;
}

// ---- 2:4 re-pack.  A 1:4, 1:8 or 2:8 weight is also a 2:4 weight (no
// group of four columns holds more than two kept members), so its product
// can run on the 2:4 sparse-MFMA tile kernels: the call first re-packs the
// weight into the 2:4 layout in the workspace (nm_repack24.hip), then runs
// the 2:4 kernel on that copy.  The copy costs one small launch (about 2 us
// on ViT-B shapes) and a few MB of traffic; the int8 2:4 kernels issue half
// the matrix instructions of the dense-expand ones (whose dense int8 MFMA
// also runs at about half the sparse one's rate) and expand nothing.
// Measured on MI355X, ViT-B int8 at T = 12608 (expand -> re-packed, us):
// 1:4 QKV 33.5 -> 28.1, proj 17.9 -> 17.1, FC1 39.1 -> 35.2, FC2 50.5 ->
// 37.9; 2:8 QKV 35.4 -> 27.9, proj 18.6 -> 17.2, FC1 43.2 -> 35.1, FC2 55.2
// -> 38.7.  For fp16 / bf16 it did not pay (Swin-T 1:4: from 4% faster to
// 24% slower), so it is taken for int8 weights only, when the product is
// large enough for the extra launch (R K T >= 2^31) and the 2:4 kernel would
// run without a K split: in the [K][T] layout in place of the dense-expand
// kernel, in the [T][K] layout (its int8 2:4 kernel) in place of the generic
// one.
// NM_SPMM_VARIANT=repack24_<2:4 tile variant> forces it (fp16 / bf16 too)
// where the 2:4 kernel's requirements hold.
constexpr const char* kRepackPrefix = "repack24_";

struct Plan {
  Variant v = V_INVALID;
  bool repack = false;
  bool split = false;        // two 2:4 layers in the workspace (g24 each)
  Geometry g24;              // the 2:4 geometry of the re-packed copy
  bool transpose = false;    // [T][K] call run as transpose, [K][T] product, transpose
  int64_t Tp = 0;            // tokens of the [K][T] product (T rounded up to 16)
  int S = 1;                 // K slices of the [K][T] product
};

size_t repack_meta_off(const Geometry& g24) { return (g24.values_bytes() + 255) / 256 * 256; }
size_t repack_bytes(const Geometry& g24) { return repack_meta_off(g24) + g24.meta_bytes(); }
// the two layers of a split: layer l's values at l * split_layer_bytes, its
// meta repack_meta_off further
size_t split_layer_bytes(const Geometry& g24) { return (repack_bytes(g24) + 255) / 256 * 256; }

bool repack_inner(Variant v) {
  return v == V_SMFMAC_I8P || v == V_SMFMAC_I8P8 || v == V_SMFMAC_I8WS || v == V_SMFMAC_H || v == V_SMFMAC_I8TK ||
         v == V_SMFMAC_I8WSTK;
}

// ---- [T][K] calls without a kernel of their own.  The generic kernel takes
// every shape in that layout but is slow at scale (about 1 ms on ViT-B
// shapes), so a large [T][K] call it would get runs as three launches in
// the caller's workspace instead: X [T][K] transposed into X' [K][T'] (T'
// = T rounded up to 16, extra tokens zero), the [K][T] product Y' [R][T']
// with the kernel that layout picks (epilogue included), and Y' transposed
// into Y [T][R] (nm_transpose.hip).  Taken when R K T >= 2^26.
// NM_SPMM_VARIANT=transpose_<[K][T] variant> forces it.
constexpr double kTransposeMinWork = 67108864.0;
constexpr const char* kTransposePrefix = "transpose_";

size_t round256(size_t n) { return (n + 255) / 256 * 256; }
size_t xkt_bytes(const Geometry& g, int64_t Tp) { return round256((size_t)g.K * Tp * g.eb); }
size_t ykt_bytes(const Geometry& g, int64_t Tp, int ydt) { return round256((size_t)g.R * Tp * nm::dtype_bytes(ydt)); }

Call transposed_call(const Call& c, int64_t Tp) {
  const void* al = reinterpret_cast<const void*>((uintptr_t)256);
  return make_call(*c.g, c.wdt, c.ydt, Tp, Tp, Tp, al, al, c.act, NM_LAYOUT_KT);
}

size_t plan_workspace(const Plan& p, const Call& c) {
  if (p.repack) return repack_bytes(p.g24);
  if (p.split) return 2 * split_layer_bytes(p.g24);
  if (p.transpose)
    return xkt_bytes(*c.g, p.Tp) + ykt_bytes(*c.g, p.Tp, c.ydt) + (p.S > 1 ? (size_t)p.S * c.g->R * p.Tp * 4 : 0);
  return workspace_for(p.v, c);
}

Plan plan_for(const Call& c) {
  Plan p;
  p.v = choose(c);
  const Forced fv = forced();
  const char* force = fv.name;
  const bool forced = force[0] != 0;
  const bool forced_rp = forced && strncmp(force, kRepackPrefix, strlen(kRepackPrefix)) == 0;
  const bool forced_tr = forced && strncmp(force, kTransposePrefix, strlen(kTransposePrefix)) == 0;
  const double work = (double)c.g->R * (double)c.g->K * (double)c.T;

  // two-layer split (its own variant)
  if (p.v == V_SPLIT24_I8WS || p.v == V_SPLIT24_I8WSTK) {
    p.split = true;
    p.g24 = geometry24(*c.g);
    return p;
  }

  // 2:4 re-pack
  if (nm::repack24_supported(*c.g) && (!forced || forced_rp) &&
      (forced_rp || (c.wdt == NM_I8 && (p.v == V_EXPAND || p.v == V_GENERIC) && work >= kRepackMinWork))) {
    const Geometry g24 = Geometry::make(c.g->R, c.g->K, 2, 4, c.g->eb);
    Call c24 = c;
    c24.g = &g24;
    Variant inner = V_INVALID;
    if (forced_rp) {
      const char* name = force + strlen(kRepackPrefix);
      for (int v = V_GENERIC; v < V_COUNT; ++v)
        if (repack_inner((Variant)v) && strcmp(name, variant_name((Variant)v)) == 0 && eligible((Variant)v, c24))
          inner = (Variant)v;
    } else {
      inner = choose_auto(c24);
    }
    // a forced re-pack runs the 2:4 kernel unsplit
    if (repack_inner(inner) && (forced_rp || ksplit_for(inner, c24) == 1)) {
      p.v = inner;
      p.repack = true;
      p.g24 = g24;
      return p;
    }
  }

  // [T][K] through the [K][T] kernels
  if (c.layout == NM_LAYOUT_TK && (!forced || forced_tr) &&
      (forced_tr || (p.v == V_GENERIC && work >= kTransposeMinWork))) {
    const int64_t Tp = (c.T + 15) / 16 * 16;
    const Call ckt = transposed_call(c, Tp);
    Variant inner = V_INVALID;
    if (forced_tr) {
      const char* name = force + strlen(kTransposePrefix);
      for (int v = V_GENERIC + 1; v < V_COUNT; ++v)
        if (strcmp(name, variant_name((Variant)v)) == 0 && eligible((Variant)v, ckt)) inner = (Variant)v;
    } else {
      inner = choose_auto(ckt, false);
    }
    if (inner != V_INVALID && inner != V_GENERIC && inner != V_SPLIT24_I8WS && inner != V_SPLIT24_I8WSTK) {
      p.v = inner;
      p.transpose = true;
      p.Tp = Tp;
      p.S = ksplit_for(inner, ckt);
    }
  }
  return p;
}

const char* plan_name(const Plan& p) {
  if (p.transpose) {
    static char names[V_COUNT][96];
    static const bool init = [] {
      for (int v = 0; v < V_COUNT; ++v)
        snprintf(names[v], sizeof names[v], "%s%s", kTransposePrefix, variant_name((Variant)v));
      return true;
    }();
    (void)init;
    return names[p.v];
  }
  if (!p.repack) return variant_name(p.v);
  switch (p.v) {
    case V_SMFMAC_I8P: return "repack24_smfmac_i8_2of4_persistent";
    case V_SMFMAC_I8P8: return "repack24_smfmac_i8_2of4_persistent_w8";
    case V_SMFMAC_I8WS: return "repack24_smfmac_i8_2of4_stationary";
    case V_SMFMAC_H: return "repack24_smfmac_h_2of4_persistent";
    case V_SMFMAC_I8TK: return "repack24_smfmac_i8_2of4_tk";
    case V_SMFMAC_I8WSTK: return "repack24_smfmac_i8_2of4_stationary_tk";
    default: return "invalid";
  }
}

}  // namespace

extern "C" {

nm_status nm_pack_size(int64_t rows, int64_t K, int32_t N, int32_t M, int32_t dtype,
                       size_t* values_bytes, size_t* meta_bytes) {
  if (!values_bytes || !meta_bytes) return NM_EINVAL;
  nm_status st = check_shape(rows, K, N, M, dtype);
  if (st != NM_OK) return st;
  Geometry g = Geometry::make(rows, K, N, M, nm::dtype_bytes(dtype));
  *values_bytes = g.values_bytes();
  *meta_bytes = g.meta_bytes();
  return NM_OK;
}

nm_status nm_pack(const void* W, int64_t ldw, nm_packed* desc, void* stream) {
  if (!W || !desc) return NM_EINVAL;
  nm_status st = check_shape(desc->rows, desc->K, desc->N, desc->M, desc->dtype);
  if (st != NM_OK) return st;
  if (ldw < desc->K) return NM_EINVAL;
  Geometry g = Geometry::make(desc->rows, desc->K, desc->N, desc->M, nm::dtype_bytes(desc->dtype));
  if (!desc->values || desc->values_bytes != g.values_bytes()) return NM_EINVAL;
  if (g.w != 0 && (!desc->meta || desc->meta_bytes != g.meta_bytes())) return NM_EINVAL;
  if (!aligned(W, (size_t)g.eb)) return NM_EUNSUPPORTED;
  if (!aligned(desc->values, 16) || (g.w != 0 && !aligned(desc->meta, 16))) return NM_EUNSUPPORTED;
  hipError_t e = nm::launch_pack(W, ldw, g, desc->dtype, static_cast<uint8_t*>(desc->values),
                                 g.w ? static_cast<uint8_t*>(desc->meta) : nullptr,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return NM_EHIP;
  desc->format_version = NM_FORMAT_VERSION;
  return NM_OK;
}

nm_status nm_spmm_workspace_size(const nm_packed* w, int64_t T, int32_t y_dtype, size_t* bytes) {
  if (!bytes) return NM_EINVAL;
  Geometry g;
  nm_status st = check_desc(w, &g);
  if (st != NM_OK) return st;
  if (T < 1) return NM_EINVAL;
  if (!pair_supported(w->dtype, y_dtype)) return NM_EUNSUPPORTED;
  // the variant may depend on strides and alignment; report the largest need
  const void* al = reinterpret_cast<const void*>((uintptr_t)256);
  const Call c = make_call(g, w->dtype, y_dtype, T, T, T, al, al);
  size_t need = 0;
  for (int v = V_GENERIC; v < V_COUNT; ++v) {
    size_t n = workspace_for((Variant)v, c);
    if (n > need) need = n;
  }
  for (int act = NM_ACT_NONE; act <= NM_ACT_GELU; ++act) {
    const Call lc = make_call(g, w->dtype, y_dtype, T, T, T, al, al, act);
    const size_t n = plan_workspace(plan_for(lc), lc);
    if (n > need) need = n;
  }
  *bytes = need;
  return NM_OK;
}

nm_status nm_spmm_tk_workspace_size(const nm_packed* w, int64_t T, int32_t y_dtype, size_t* bytes) {
  if (!bytes) return NM_EINVAL;
  Geometry g;
  nm_status st = check_desc(w, &g);
  if (st != NM_OK) return st;
  if (T < 1) return NM_EINVAL;
  if (!pair_supported(w->dtype, y_dtype)) return NM_EUNSUPPORTED;
  const void* al = reinterpret_cast<const void*>((uintptr_t)256);
  size_t need = 0;
  for (int act = NM_ACT_NONE; act <= NM_ACT_GELU; ++act) {
    const Call lc = make_call(g, w->dtype, y_dtype, T, g.K, g.R, al, al, act, NM_LAYOUT_TK);
    const size_t n = plan_workspace(plan_for(lc), lc);
    if (n > need) need = n;
  }
  *bytes = need;
  return NM_OK;
}

}  // extern "C"

namespace {

// One [K][T]-or-[T][K] product with variant v: K split into S slices (raw
// partial sums at `part`, then the reduction applies a's epilogue) or one
// launch.
// The three-layer kernel's schedule on a plain 2:4 weight (its Sparse-TC
// layer alone): same 16-row x 64-column blocks, same position words.
hipError_t launch_stream24(const SpmmArgs& s24, hipStream_t s) {
  nm::HybridArgs a{};
  a.R = s24.g.R;
  a.K = s24.g.K;
  a.nRB = s24.g.nRB;
  a.nKB = s24.g.nKB;
  a.nSeg = (a.nKB + 7) / 8;
  a.wdt = s24.wdt;
  a.ydt = s24.ydt;
  a.act = s24.act;
  a.values = s24.values;
  a.meta = s24.meta;
  a.codes = s24.meta;          // unused by the plain form
  a.res_ptr = nullptr;
  a.res_ent = nullptr;
  a.values_bytes = (int64_t)s24.g.values_bytes();
  a.meta_bytes = (int64_t)s24.g.meta_bytes();
  a.X = s24.X;
  a.ldx = s24.ldx;
  a.T = s24.T;
  a.Y = s24.Y;
  a.ldy = s24.ldy;
  a.bias = static_cast<const float*>(s24.bias);
  const int64_t cus = device_cus();
  const int64_t mrb = nm::kHybridMaxRB[0], nw = nm::kHybridWaves[0];
  a.G = (int)std::max<int64_t>((a.nRB + mrb - 1) / mrb, std::min<int64_t>(a.nRB, cus));
  a.nChunk = (int)((a.nSeg + nw - 1) / nw);
  a.patch_last = (a.T & 1) && a.ldx == a.T;
  return nm::launch_spmm_hybrid(a, false, s);
}

nm_status run_variant(Variant v, int S, const SpmmArgs& a, void* part, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (S > 1) {
    // K slices write raw 32-bit partial sums to the workspace; the reduction
    // adds them and applies this call's epilogue
    SpmmArgs p = a;
    p.ydt = a.wdt == NM_I8 ? NM_I32 : NM_F32;
    p.Y = part;
    p.ldy = a.T;
    p.bias = nullptr;
    p.scale = nullptr;
    p.act = NM_ACT_NONE;
    p.ksplit = S;
    p.kbs = (int)(a.g.nKB / S);
    p.ys = a.g.R * a.T;
    e = v == V_SMFMAC_H ? nm::launch_spmm_smfmac_h(p, s) : nm::launch_spmm_expand(p, s);
    if (e != hipSuccess) return NM_EHIP;
    SpmmArgs r = a;
    r.ksplit = S;
    r.ys = p.ys;
    r.ws = part;
    e = nm::launch_splitk_reduce(r, s);
    return e == hipSuccess ? NM_OK : NM_EHIP;
  }
  switch (v) {
    case V_GENERIC: e = nm::launch_spmm_generic(a, s); break;
    case V_SMFMAC_I8P: e = nm::launch_spmm_smfmac_i8p(a, 0, s); break;
    case V_SMFMAC_I8P8: e = nm::launch_spmm_smfmac_i8p(a, 1, s); break;
    case V_SMFMAC_I8WS: e = nm::launch_spmm_smfmac_i8ws(a, s); break;
    case V_SMFMAC_I8SM: e = nm::launch_spmm_smfmac_i8small(a, s); break;
    case V_SMFMAC_H: e = nm::launch_spmm_smfmac_h(a, s); break;
    case V_SMFMAC_HD: e = nm::launch_spmm_smfmac_hd(a, s); break;
    case V_EXPAND: e = nm::launch_spmm_expand(a, s); break;
    case V_EXPAND_DECODE: e = nm::launch_spmm_expand_decode(a, s); break;
    case V_SMFMAC_I8TK: e = nm::launch_spmm_smfmac_i8tk(a, s); break;
    case V_SMFMAC_I8WSTK: e = nm::launch_spmm_smfmac_i8wstk(a, s); break;
    case V_STREAM24: e = launch_stream24(a, s); break;
    case V_SPLIT24_I8WS:
    case V_SPLIT24_I8WSTK: e = nm::launch_spmm_smfmac_i8ws2(a, s); break;
    case V_DENSE24_I8WS:
    case V_DENSE24_I8WSTK: e = nm::launch_spmm_smfmac_i8ws2_dense(a, s); break;
    default: return NM_EINVAL;
  }
  return e == hipSuccess ? NM_OK : NM_EHIP;
}

nm_status spmm_call(const nm_packed* w, const void* X, int64_t ldx, int64_t T, void* Y, int64_t ldy,
                    int32_t y_dtype, const void* bias, const float* scale, int32_t act, float out_scale,
                    int layout, void* workspace, size_t workspace_bytes, void* stream) {
  Geometry g;
  nm_status st = check_desc(w, &g);
  if (st != NM_OK) return st;
  if (w->format_version != NM_FORMAT_VERSION) return NM_EINVAL;
  if (!X || !Y || T < 1) return NM_EINVAL;
  if (layout == NM_LAYOUT_KT && (ldx < T || ldy < T)) return NM_EINVAL;
  if (layout == NM_LAYOUT_TK && (ldx < g.K || ldy < g.R)) return NM_EINVAL;
  if (!pair_supported(w->dtype, y_dtype)) return NM_EUNSUPPORTED;
  if (act != NM_ACT_NONE && act != NM_ACT_GELU) return NM_EUNSUPPORTED;
  if (act != NM_ACT_NONE && y_dtype == NM_I32) return NM_EUNSUPPORTED;
  if (!(out_scale - out_scale == 0.0f)) return NM_EINVAL;   // not finite
  if (y_dtype == NM_I8 && !scale) return NM_EINVAL;
  if (!aligned(X, (size_t)g.eb) || !aligned(Y, (size_t)nm::dtype_bytes(y_dtype))) return NM_EUNSUPPORTED;
  if (bias && !aligned(bias, 4)) return NM_EUNSUPPORTED;
  if (scale && !aligned(scale, 4)) return NM_EUNSUPPORTED;
  const Call call = make_call(g, w->dtype, y_dtype, T, ldx, ldy, X, Y, act, layout);
  Plan pl = plan_for(call);
  // a workspace too small (or not 256-byte aligned) for the re-packed copy
  // or the transposed operands: the kernel the plain choice gives (same
  // result)
  if ((pl.repack || pl.transpose || pl.split) &&
      (!workspace || workspace_bytes < plan_workspace(pl, call) || !aligned(workspace, 256))) {
    pl = Plan();
    pl.v = choose(call, false);
  }
  const Variant v = pl.v;
  const int S = pl.repack ? 1 : pl.transpose ? pl.S : ksplit_for(v, call);
  const size_t need = plan_workspace(pl, call);
  if (workspace_bytes < need || (need && !workspace)) return NM_EINVAL;
  if (need && !aligned(workspace, 16)) return NM_EUNSUPPORTED;

  SpmmArgs a;
  a.g = g;
  a.wdt = w->dtype;
  a.ydt = y_dtype;
  a.values = static_cast<const uint8_t*>(w->values);
  a.meta = g.w ? static_cast<const uint8_t*>(w->meta) : nullptr;
  a.X = X;
  a.ldx = ldx;
  a.T = T;
  a.Y = Y;
  a.ldy = ldy;
  a.bias = bias;
  a.scale = (y_dtype == NM_I8) ? scale : nullptr;
  a.ws = workspace;
  a.ws_bytes = workspace_bytes;
  a.ksplit = 1;
  a.kbs = (int)g.nKB;
  a.ys = 0;
  a.act = act;
  a.out_scale = out_scale;
  a.layout = layout;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (pl.repack) {
    uint8_t* wv = static_cast<uint8_t*>(workspace);
    uint8_t* wm = static_cast<uint8_t*>(workspace) + repack_meta_off(pl.g24);
    e = nm::launch_repack24(g, a.values, a.meta, pl.g24, wv, wm, s);
    if (e != hipSuccess) return NM_EHIP;
    a.g = pl.g24;
    a.values = wv;
    a.meta = wm;
  }
  if (pl.split) {
    uint8_t* l0 = static_cast<uint8_t*>(workspace);
    uint8_t* l1 = l0 + split_layer_bytes(pl.g24);
    const size_t mo = repack_meta_off(pl.g24);
    e = nm::launch_split24(g, a.values, a.meta, pl.g24, l0, l0 + mo, l1, l1 + mo, s);
    if (e != hipSuccess) return NM_EHIP;
    a.g = pl.g24;
    a.values = l0;
    a.meta = l0 + mo;
    a.values2 = l1;
    a.meta2 = l1 + mo;
  }
  if (pl.transpose) {
    // X [T][K] -> X' [K][T'], the [K][T] product into Y' [R][T'], Y' -> Y [T][R]
    uint8_t* xkt = static_cast<uint8_t*>(workspace);
    uint8_t* ykt = xkt + xkt_bytes(g, pl.Tp);
    void* part = ykt + ykt_bytes(g, pl.Tp, y_dtype);
    e = nm::launch_transpose(X, T, g.K, ldx, xkt, pl.Tp, pl.Tp, g.eb, s);
    if (e != hipSuccess) return NM_EHIP;
    SpmmArgs k = a;
    k.X = xkt;
    k.ldx = pl.Tp;
    k.T = pl.Tp;
    k.Y = ykt;
    k.ldy = pl.Tp;
    k.layout = NM_LAYOUT_KT;
    k.ws = part;
    const nm_status r = run_variant(v, S, k, part, s);
    if (r != NM_OK) return r;
    e = nm::launch_transpose(ykt, g.R, T, pl.Tp, Y, ldy, g.R, nm::dtype_bytes(y_dtype), s);
    return e == hipSuccess ? NM_OK : NM_EHIP;
  }
  return run_variant(v, S, a, workspace, s);
}

}  // namespace

// ---- scratch for callers that cannot allocate (nm_spmm_noalloc).  One
// copy of this array per device, held until the process ends.  In host code
// its name is a host-side stand-in: every host use goes through the device
// address hipGetSymbolAddress returns, cached per device.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

namespace {

std::atomic<void*> g_scratch[64];
std::mutex g_scratch_mu;

// the calling thread's current device's copy of `scratch` (nullptr on error)
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

nm_status nm_spmm_noalloc(const nm_packed* w, const void* X, int64_t ldx, int64_t T, void* Y, int64_t ldy,
                          int32_t y_dtype, const void* bias, const float* scale, int32_t act, float out_scale,
                          void* stream) {
  void* ws = scratch_ptr();
  if (!ws) return NM_EHIP;
  // the plan of nm_spmm_act given kScratchBytes of workspace: a K split whose
  // partial sums exceed it is rejected (NM_EINVAL); a re-pack or transpose
  // copy that does not fit runs the plain kernel, as with any small workspace
  return spmm_call(w, X, ldx, T, Y, ldy, y_dtype, bias, scale, act, out_scale, NM_LAYOUT_KT, ws, kScratchBytes,
                   stream);
}

size_t nm_spmm_noalloc_max_bytes(void) { return kScratchBytes; }

nm_status nm_spmm_act(const nm_packed* w, const void* X, int64_t ldx, int64_t T, void* Y, int64_t ldy,
                      int32_t y_dtype, const void* bias, const float* scale, int32_t act, float out_scale,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return spmm_call(w, X, ldx, T, Y, ldy, y_dtype, bias, scale, act, out_scale, NM_LAYOUT_KT, workspace,
                   workspace_bytes, stream);
}

nm_status nm_spmm_tk(const nm_packed* w, const void* Xt, int64_t ldx, int64_t T, void* Yt, int64_t ldy,
                     int32_t y_dtype, const void* bias, const float* scale, int32_t act, float out_scale,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return spmm_call(w, Xt, ldx, T, Yt, ldy, y_dtype, bias, scale, act, out_scale, NM_LAYOUT_TK, workspace,
                   workspace_bytes, stream);
}

nm_status nm_spmm(const nm_packed* w, const void* X, int64_t ldx, int64_t T, void* Y, int64_t ldy,
                  int32_t y_dtype, const void* bias, const float* scale, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return nm_spmm_act(w, X, ldx, T, Y, ldy, y_dtype, bias, scale, NM_ACT_NONE, 1.0f, workspace, workspace_bytes,
                     stream);
}

const char* nm_status_str(nm_status s) {
  switch (s) {
    case NM_OK: return "NM_OK: success";
    case NM_EINVAL: return "NM_EINVAL: invalid argument";
    case NM_EUNSUPPORTED: return "NM_EUNSUPPORTED: unsupported configuration";
    case NM_EHIP: return "NM_EHIP: HIP runtime error at launch";
    default: return "unknown nm_status";
  }
}

const char* nm_spmm_variant_act(const nm_packed* w, int64_t T, int32_t y_dtype, int32_t act) {
  Geometry g;
  if (check_desc(w, &g) != NM_OK || T < 1 || !pair_supported(w->dtype, y_dtype)) return "invalid";
  if ((act != NM_ACT_NONE && act != NM_ACT_GELU) || (act != NM_ACT_NONE && y_dtype == NM_I32)) return "invalid";
  // dense row-major operands, 256-byte aligned (what a fresh allocation gives)
  const void* al = reinterpret_cast<const void*>((uintptr_t)256);
  return plan_name(plan_for(make_call(g, w->dtype, y_dtype, T, T, T, al, al, act)));
}

const char* nm_spmm_variant(const nm_packed* w, int64_t T, int32_t y_dtype) {
  return nm_spmm_variant_act(w, T, y_dtype, NM_ACT_NONE);
}

const char* nm_spmm_variant_tk(const nm_packed* w, int64_t T, int32_t y_dtype, int32_t act) {
  Geometry g;
  if (check_desc(w, &g) != NM_OK || T < 1 || !pair_supported(w->dtype, y_dtype)) return "invalid";
  if ((act != NM_ACT_NONE && act != NM_ACT_GELU) || (act != NM_ACT_NONE && y_dtype == NM_I32)) return "invalid";
  const void* al = reinterpret_cast<const void*>((uintptr_t)256);
  return plan_name(plan_for(make_call(g, w->dtype, y_dtype, T, g.K, g.R, al, al, act, NM_LAYOUT_TK)));
}

int32_t nm_spmm_ksplit(const nm_packed* w, int64_t T, int32_t y_dtype, int32_t act) {
  Geometry g;
  if (check_desc(w, &g) != NM_OK || T < 1 || !pair_supported(w->dtype, y_dtype)) return 0;
  if ((act != NM_ACT_NONE && act != NM_ACT_GELU) || (act != NM_ACT_NONE && y_dtype == NM_I32)) return 0;
  const void* al = reinterpret_cast<const void*>((uintptr_t)256);
  const Call c = make_call(g, w->dtype, y_dtype, T, T, T, al, al, act);
  const Plan p = plan_for(c);
  return p.repack ? 1 : ksplit_for(p.v, c);
}

}  // extern "C"

// ---------------------------------------------------------------- three-layer format
namespace {

bool hy_sizes_ok(const nm_hybrid* w, int64_t nRB, int64_t nKB, int64_t nSeg) {
  if ((int64_t)w->values_bytes != nRB * nKB * 1024 || (int64_t)w->meta_bytes != nRB * nKB * 128) return false;
  if ((int64_t)w->codes_bytes != nRB * nSeg * 512) return false;
  if ((int64_t)w->res_ptr_bytes != (nRB * nSeg * 16 + 1) * 4) return false;
  if (w->n_res < 0 || (int64_t)w->res_ent_bytes != w->n_res * 4) return false;
  return w->values && w->meta && w->codes && w->res_ptr && (w->n_res == 0 || w->res_ent);
}

}  // namespace

extern "C" {

nm_status nm_hybrid_spmm(const nm_hybrid* w, const void* X, int64_t ldx, int64_t T, void* Y, int64_t ldy,
                         int32_t y_dtype, const void* bias, int32_t act, void* stream) {
  if (!w || !X || !Y || T < 1 || ldx < T || ldy < T) return NM_EINVAL;
  if (w->rows < 1 || w->K < 4 || w->K % 4) return NM_EINVAL;
  if (w->dtype != NM_F16 && w->dtype != NM_BF16) return NM_EUNSUPPORTED;
  if (y_dtype != w->dtype && y_dtype != NM_F32) return NM_EUNSUPPORTED;
  if (act != NM_ACT_NONE && act != NM_ACT_GELU) return NM_EINVAL;
  if (w->format_version != NM_FORMAT_VERSION) return NM_EUNSUPPORTED;
  const int64_t nRB = (w->rows + 15) / 16, nKB = (w->K + 63) / 64, nSeg = (nKB + 7) / 8;
  if (!hy_sizes_ok(w, nRB, nKB, nSeg)) return NM_EINVAL;
  if (!aligned(w->values, 16) || !aligned(w->meta, 16) || !aligned(w->codes, 16) || !aligned(w->res_ptr, 16) ||
      (w->res_ent && !aligned(w->res_ent, 16)) || !aligned(X, 2))
    return NM_EUNSUPPORTED;
  // 32-bit buffer offsets
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)w->values_bytes >= lim || (int64_t)w->res_ent_bytes >= lim || w->K * ldx * 2 >= lim ||
      (int64_t)w->codes_bytes >= lim)
    return NM_EUNSUPPORTED;
  nm::HybridArgs a{};
  a.R = w->rows;
  a.K = w->K;
  a.nRB = nRB;
  a.nKB = nKB;
  a.nSeg = nSeg;
  a.wdt = w->dtype;
  a.ydt = y_dtype;
  a.act = act;
  a.values = static_cast<const uint8_t*>(w->values);
  a.meta = static_cast<const uint8_t*>(w->meta);
  a.codes = static_cast<const uint8_t*>(w->codes);
  a.res_ptr = static_cast<const int32_t*>(w->res_ptr);
  a.res_ent = w->n_res ? static_cast<const uint32_t*>(w->res_ent) : reinterpret_cast<const uint32_t*>(w->res_ptr);
  a.values_bytes = (int64_t)w->values_bytes;
  a.meta_bytes = (int64_t)w->meta_bytes;
  a.codes_bytes = (int64_t)w->codes_bytes;
  a.res_ptr_bytes = (int64_t)w->res_ptr_bytes;
  // with no residual the entry loads read the row pointers instead (in range, unused)
  a.res_ent_bytes = w->n_res ? (int64_t)w->res_ent_bytes : (int64_t)w->res_ptr_bytes;
  a.X = X;
  a.ldx = ldx;
  a.T = T;
  a.Y = Y;
  a.ldy = ldy;
  a.bias = static_cast<const float*>(bias);
  // one workgroup per compute unit walking row blocks b, b + G, ...; at most
  // kHybridMaxRB[1] row blocks each
  const int64_t cus = device_cus();
  const int64_t mrb = nm::kHybridMaxRB[1], nw = nm::kHybridWaves[1];
  a.G = (int)std::max<int64_t>((nRB + mrb - 1) / mrb, std::min<int64_t>(nRB, cus));
  a.nChunk = (int)((nSeg + nw - 1) / nw);
  a.patch_last = (T & 1) && ldx == T;
  return nm::launch_spmm_hybrid(a, true, static_cast<hipStream_t>(stream)) == hipSuccess ? NM_OK : NM_EHIP;
}

}  // extern "C"
