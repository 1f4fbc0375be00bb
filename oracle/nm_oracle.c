/*
 * nm_oracle.c -- plain, slow, obviously-correct CPU oracle for the N:M
 * semi-structured sparse weight x dense activation product
 *
 *     Y = epilogue( (mask (.) W) . X )
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP library; it is built with gcc, not hipcc.
 *
 * What it follows (paper: "Realizable N:M Sparse Transformer Inference via
 * Search-Kernel Co-Design", arXiv 2607.12505):
 *   - Sec. 2.1: N:M sparsity keeps N nonzero weights in every group of M.
 *   - Sec. 4.2: micro-dense execution computes only on the N kept values of
 *     each window, stored packed with their in-window positions; it changes
 *     how the product is executed, not what it equals.  The oracle is
 *     therefore the plain definition written out.
 *   - The selection rule (top-N by |w| along K) and the int8 requantising
 *     epilogue are readings where the pages are silent; they are listed with
 *     the packed-format reader in the design notes and restated at each
 *     function below.
 *
 * Integer inputs accumulate exactly in int64.  fp16/bf16 inputs are decoded to
 * fp64 and products (exact in fp64) are summed in fp64 in ascending k order.
 * Rounding to an output dtype is left to the caller.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* oracle-private dtype codes */
enum { ORC_I8 = 0, ORC_F16 = 1, ORC_BF16 = 2 };

static int elt_bytes(int dt) { return dt == ORC_I8 ? 1 : 2; }

/* IEEE-754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double f16_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);                    /* subnormal: f * 2^-24 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);        /* (1.f) * 2^(e-15) */
  return s ? -v : v;
}

/* bfloat16 is the upper 16 bits of an IEEE binary32. */
static double bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* element i of a W/X buffer as a double (exact for all three dtypes) */
static double elem(const void* p, int dt, int64_t i) {
  if (dt == ORC_I8) return (double)((const int8_t*)p)[i];
  uint16_t h = ((const uint16_t*)p)[i];
  return dt == ORC_F16 ? f16_to_f64(h) : bf16_to_f64(h);
}

static int check_nm(int64_t R, int64_t K, int N, int M, int dt) {
  if (R < 0 || K < 0 || M <= 0 || M > 64 || N < 1 || N > M || K % M) return -1;
  if (dt < ORC_I8 || dt > ORC_BF16) return -1;
  return 0;
}

/*
 * orc_compress: choose the kept set of every group and emit it in canonical
 * form.  vals[r][g][j] (raw W element bytes) and idx[r][g][j] (in-group
 * position 0..M-1), j = 0..N-1 in ascending position order.
 *
 * Selection (N:M constraint, paper Sec. 2.1; criterion "largest magnitude"):
 * order the M members of a group by magnitude descending, equal magnitudes by
 * position ascending (a stable sort of the position-ordered group), and keep
 * the first N.  Exactly N slots are kept per group, even when some kept
 * values are zero.
 *
 * Magnitude of a non-finite fp16 / bf16 weight (the pages only meet finite
 * weights; this is the reading the library's header documents): every
 * infinity ranks above every finite value, every NaN above every infinity,
 * and NaNs rank among themselves by their payload (the fraction field read as
 * an unsigned integer); the sign never matters.  See sel_key / sel_beats.
 */
/* Selection key of one weight: a class (0 finite, 1 infinite, 2 NaN) and,
 * inside the class, |w| (finite) or the NaN payload.  Decoded from the raw
 * element bits field by field, independently of elem(). */
typedef struct {
  int cls;
  double mag;
  uint32_t payload;
} sel_key_t;

static sel_key_t sel_key(const void* p, int dt, int64_t i) {
  sel_key_t k = {0, 0.0, 0};
  if (dt == ORC_I8) {
    k.mag = fabs((double)((const int8_t*)p)[i]);
    return k;
  }
  const uint16_t h = ((const uint16_t*)p)[i];
  /* binary16: exponent bits 14..10, fraction 9..0; bfloat16: exponent bits
   * 14..7, fraction 6..0.  An all-ones exponent is an infinity (zero
   * fraction) or a NaN (nonzero fraction). */
  const uint32_t emax = dt == ORC_F16 ? 0x1Fu : 0xFFu;
  const int fbits = dt == ORC_F16 ? 10 : 7;
  const uint32_t e = (h >> fbits) & emax, f = h & ((1u << fbits) - 1u);
  if (e == emax) {
    k.cls = f ? 2 : 1;
    k.payload = f;
    return k;
  }
  k.mag = fabs(elem(p, dt, i));
  return k;
}

/* a ranks strictly above b by magnitude */
static int sel_beats(sel_key_t a, sel_key_t b) {
  if (a.cls != b.cls) return a.cls > b.cls;
  if (a.cls == 0) return a.mag > b.mag;
  return a.payload > b.payload;
}

int orc_compress(const void* W, int64_t R, int64_t K, int N, int M, int dt,
                 void* vals, uint8_t* idx) {
  if (check_nm(R, K, N, M, dt)) return -1;
  int b = elt_bytes(dt);
  int64_t G = K / M;
  int order[64];
  sel_key_t mag[64];
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t g = 0; g < G; ++g) {
      int64_t base = r * K + g * M;
      for (int i = 0; i < M; ++i) {
        order[i] = i;
        mag[i] = sel_key(W, dt, base + i);
      }
      /* stable insertion sort by magnitude, descending: an element moves
       * ahead only past members it strictly beats */
      for (int i = 1; i < M; ++i) {
        int cur = order[i];
        int j = i - 1;
        while (j >= 0 && sel_beats(mag[cur], mag[order[j]])) {
          order[j + 1] = order[j];
          --j;
        }
        order[j + 1] = cur;
      }
      /* the first N, back in ascending position order */
      int keep[64];
      for (int j = 0; j < N; ++j) keep[j] = order[j];
      for (int i = 1; i < N; ++i) {
        int cur = keep[i];
        int j = i - 1;
        while (j >= 0 && keep[j] > cur) {
          keep[j + 1] = keep[j];
          --j;
        }
        keep[j + 1] = cur;
      }
      int64_t out = (r * G + g) * N;
      for (int j = 0; j < N; ++j) {
        idx[out + j] = (uint8_t)keep[j];
        memcpy((char*)vals + (out + j) * b, (const char*)W + (base + keep[j]) * b, b);
      }
    }
  }
  return 0;
}

/* orc_decompress: Wm = mask (.) W as a zero-filled dense [R][K] matrix of the
 * same dtype (kept slots restored at their positions). */
int orc_decompress(const void* vals, const uint8_t* idx, int64_t R, int64_t K, int N, int M,
                   int dt, void* Wm) {
  if (check_nm(R, K, N, M, dt)) return -1;
  int b = elt_bytes(dt);
  int64_t G = K / M;
  memset(Wm, 0, (size_t)(R * K * b));
  for (int64_t r = 0; r < R; ++r)
    for (int64_t g = 0; g < G; ++g)
      for (int j = 0; j < N; ++j) {
        int64_t s = (r * G + g) * N + j;
        if (idx[s] >= M) return -2;
        memcpy((char*)Wm + (r * K + g * M + idx[s]) * b, (const char*)vals + s * b, b);
      }
  return 0;
}

/*
 * O1, orc_spmm_dense: naive triple loop over the decompressed matrix,
 * acc[r][t] = sum_{k=0..K-1} Wm[r][k] * X[k][t], k ascending.
 * X is [K][T] row-major (tokens contiguous).  Integer dtype: acc is int64
 * (acc_i); fp dtypes: acc is double (acc_f).  The unused pointer may be NULL.
 */
int orc_spmm_dense(const void* Wm, const void* X, int64_t R, int64_t K, int64_t T, int dt,
                   int64_t* acc_i, double* acc_f) {
  if (R < 0 || K < 0 || T < 0 || dt < ORC_I8 || dt > ORC_BF16) return -1;
  for (int64_t r = 0; r < R; ++r)
    for (int64_t t = 0; t < T; ++t) {
      if (dt == ORC_I8) {
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k)
          s += (int64_t)((const int8_t*)Wm)[r * K + k] * (int64_t)((const int8_t*)X)[k * T + t];
        acc_i[r * T + t] = s;
      } else {
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) s += elem(Wm, dt, r * K + k) * elem(X, dt, k * T + t);
        acc_f[r * T + t] = s;
      }
    }
  return 0;
}

/*
 * O2, orc_spmm_direct: loop straight over the compressed representation,
 * acc[r][t] += vals[r][g][j] * X[g*M + idx[r][g][j]][t], for g, j ascending
 * (so k ascending, the same addition order as O1 over the nonzero products).
 *
 * Computes only the rows listed in rows[0..nrows-1] (rows == NULL: all R rows,
 * nrows ignored); output row i of acc belongs to rows[i].  OpenMP splits the
 * listed rows statically over nthreads threads (<= 0: the runtime default).
 */
int orc_spmm_direct(const void* vals, const uint8_t* idx, const void* X, int64_t R, int64_t K,
                    int64_t T, int N, int M, int dt, const int64_t* rows, int64_t nrows,
                    int64_t* acc_i, double* acc_f, int nthreads) {
  if (check_nm(R, K, N, M, dt) || T < 0) return -1;
  if (!rows) nrows = R;
  for (int64_t i = 0; i < nrows; ++i)
    if (rows && (rows[i] < 0 || rows[i] >= R)) return -1;
  int64_t G = K / M;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
  for (int64_t i = 0; i < nrows; ++i) {
    int64_t r = rows ? rows[i] : i;
    if (dt == ORC_I8) {
      int64_t* a = acc_i + i * T;
      for (int64_t t = 0; t < T; ++t) a[t] = 0;
      for (int64_t g = 0; g < G; ++g)
        for (int j = 0; j < N; ++j) {
          int64_t s = (r * G + g) * N + j;
          int64_t v = ((const int8_t*)vals)[s];
          const int8_t* xr = (const int8_t*)X + (g * M + idx[s]) * T;
          for (int64_t t = 0; t < T; ++t) a[t] += v * (int64_t)xr[t];
        }
    } else {
      double* a = acc_f + i * T;
      for (int64_t t = 0; t < T; ++t) a[t] = 0.0;
      for (int64_t g = 0; g < G; ++g)
        for (int j = 0; j < N; ++j) {
          int64_t s = (r * G + g) * N + j;
          double v = elem(vals, dt, s);
          int64_t k = g * M + idx[s];
          for (int64_t t = 0; t < T; ++t) a[t] += v * elem(X, dt, k * T + t);
        }
    }
  }
  return 0;
}

/*
 * Requantising epilogue to int8 (the pages describe no epilogue; this is the
 * reading adopted for "fused bias + requant"):
 *   y = saturate_[-128,127]( round_half_even( f32(acc + bias[r]) * scale[r] ) )
 * acc + bias is an exact integer sum, its conversion to binary32 rounds to
 * nearest-even, the product is one binary32 multiply (no fused multiply-add),
 * and nearbyintf rounds half to even under the default rounding mode.
 * bias may be NULL (zero).
 */
int orc_requant_i8(const int64_t* acc, int64_t R, int64_t T, const int32_t* bias,
                   const float* scale, int8_t* y) {
  if (R < 0 || T < 0 || !scale) return -1;
  for (int64_t r = 0; r < R; ++r)
    for (int64_t t = 0; t < T; ++t) {
      int64_t a = acc[r * T + t] + (bias ? (int64_t)bias[r] : 0);
      float f = (float)a;
      volatile float p = f * scale[r]; /* one rounded binary32 product */
      float q = nearbyintf(p);
      if (q > 127.0f) q = 127.0f;
      if (q < -128.0f) q = -128.0f;
      y[r * T + t] = (int8_t)q;
    }
  return 0;
}

/*
 * GELU activation for the fused FC1 epilogue (the pages name no activation;
 * the reading adopted is the exact Gaussian-error linear unit of the ViT /
 * Swin MLP):  gelu(x) = x * Phi(x) = 0.5 * x * (1 + erf(x / sqrt(2))),
 * evaluated in binary64 with the C library's erf.
 */
static double gelu64(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }

int orc_gelu(const double* x, int64_t n, double* y) {
  if (n < 0) return -1;
  for (int64_t i = 0; i < n; ++i) y[i] = gelu64(x[i]);
  return 0;
}

/*
 * int8 output with the activation between dequantisation and
 * requantisation (reading adopted for a fused GELU on an int8 layer):
 *   p = f32(acc + bias[r]) * scale[r]          (binary32, one rounding each,
 *                                               as in orc_requant_i8)
 *   v = gelu(p) * out_scale                    (exact value, binary64)
 *   y = saturate_[-128,127]( round_half_even(v) )
 * A fast path evaluates gelu and the second product in binary32 with an erf
 * of absolute error up to 6e-7 (e.g. the rational approximation of
 * Abramowitz & Stegun eq. 7.1.26, 1.5e-7, plus binary32 rounding), so its
 * gelu is off by at most 2.5e-7 |p| + 2.4e-7 |gelu(p)| and its v by that
 * times out_scale plus one rounding (6e-8 |v|); its rounding decision may
 * therefore differ where v lies that close to a half-integer.  near[r][t] = 1
 * marks every v within max(tol, 4 x that bound) of a half-integer (the
 * caller accepts either neighbouring code there).
 */
int orc_requant_gelu_i8(const int64_t* acc, int64_t R, int64_t T, const int32_t* bias,
                        const float* scale, float out_scale, double tol, int8_t* y, uint8_t* near) {
  if (R < 0 || T < 0 || !scale) return -1;
  for (int64_t r = 0; r < R; ++r)
    for (int64_t t = 0; t < T; ++t) {
      int64_t a = acc[r * T + t] + (bias ? (int64_t)bias[r] : 0);
      float f = (float)a;
      volatile float p = f * scale[r];
      double v = gelu64((double)p) * (double)out_scale;
      double q = nearbyint(v);
      if (q > 127.0) q = 127.0;
      if (q < -128.0) q = -128.0;
      y[r * T + t] = (int8_t)q;
      double g = gelu64((double)p);
      double band = 4.0 * (fabs((double)out_scale) * (2.5e-7 * fabs((double)p) + 2.4e-7 * fabs(g)) +
                           6e-8 * fabs(v));
      if (band < tol) band = tol;
      double fr = v - floor(v);
      near[r * T + t] = (uint8_t)(fabs(fr - 0.5) <= band);
    }
  return 0;
}

/*
 * orc_read_packed: decode the GPU library's packed weight layout into the
 * canonical (vals, idx) form of orc_compress.  Written from the layout's
 * prose description, independently of the packer:
 *
 *   b = element bytes, KB = 128 / b dense columns per block, w = log2(M) index
 *   bits; a block covers 16 rows x KB columns and holds C = (KB / M) * N kept
 *   slots per row.  nRB = ceil(R / 16), nKB = ceil(K / KB); block (rb, kb) is
 *   number rb * nKB + kb.
 *   values: block n at n * 16*C*b bytes; row rr of it at rr*C*b; slot c at c*b.
 *   meta (none when N == M): block n at n * 16*MR bytes, MR = ceil(C*w/8)
 *   rounded up to a multiple of 4; row rr at rr*MR; slot c's position in bits
 *   [c*w, c*w + w) of that row, bit i being bit (i % 8) of byte i / 8.
 *   Slot c of block kb belongs to group kb*(KB/M) + c/N, kept member c % N.
 */
int orc_read_packed(const void* values, const uint8_t* meta, int64_t R, int64_t K, int N, int M,
                    int dt, void* vals, uint8_t* idx) {
  if (check_nm(R, K, N, M, dt) || (M != 4 && M != 8)) return -1;
  int b = elt_bytes(dt);
  int64_t KB = 128 / b, GB = KB / M, C = GB * N;
  int w = (M == 4) ? 2 : 3;
  int64_t MR = (C * w + 7) / 8;
  MR = (MR + 3) / 4 * 4;
  int64_t nKB = (K + KB - 1) / KB, G = K / M;
  for (int64_t r = 0; r < R; ++r)
    for (int64_t g = 0; g < G; ++g)
      for (int j = 0; j < N; ++j) {
        int64_t rb = r / 16, rr = r % 16, kb = g / GB;
        int64_t c = (g % GB) * N + j;
        int64_t blk = rb * nKB + kb;
        int64_t s = (r * G + g) * N + j;
        memcpy((char*)vals + s * b, (const char*)values + (blk * 16 * C + rr * C + c) * b, b);
        if (N == M) {
          idx[s] = (uint8_t)j;
        } else {
          const uint8_t* row = meta + blk * 16 * MR + rr * MR;
          int v = 0;
          for (int bit = 0; bit < w; ++bit) {
            int64_t pos = c * w + bit;
            v |= ((row[pos / 8] >> (pos % 8)) & 1) << bit;
          }
          idx[s] = (uint8_t)v;
        }
      }
  return 0;
}

/*
 * orc_check_padding: count violations of the packed layout's padding rule in
 * the slots that lie outside the R x K matrix (rows >= R, or groups >= K/M in
 * the last column block): each such value must be zero and each such index
 * must equal its kept-member number (0..N-1); meta bits beyond C*w in a row
 * must be zero.  Same layout description as orc_read_packed.
 */
int64_t orc_check_padding(const void* values, const uint8_t* meta, int64_t R, int64_t K, int N,
                          int M, int dt) {
  if (check_nm(R, K, N, M, dt) || (M != 4 && M != 8)) return -1;
  int b = elt_bytes(dt);
  int64_t KB = 128 / b, GB = KB / M, C = GB * N;
  int w = (M == 4) ? 2 : 3;
  int64_t MR = (C * w + 7) / 8;
  MR = (MR + 3) / 4 * 4;
  int64_t nRB = (R + 15) / 16, nKB = (K + KB - 1) / KB, G = K / M;
  int64_t bad = 0;
  for (int64_t rb = 0; rb < nRB; ++rb)
    for (int64_t kb = 0; kb < nKB; ++kb) {
      int64_t blk = rb * nKB + kb;
      for (int64_t rr = 0; rr < 16; ++rr) {
        int64_t r = rb * 16 + rr;
        const uint8_t* row = meta ? meta + blk * 16 * MR + rr * MR : NULL;
        for (int64_t c = 0; c < C; ++c) {
          int64_t g = kb * GB + c / N;
          if (r < R && g < G) continue;
          const uint8_t* v = (const uint8_t*)values + (blk * 16 * C + rr * C + c) * b;
          for (int i = 0; i < b; ++i) bad += v[i] != 0;
          if (N < M) {
            int x = 0;
            for (int bit = 0; bit < w; ++bit) {
              int64_t pos = c * w + bit;
              x |= ((row[pos / 8] >> (pos % 8)) & 1) << bit;
            }
            bad += x != (int)(c % N);
          }
        }
        if (N < M)
          for (int64_t pos = C * w; pos < MR * 8; ++pos) bad += (row[pos / 8] >> (pos % 8)) & 1;
      }
    }
  return bad;
}

/* number of threads an OpenMP region started now would use */
int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ====================================================================
 * Three-layer format for moderately unstructured fp16 / bf16 weights
 * (page "Accelerating GPU Inference of Large Language Models with
 * Moderately Unstructured Sparse Weight Matrices", Methodology 1: a
 * Sparse-TC 2:4 layer with 2-bit positions, a Slot-Filling layer whose
 * elements sit in the empty 2:4 slots with 4-bit relative distances (PDD)
 * and dummy points for long gaps, and a CSR residual layer).
 *
 * Written from this prose description of the byte image, independently of
 * the library's packer:
 *   nRB = ceil(R/16), nKB = ceil(K/64), nSeg = ceil(nKB/8).  Column block kb
 *   = columns 64kb..64kb+63; segment s = blocks 8s .. min(8s+8, nKB)-1.
 *   Rows >= R and columns >= K are zero.  A group is 4 columns 4g..4g+3.
 *   Fill unit (r, s, q), q = 0..3: in every block kb of segment s the 16
 *   columns 64kb+16q .. +15.  Its local column u = 16 (kb - 8s) + (c mod 16);
 *   its slots sigma = 8 (kb - 8s) + 2 t + j for group t = 0..3 of the quad and
 *   slot j = 0, 1.
 *   Layer 1 (values, meta) in the 2:4 packed layout: block rb*nKB+kb at
 *   1024 B (values) / 128 B (meta); row rr at 64 B / 8 B; group gb (0..15) of
 *   the block has slots 2gb, 2gb+1, value at 2 bytes each, 2-bit position at
 *   bits 2c..2c+1 of the row's 64-bit little-endian meta word.
 *     nz >= 2 nonzeros (bits & 0x7FFF != 0): the two ranked highest by the
 *       selection order (sel_key / sel_beats; ties to the lower column), in
 *       ascending column order, positions i0 < i1.
 *     nz == 1 at p: slot 0 = w_p at p; slot 1 empty, position p.
 *     nz == 0: both empty, positions 1 (slot 0) and 0 (slot 1).
 *   Surplus = nonzeros of groups with nz >= 3 that layer 1 does not hold.
 *   Layer 2 (codes): 8 bytes per fill unit at ((rb*nSeg + s)*64 + 16q + rr)*8,
 *   sixteen 4-bit codes, code i in bits 4(i%2) of byte i/2.  Greedy over the
 *   unit's surplus in ascending u, prev = -1, used = 0, f = 0, E = number of
 *   empty slots: d = u - prev, n0 = (d-1)/15; if f < E and used+n0+1 <= 16:
 *   n0 codes 0 (dummy point: advance 15, no value), then code d - 15 n0, the
 *   value goes to the f-th empty slot in ascending sigma, f++, prev = u;
 *   otherwise the element goes to layer 3.  Unused codes are 0.  Empty slots
 *   not filled hold +0.
 *   Layer 3 (res_ptr, res_ent): CSR over segment rows z = (rb*nSeg + s)*16 +
 *   rr; res_ptr[0] = 0, res_ptr[z+1] - res_ptr[z] entries of row z in
 *   ascending column, each (column - 512 s) << 16 | value bits.
 * ==================================================================== */

static int hy_nonzero(const uint16_t* W, int64_t ldw, int64_t R, int64_t K, int64_t r, int64_t c) {
  if (r >= R || c >= K) return 0;
  return (W[r * ldw + c] & 0x7FFF) != 0;
}

static uint16_t hy_at(const uint16_t* W, int64_t ldw, int64_t R, int64_t K, int64_t r, int64_t c) {
  return (r < R && c < K) ? W[r * ldw + c] : 0;
}

/* which layer holds each element: 0 zero, 1 Sparse-TC, 2 slot-filled,
 * 3 residual (layer[r*K + c]); also per fill unit the codes, and per empty
 * slot the filled value.  Shared by the byte-image writer below. */
typedef struct {
  int64_t R, K, nRB, nKB, nSeg;
} hy_geo_t;

static hy_geo_t hy_geo(int64_t R, int64_t K) {
  hy_geo_t g;
  g.R = R; g.K = K;
  g.nRB = (R + 15) / 16;
  g.nKB = (K + 63) / 64;
  g.nSeg = (g.nKB + 7) / 8;
  return g;
}

/*
 * orc_hy_encode: write the byte image of W (raw fp16 / bf16 bits, row stride
 * ldw).  values / meta / codes must hold nRB*nKB*1024, nRB*nKB*128 and
 * nRB*nSeg*512 bytes, res_ptr nRB*nSeg*16 + 1 int32.  res_ent receives at
 * most cap entries; *n_res is set to the number needed either way (call with
 * cap 0 to size it).  Returns 0, -1 on bad arguments, 1 if cap was short.
 */
int orc_hy_encode(const uint16_t* W, int64_t ldw, int64_t R, int64_t K, int dt, uint8_t* values,
                  uint8_t* meta, uint8_t* codes, int32_t* res_ptr, uint32_t* res_ent, int64_t cap,
                  int64_t* n_res) {
  if (R < 1 || K < 4 || K % 4 || ldw < K || (dt != ORC_F16 && dt != ORC_BF16)) return -1;
  hy_geo_t g = hy_geo(R, K);
  memset(values, 0, (size_t)(g.nRB * g.nKB * 1024));
  memset(meta, 0, (size_t)(g.nRB * g.nKB * 128));
  memset(codes, 0, (size_t)(g.nRB * g.nSeg * 512));
  /* residual elements per segment row, collected column-sorted afterwards */
  const int64_t nz_rows = g.nRB * g.nSeg * 16;
  int64_t total = 0;
  res_ptr[0] = 0;
  for (int64_t rb = 0; rb < g.nRB; ++rb)
    for (int64_t s = 0; s < g.nSeg; ++s)
      for (int64_t rr = 0; rr < 16; ++rr) {
        const int64_t r = rb * 16 + rr;
        const int64_t kb0 = 8 * s, kb1 = (8 * s + 8 < g.nKB) ? 8 * s + 8 : g.nKB;
        /* residual columns of this segment row, one flag per column */
        uint8_t resflag[512];
        uint16_t resval[512];
        memset(resflag, 0, sizeof resflag);
        for (int q = 0; q < 4; ++q) {
          /* pass 1: layer 1 of every group of the unit, empty slots, surplus */
          int64_t slot_col[64];     /* dense column of each slot's element, -1 if empty */
          int empty_sigma[64], E = 0;
          int sur_u[64], S = 0;
          uint16_t sur_v[64];
          const int nb = (int)(kb1 - kb0);
          for (int sg = 0; sg < 64; ++sg) slot_col[sg] = -1;
          for (int bi = 0; bi < nb; ++bi)
            for (int t = 0; t < 4; ++t) {
              const int64_t kb = kb0 + bi;
              const int gb = 4 * q + t;                 /* group within the block */
              const int64_t c0 = 64 * kb + 4 * gb;      /* first column of the group */
              int nzc = 0;
              for (int p = 0; p < 4; ++p) nzc += hy_nonzero(W, ldw, R, K, r, c0 + p);
              int sel[2] = {-1, -1}, pos[2];
              if (nzc >= 2) {
                /* rank = number of group members that beat p (ties: lower
                 * column first); the two with rank 0 and 1 are selected */
                for (int p = 0; p < 4; ++p) {
                  if (!hy_nonzero(W, ldw, R, K, r, c0 + p)) continue;
                  sel_key_t kp = sel_key(W, dt, r * ldw + c0 + p);
                  int rank = 0;
                  for (int o = 0; o < 4; ++o) {
                    if (o == p || !hy_nonzero(W, ldw, R, K, r, c0 + o)) continue;
                    sel_key_t ko = sel_key(W, dt, r * ldw + c0 + o);
                    if (sel_beats(ko, kp) || (!sel_beats(kp, ko) && o < p)) ++rank;
                  }
                  if (rank < 2) {
                    if (sel[0] < 0) sel[0] = p; else sel[1] = p;   /* p ascending */
                  }
                }
                pos[0] = sel[0]; pos[1] = sel[1];
              } else if (nzc == 1) {
                for (int p = 0; p < 4; ++p)
                  if (hy_nonzero(W, ldw, R, K, r, c0 + p)) sel[0] = p;
                pos[0] = sel[0]; pos[1] = sel[0];
              } else {
                pos[0] = 1; pos[1] = 0;
              }
              const int64_t blk = rb * g.nKB + kb;
              for (int j = 0; j < 2; ++j) {
                const int c = 2 * gb + j;
                uint8_t* mrow = meta + blk * 128 + rr * 8;
                mrow[(2 * c) / 8] |= (uint8_t)(pos[j] << ((2 * c) % 8));
                const int sigma = 8 * bi + 2 * t + j;
                if (sel[j] >= 0) {
                  const uint16_t v = hy_at(W, ldw, R, K, r, c0 + sel[j]);
                  memcpy(values + blk * 1024 + rr * 64 + 2 * c, &v, 2);
                  slot_col[sigma] = c0 + sel[j];
                } else {
                  empty_sigma[E++] = sigma;
                }
              }
              /* surplus: the group's other nonzeros, ascending column */
              if (nzc >= 3)
                for (int p = 0; p < 4; ++p)
                  if (hy_nonzero(W, ldw, R, K, r, c0 + p) && p != sel[0] && p != sel[1]) {
                    sur_u[S] = 16 * bi + 4 * t + p;
                    sur_v[S] = hy_at(W, ldw, R, K, r, c0 + p);
                    ++S;
                  }
            }
          (void)slot_col;
          /* pass 2: greedy slot filling with PDD codes */
          int prev = -1, used = 0, f = 0;
          uint8_t* cu = codes + ((rb * g.nSeg + s) * 64 + 16 * q + rr) * 8;
          for (int i = 0; i < S; ++i) {
            const int d = sur_u[i] - prev, n0 = (d - 1) / 15;
            if (f < E && used + n0 + 1 <= 16) {
              for (int z = 0; z < n0; ++z) ++used;              /* code 0: dummy point */
              const int code = d - 15 * n0;
              cu[used / 2] |= (uint8_t)(code << (4 * (used % 2)));
              ++used;
              const int sigma = empty_sigma[f++];
              const int64_t kb = kb0 + sigma / 8;
              const int c = 2 * (4 * q + (sigma % 8) / 2) + sigma % 2;
              memcpy(values + (rb * g.nKB + kb) * 1024 + rr * 64 + 2 * c, &sur_v[i], 2);
              prev = sur_u[i];
            } else {
              const int u = sur_u[i];
              const int64_t col_in_seg = 64 * (u / 16) + 16 * q + u % 16;
              resflag[col_in_seg] = 1;
              resval[col_in_seg] = sur_v[i];
            }
          }
        }
        for (int c = 0; c < 512; ++c)
          if (resflag[c]) {
            if (total < cap) res_ent[total] = ((uint32_t)c << 16) | resval[c];
            ++total;
          }
        const int64_t z = (rb * g.nSeg + s) * 16 + rr;
        if (total > INT32_MAX) return -1;
        res_ptr[z + 1] = (int32_t)total;
      }
  (void)nz_rows;
  *n_res = total;
  return total > cap ? 1 : 0;
}

/*
 * orc_hy_read: rebuild dense W (raw bits, R x K, zero-filled) from a byte
 * image, layer by layer.  Returns 0, -1 on bad arguments, -2 when the image
 * is inconsistent (more points than empty slots, a point outside its unit, an
 * element written twice, a residual column outside the matrix, a stored
 * element whose value is zero).
 */
int orc_hy_read(const uint8_t* values, const uint8_t* meta, const uint8_t* codes,
                const int32_t* res_ptr, const uint32_t* res_ent, int64_t R, int64_t K, int dt,
                uint16_t* W) {
  if (R < 1 || K < 4 || K % 4 || (dt != ORC_F16 && dt != ORC_BF16)) return -1;
  hy_geo_t g = hy_geo(R, K);
  memset(W, 0, (size_t)(R * K * 2));
  uint8_t* seen = (uint8_t*)calloc((size_t)(R * K), 1);
  if (!seen) return -1;
  int rc = 0;
#define HY_PUT(rw, cl, val)                                                   \
  do {                                                                        \
    int64_t r_ = (rw), c_ = (cl);                                             \
    uint16_t v_ = (val);                                                      \
    if (r_ >= R || c_ >= K || c_ < 0) { if (v_ & 0x7FFF) rc = -2; break; }    \
    if (!(v_ & 0x7FFF) || seen[r_ * K + c_]) { rc = -2; break; }              \
    seen[r_ * K + c_] = 1;                                                    \
    W[r_ * K + c_] = v_;                                                      \
  } while (0)
  for (int64_t rb = 0; rb < g.nRB; ++rb)
    for (int64_t s = 0; s < g.nSeg; ++s)
      for (int64_t rr = 0; rr < 16; ++rr) {
        const int64_t r = rb * 16 + rr;
        const int64_t kb0 = 8 * s, kb1 = (8 * s + 8 < g.nKB) ? 8 * s + 8 : g.nKB;
        const int nb = (int)(kb1 - kb0);
        for (int q = 0; q < 4; ++q) {
          uint16_t empty_val[64];
          int E = 0;
          for (int bi = 0; bi < nb; ++bi)
            for (int t = 0; t < 4; ++t) {
              const int64_t kb = kb0 + bi, blk = rb * g.nKB + kb;
              const int gb = 4 * q + t;
              int pos[2];
              uint16_t val[2];
              for (int j = 0; j < 2; ++j) {
                const int c = 2 * gb + j;
                pos[j] = (meta[blk * 128 + rr * 8 + (2 * c) / 8] >> ((2 * c) % 8)) & 3;
                memcpy(&val[j], values + blk * 1024 + rr * 64 + 2 * c, 2);
              }
              const int e0 = pos[0] > pos[1], e1 = pos[0] >= pos[1];
              if (!e0) HY_PUT(r, 64 * kb + 4 * gb + pos[0], val[0]);
              else empty_val[E++] = val[0];
              if (!e1) HY_PUT(r, 64 * kb + 4 * gb + pos[1], val[1]);
              else empty_val[E++] = val[1];
            }
          const uint8_t* cu = codes + ((rb * g.nSeg + s) * 64 + 16 * q + rr) * 8;
          int p = -1, k = 0;
          for (int i = 0; i < 16; ++i) {
            const int code = (cu[i / 2] >> (4 * (i % 2))) & 15;
            if (code == 0) { p += 15; continue; }
            p += code;
            if (k >= E || p >= 16 * nb) { rc = -2; break; }
            HY_PUT(r, 64 * (kb0 + p / 16) + 16 * q + p % 16, empty_val[k]);
            ++k;
          }
          for (; k < E; ++k)
            if (empty_val[k] & 0x7FFF) rc = -2;     /* unfilled empty slot must hold +-0 */
        }
        const int64_t z = (rb * g.nSeg + s) * 16 + rr;
        for (int32_t e = res_ptr[z]; e < res_ptr[z + 1]; ++e) {
          const int64_t col = 512 * s + (res_ent[e] >> 16);
          if (col >= 64 * kb1) { rc = -2; break; }
          HY_PUT(r, col, (uint16_t)(res_ent[e] & 0xFFFF));
        }
      }
#undef HY_PUT
  free(seen);
  return rc;
}
