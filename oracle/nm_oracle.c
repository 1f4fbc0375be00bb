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
