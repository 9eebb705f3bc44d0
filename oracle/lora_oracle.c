/*
 * fp64 CPU oracle for the heterogeneous-adapter LoRA apply.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may call, link or load this file; only the tests, the
 * smoke check and the benchmark's CPU-baseline leg use it.  It shares no code,
 * header, table or constant with the HIP library.
 *
 * What it computes (the plain definition, no blocking, fusion or reordering):
 *   for every token i with adapter id a = ids[i]:
 *     a < 0   : y_i = y0_i                       (the "negative id = no adapter"
 *               rule of the reference loop in the S-LoRA paper explainer,
 *               0h-n0.github.io, section "BGMVカーネル")
 *     a >= 0  : v_k   = sum_j A_a[k][j] * x_i[j]          k < r_a   (shrink)
 *               y_i[m] = y0_i[m] + s_a * sum_k B_a[m][k] * v_k       (expand)
 *   i.e. y_i += s_a * B_a (A_a x_i): the BGMV equation of that same section,
 *   with the per-adapter alpha/r scale of the LoRA formula in the SGMV section
 *   of the multi-LoRA serving article (produtoramaxvision.com.br), whose naming
 *   is followed here (A = shrink r x d_in, B = expand d_out x r).
 *
 * Inputs arrive as raw storage bits (fp32, IEEE fp16, bf16, or OCP FP8 E4M3
 * codes for quantised adapters) and are decoded exactly to double here, with
 * this file's own decoders.  Quantised adapters carry fp32 scales: one per rank
 * row of A and one per rank column of B, so that the dequantised matrices are
 *     A[k][j] = sa[k] * code(A)[k][j]      B[m][k] = code(B)[m][k] * sb[k]
 * (each product exact in double).  Sums run in ascending index order in
 * double.  The adapter scale s_a is the stored fp32 value.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ODT_F32 = 0, ODT_F16 = 1, ODT_BF16 = 2, ODT_E4M3 = 3 };

static int elt_size(int32_t dt) { return dt == ODT_F32 ? 4 : (dt == ODT_E4M3 ? 1 : 2); }

/* ---- exact decoders ---------------------------------------------------- */
static double dec_f16(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);                  /* subnormal / zero */
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}
static double dec_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}
static double dec_f32(const void* p) {
  float f;
  memcpy(&f, p, 4);
  return (double)f;
}
/* OCP 8-bit floating point E4M3: sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent field 0 holds subnormals m/8 * 2^-6; no infinities; the codes
 * with every exponent and mantissa bit set are NaN; the largest finite value is
 * 1.75 * 2^8 = 448. */
static double dec_e4m3(uint8_t b) {
  const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);
  else v = ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}
static double dec_at(const void* base, int32_t dt, int64_t idx) {
  if (dt == ODT_F32) return dec_f32((const char*)base + 4 * idx);
  if (dt == ODT_E4M3) return dec_e4m3(((const uint8_t*)base)[idx]);
  uint16_t h;
  memcpy(&h, (const char*)base + 2 * idx, 2);
  return dt == ODT_F16 ? dec_f16(h) : dec_bf16(h);
}

/* ---- round to nearest, ties to even, straight from double --------------- */
/* p = significand bits incl. the implicit one, emin = smallest normal exponent,
 * emax = largest exponent.  Values below the normal range keep the fixed
 * subnormal quantum; values past the overflow threshold become infinities. */
static double rne_format(double v, int p, int emin, int emax) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  frexp(v, &e);             /* v = f * 2^e with 0.5 <= |f| < 1 */
  int ex = e - 1;           /* exponent of the 1.xxx form */
  if (ex < emin) ex = emin;
  double quantum = ldexp(1.0, ex - (p - 1));
  double q = nearbyint(v / quantum) * quantum;   /* default mode: ties to even */
  if (fabs(q) >= ldexp(1.0, emax + 1)) q = copysign(INFINITY, v);
  return q;
}

static uint16_t enc_f16(double q) { /* q already representable in fp16 */
  uint16_t s = signbit(q) ? 0x8000 : 0;
  double a = fabs(q);
  if (isnan(q)) return 0x7E00;
  if (isinf(a)) return s | 0x7C00;
  if (a == 0.0) return s;
  int e;
  double f = frexp(a, &e);  /* a = f 2^e */
  int ex = e - 1;
  if (ex < -14) return s | (uint16_t)llrint(ldexp(a, 24)); /* subnormal */
  uint16_t mant = (uint16_t)(llrint(ldexp(f, 11)) - 1024);
  return s | (uint16_t)((ex + 15) << 10) | mant;
}
static uint16_t enc_bf16(double q) { /* q representable in bf16 => exact in fp32 */
  float f = (float)q;
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(q)) return 0x7FC0;
  return (uint16_t)(u >> 16);
}

/* Round n doubles to the storage type (RNE) and write the stored bits. */
int oracle_round(const double* in, int64_t n, int32_t dt, void* out) {
  for (int64_t i = 0; i < n; ++i) {
    if (dt == ODT_F32) {
      float f = (float)rne_format(in[i], 24, -126, 127);
      memcpy((char*)out + 4 * i, &f, 4);
    } else if (dt == ODT_F16) {
      uint16_t h = enc_f16(rne_format(in[i], 11, -14, 15));
      memcpy((char*)out + 2 * i, &h, 2);
    } else if (dt == ODT_BF16) {
      uint16_t h = enc_bf16(rne_format(in[i], 8, -126, 127));
      memcpy((char*)out + 2 * i, &h, 2);
    } else {
      return -2;
    }
  }
  return 0;
}

/* Decode n stored values to double. */
int oracle_decode(const void* in, int64_t n, int32_t dt, double* out) {
  if (dt < 0 || dt > 3) return -2;
  for (int64_t i = 0; i < n; ++i) out[i] = dec_at(in, dt, i);
  return 0;
}

/*
 * The LoRA apply, one token at a time.
 *   x_bits  [n][d_in]  in x_dtype        y0_bits [n][d_out] in y_dtype
 *   ids     [n]        adapter id per token (negative: no adapter)
 *   A[a]    [r_a][d_in]   B[a] [d_out][r_a]   (stored bits, w_dtype), NULL if
 *                          that adapter is not supplied
 *   a_scale[a] [r_a], b_scale[a] [r_a]: scales of a quantised adapter (NULL
 *                          table or NULL entry: none, i.e. 1)
 *   ranks/scales [n_adapters]
 *   y_out   [n][d_out] double      v_out (optional) [n][v_ld] double, zero past r
 * Returns 0, -1 if a token names an adapter with no supplied weights, -2 on
 * bad arguments.
 */
int oracle_lora_apply(int64_t n, int32_t d_in, int32_t d_out, int32_t w_dtype, int32_t x_dtype,
                      int32_t y_dtype, const void* x_bits, const int32_t* ids,
                      int32_t n_adapters, const int32_t* ranks, const float* scales,
                      const void* const* A, const void* const* B,
                      const float* const* a_scale, const float* const* b_scale,
                      const void* y0_bits, double* y_out, double* v_out, int32_t v_ld,
                      int32_t n_threads) {
  if (n < 0 || d_in <= 0 || d_out <= 0 || w_dtype < 0 || w_dtype > 3 || x_dtype < 0 ||
      x_dtype > 2 || y_dtype < 0 || y_dtype > 2)
    return -2;
  for (int64_t i = 0; i < n; ++i) {
    int32_t a = ids[i];
    if (a < 0) continue;
    if (a >= n_adapters || !A[a] || !B[a] || ranks[a] <= 0) return -1;
    if (v_out && ranks[a] > v_ld) return -2;
  }
  int bad = 0;
#ifdef _OPENMP
  if (n_threads <= 0) n_threads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(| : bad)
#endif
  for (int64_t i = 0; i < n; ++i) {
    const int32_t a = ids[i];
    double* yi = y_out + i * (int64_t)d_out;
    for (int32_t m = 0; m < d_out; ++m) yi[m] = dec_at(y0_bits, y_dtype, i * (int64_t)d_out + m);
    if (v_out)
      for (int32_t k = 0; k < v_ld; ++k) v_out[i * (int64_t)v_ld + k] = 0.0;
    if (a < 0) continue;
    const int32_t r = ranks[a];
    const double s = (double)scales[a];
    const float* sa = a_scale ? a_scale[a] : NULL;
    const float* sb = b_scale ? b_scale[a] : NULL;
    double* v = (double*)malloc(sizeof(double) * (size_t)r);
    if (!v) { bad |= 1; continue; }
    /* shrink: v_k = sum_j A[k][j] x[j] */
    for (int32_t k = 0; k < r; ++k) {
      const double ak = sa ? (double)sa[k] : 1.0;
      double acc = 0.0;
      for (int32_t j = 0; j < d_in; ++j)
        acc += (ak * dec_at(A[a], w_dtype, (int64_t)k * d_in + j)) *
               dec_at(x_bits, x_dtype, i * (int64_t)d_in + j);
      v[k] = acc;
      if (v_out) v_out[i * (int64_t)v_ld + k] = acc;
    }
    /* expand: y[m] = y0[m] + s * sum_k B[m][k] v_k */
    for (int32_t m = 0; m < d_out; ++m) {
      double acc = 0.0;
      for (int32_t k = 0; k < r; ++k)
        acc += (dec_at(B[a], w_dtype, (int64_t)m * r + k) * (sb ? (double)sb[k] : 1.0)) * v[k];
      yi[m] = yi[m] + s * acc;
    }
    free(v);
  }
  return bad ? -3 : 0;
}

/*
 * Page walker: rebuild one adapter slice's dense A and B from a host image of
 * the unified page pool, following the pool layout the library documents:
 *   r_s  = rank rounded up to a multiple of 16 bytes' worth of elements
 *   A    : row k spans ceil(d_in/P) pages; element j of row k lives in page
 *          a_pages[k*ceil(d_in/P) + j/P] at position j % P
 *   B    : floor(P/r_s) rows per page; row m lives in page b_pages[m / rpp] at
 *          position (m % rpp) * r_s, columns [r, r_s) hold zeros
 * Copies bits only.  Returns 0, -1 if a page id is out of range, -4 if a
 * padding column is not zero, -2 on bad arguments.
 */
int oracle_walk_adapter(const void* pool, int32_t dt, int32_t P, int64_t n_pages,
                        int32_t d_in, int32_t d_out, int32_t rank, const int32_t* a_pages,
                        const int32_t* b_pages, void* A_out, void* B_out) {
  if (dt < 0 || dt > 3 || P <= 0 || rank <= 0) return -2;
  const int es = elt_size(dt);
  const int per16 = 16 / es;
  const int32_t rs = (rank + per16 - 1) / per16 * per16;
  if (rs > P) return -2;
  const int32_t npa = (d_in + P - 1) / P;
  const int32_t rpp = P / rs;
  const char* base = (const char*)pool;
  for (int32_t k = 0; k < rank; ++k)
    for (int32_t j = 0; j < d_in; ++j) {
      int64_t pg = a_pages[(int64_t)k * npa + j / P];
      if (pg < 0 || pg >= n_pages) return -1;
      memcpy((char*)A_out + ((int64_t)k * d_in + j) * es, base + (pg * P + j % P) * es, es);
    }
  for (int32_t m = 0; m < d_out; ++m) {
    int64_t pg = b_pages[m / rpp];
    if (pg < 0 || pg >= n_pages) return -1;
    int64_t row0 = pg * P + (int64_t)(m % rpp) * rs;
    for (int32_t k = 0; k < rs; ++k) {
      const char* src = base + (row0 + k) * es;
      if (k < rank) {
        memcpy((char*)B_out + ((int64_t)m * rank + k) * es, src, es);
      } else {
        for (int b = 0; b < es; ++b)
          if (src[b] != 0) return -4;
      }
    }
  }
  return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
