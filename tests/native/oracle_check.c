/* The oracle's C entry points under AddressSanitizer / UndefinedBehaviorSanitizer
 * (built with gcc by tests/test_sanitizers.py): seeded small cases of every
 * dtype, with and without v, missing adapters, bad arguments, the rounding and
 * decoding helpers and the page walker on a hand-laid pool image. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_round(const double* in, int64_t n, int32_t dt, void* out);
int oracle_decode(const void* in, int64_t n, int32_t dt, double* out);
int oracle_lora_apply(int64_t n, int32_t d_in, int32_t d_out, int32_t w_dtype, int32_t x_dtype,
                      int32_t y_dtype, const void* x_bits, const int32_t* ids, int32_t n_adapters,
                      const int32_t* ranks, const float* scales, const void* const* A,
                      const void* const* B, const float* const* a_scale,
                      const float* const* b_scale, const void* y0_bits, double* y_out,
                      double* v_out, int32_t v_ld, int32_t n_threads);
int oracle_walk_adapter(const void* pool, int32_t dt, int32_t P, int64_t n_pages, int32_t d_in,
                        int32_t d_out, int32_t rank, const int32_t* a_pages,
                        const int32_t* b_pages, void* A_out, void* B_out);

static uint64_t st = 12345;
static uint32_t rnd(void) {
  st = st * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(st >> 33);
}
static int bad = 0;
#define CHECK(c) do { if (!(c)) { ++bad; printf("FAIL line %d: %s\n", __LINE__, #c); } } while (0)

static void* rand_bits(int dt, int64_t n) {
  const int es = dt == 0 ? 4 : 2;
  double* v = malloc(sizeof(double) * (size_t)(n ? n : 1));
  for (int64_t i = 0; i < n; ++i) v[i] = ((double)(rnd() % 2001) - 1000.0) / 512.0;
  void* out = malloc((size_t)(n ? n : 1) * es);
  CHECK(oracle_round(v, n, dt, out) == 0);
  free(v);
  return out;
}

int main(void) {
  for (int trial = 0; trial < 200; ++trial) {
    const int dt = (int)(rnd() % 3), ydt = (rnd() % 2) ? 0 : dt;
    const int n = (int)(rnd() % 9), d_in = 1 + (int)(rnd() % 40), d_out = 1 + (int)(rnd() % 40);
    const int na = 1 + (int)(rnd() % 5);
    int32_t ranks[5];
    float scales[5];
    const void* A[5];
    const void* B[5];
    int vld = 0;
    for (int a = 0; a < na; ++a) {
      ranks[a] = 1 + (int)(rnd() % 6);
      if (ranks[a] > vld) vld = ranks[a];
      scales[a] = 0.25f * (float)(rnd() % 9);
      A[a] = rand_bits(dt, (int64_t)ranks[a] * d_in);
      B[a] = rand_bits(dt, (int64_t)d_out * ranks[a]);
    }
    int32_t ids[9];
    for (int i = 0; i < n; ++i) ids[i] = (int32_t)(rnd() % (unsigned)(na + 1)) - 1;
    void* x = rand_bits(dt, (int64_t)n * d_in);
    void* y0 = rand_bits(ydt, (int64_t)n * d_out);
    double* y = malloc(sizeof(double) * (size_t)(n * d_out + 1));
    double* v = malloc(sizeof(double) * (size_t)(n * vld + 1));
    CHECK(oracle_lora_apply(n, d_in, d_out, dt, dt, ydt, x, ids, na, ranks, scales, A, B, NULL, NULL, y0, y, v, vld,
                            1 + (int)(rnd() % 3)) == 0);
    CHECK(oracle_lora_apply(n, d_in, d_out, dt, dt, ydt, x, ids, na, ranks, scales, A, B, NULL, NULL, y0, y, NULL, 0,
                            1) == 0);
    if (n > 0 && vld > 1)
      CHECK(oracle_lora_apply(n, d_in, d_out, dt, dt, ydt, x, ids, na, ranks, scales, A, B, NULL, NULL,
                              y0, y, v, 0, 1) != 0 || ids[0] < 0);
    void* rb = malloc((size_t)(n * d_out + 1) * 4);
    CHECK(oracle_round(y, (int64_t)n * d_out, ydt, rb) == 0);
    double* back = malloc(sizeof(double) * (size_t)(n * d_out + 1));
    CHECK(oracle_decode(rb, (int64_t)n * d_out, ydt, back) == 0);
    /* a token naming an adapter whose weights are missing */
    if (n > 0) {
      const void* Anull[5] = {0};
      ids[0] = 0;
      CHECK(oracle_lora_apply(n, d_in, d_out, dt, dt, ydt, x, ids, na, ranks, scales, Anull, B, NULL,
                              NULL, y0, y, NULL, 0, 1) == -1);
    }
    CHECK(oracle_lora_apply(n, 0, d_out, dt, dt, ydt, x, ids, na, ranks, scales, A, B, NULL, NULL, y0,
                            y, NULL, 0, 1) == -2);
    for (int a = 0; a < na; ++a) {
      free((void*)A[a]);
      free((void*)B[a]);
    }
    free(x); free(y0); free(y); free(v); free(rb); free(back);
  }
  /* page walker: a bf16 image of 16 pages of P = 8, rank 3 (r_s = 8), d_in 12
   * (two pages per A row), d_out 5 (one B page) */
  {
    const int P = 8, np = 16, d_in = 12, d_out = 5, r = 3;
    uint16_t pool[16 * 8];
    memset(pool, 0, sizeof(pool));
    int32_t ap[6] = {3, 9, 1, 14, 7, 0};
    int32_t bp5[5] = {11, 12, 13, 2, 4}; /* rpp = floor(8 / 8) = 1: one B row per page */
    for (int k = 0; k < r; ++k)
      for (int j = 0; j < d_in; ++j) pool[ap[k * 2 + j / P] * P + j % P] = (uint16_t)(0x3f80 + k * 16 + j);
    for (int m = 0; m < d_out; ++m)
      for (int k = 0; k < r; ++k) pool[bp5[m] * P + k] = (uint16_t)(0x4000 + m * 4 + k);
    uint16_t Ao[3 * 12], Bo[5 * 3];
    CHECK(oracle_walk_adapter(pool, 2, P, np, d_in, d_out, r, ap, bp5, Ao, Bo) == 0);
    for (int k = 0; k < r; ++k)
      for (int j = 0; j < d_in; ++j) CHECK(Ao[k * d_in + j] == (uint16_t)(0x3f80 + k * 16 + j));
    for (int m = 0; m < d_out; ++m)
      for (int k = 0; k < r; ++k) CHECK(Bo[m * r + k] == (uint16_t)(0x4000 + m * 4 + k));
    int32_t badp[6] = {3, 9, 1, 99, 7, 0};
    CHECK(oracle_walk_adapter(pool, 2, P, np, d_in, d_out, r, badp, bp5, Ao, Bo) == -1);
    pool[12 * P + 5] = 1; /* non-zero padding of row m = 1 */
    CHECK(oracle_walk_adapter(pool, 2, P, np, d_in, d_out, r, ap, bp5, Ao, Bo) == -4);
    CHECK(oracle_walk_adapter(pool, 7, P, np, d_in, d_out, r, ap, bp5, Ao, Bo) == -2);
  }
  printf("oracle under sanitizers: %d failures\n", bad);
  return bad ? 1 : 0;
}
