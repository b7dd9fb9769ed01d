/*
 * The fp64 oracle (oracle/oracle.c) on seeded small inputs with ragged
 * shapes, built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py.  Every entry point runs; a few closed forms are
 * checked (a one-hot activation row selects s * c, a unit plane gives the
 * signed sum, the planted-free argmax lies in range).  Exit status 0 means
 * every check passed and no sanitizer fired.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_linear_w4a16(const int8_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, int64_t,
                        double*, double*);
int oracle_linear_binplane(const int8_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, int64_t,
                           int64_t, double*, double*);
int oracle_linear_sa(const int8_t*, const uint8_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t,
                     int64_t, int64_t, double*, double*);
int oracle_argmax_w4a16(const int8_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, int64_t,
                        const int32_t*, int32_t*, int32_t*, double*, double*, double*);
int oracle_argmax_binplane(const int8_t*, const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, int64_t,
                           int64_t, const int32_t*, int32_t*, int32_t*, double*, double*, double*);
int oracle_verify_greedy(const int32_t*, const int32_t*, int64_t);
int64_t oracle_int4_blob_bytes(int64_t, int64_t);
int oracle_pack_int4(const int8_t*, const uint16_t*, int64_t, int64_t, uint8_t*);
int64_t oracle_binplane_blob_bytes(int64_t, int64_t, int64_t);
int oracle_pack_binplane(const int8_t*, const uint16_t*, int64_t, int64_t, int64_t, uint8_t*);
int64_t oracle_sa_blob_bytes(int64_t, int64_t, int64_t, int64_t);
int oracle_pack_sa(const int8_t*, const uint8_t*, const uint16_t*, int64_t, int64_t, int64_t, int64_t, uint8_t*);
int oracle_requant_int4(const uint16_t*, const uint16_t*, int64_t, int64_t, int64_t, int8_t*);
int oracle_fit_planes(const uint16_t*, int64_t, int64_t, int64_t, int64_t, int64_t, int8_t*, double*, uint16_t*);
int oracle_snap_sa(const uint16_t*, int64_t, int64_t, int64_t, int64_t, uint8_t*, uint16_t*);
double oracle_bf16_value(uint16_t);

static uint64_t state = 0x243F6A8885A308D3ull;
static uint32_t next_u32(void) { /* xorshift64* */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (uint32_t)((state * 0x2545F4914F6CDD1Dull) >> 32);
}

static int fails = 0;
#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) {                                                          \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);   \
      ++fails;                                                           \
    }                                                                    \
  } while (0)

static void *xmalloc(size_t n) {
  void *p = calloc(n ? n : 1, 1);
  if (!p) abort();
  return p;
}

static void run_case(int64_t M, int64_t N, int64_t K, int64_t P, int64_t G) {
  int8_t *codes = xmalloc(N * K), *signs = xmalloc(P * N * K);
  uint16_t *scales = xmalloc(2 * N * (K / 128)), *alpha = xmalloc(2 * P * N * (K / 128));
  uint16_t *x = xmalloc(2 * M * K), *w = xmalloc(2 * N * K), *d = xmalloc(2 * N * (K / 256 + 1));
  uint8_t *sacodes = xmalloc(P * N * (K / G));
  double *y = xmalloc(8 * M * N), *a = xmalloc(8 * M * N);
  for (int64_t i = 0; i < N * K; ++i) codes[i] = (int8_t)((int)(next_u32() % 16) - 8);
  for (int64_t i = 0; i < P * N * K; ++i) signs[i] = (next_u32() & 1) ? 1 : -1;
  for (int64_t i = 0; i < N * (K / 128); ++i) scales[i] = (uint16_t)(0x3BA0 + next_u32() % 64);
  for (int64_t i = 0; i < P * N * (K / 128); ++i) alpha[i] = (uint16_t)(0x2000 + next_u32() % 0x800);
  for (int64_t i = 0; i < N * K; ++i) w[i] = (uint16_t)(0x3C00 + next_u32() % 0x300) | ((next_u32() & 1) << 15);
  for (int64_t i = 0; i < P * N * (K / G); ++i) sacodes[i] = (uint8_t)next_u32();
  for (int64_t i = 0; i < N * (K / 256); ++i) d[i] = (uint16_t)(0x0400 + next_u32() % 0x2000);
  /* x: one-hot rows (row m selects k = 7m mod K) */
  memset(x, 0, 2 * M * K);
  for (int64_t m = 0; m < M; ++m) x[m * K + (7 * m) % K] = 0x3F80;
  CHECK(oracle_linear_w4a16(codes, scales, x, M, N, K, 128, y, a) == 0);
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      const int64_t k = (7 * m) % K;
      CHECK(y[m * N + n] == codes[n * K + k] * oracle_bf16_value(scales[n * (K / 128) + k / 128]));
    }
  CHECK(oracle_linear_binplane(signs, alpha, x, M, N, K, 128, P, y, a) == 0);
  if (K % 256 == 0) CHECK(oracle_linear_sa(signs, sacodes, d, x, M, N, K, G, P, y, a) == 0);
  int32_t *out = xmalloc(4 * M), *idx = xmalloc(4 * M);
  double *zmax = xmalloc(8 * M), *amax = xmalloc(8 * M), *zs = xmalloc(8 * M);
  CHECK(oracle_argmax_w4a16(codes, scales, x, M, N, K, 128, NULL, out, idx, zmax, amax, zs) == 0);
  for (int64_t m = 0; m < M; ++m) CHECK(idx[m] >= 0 && idx[m] < N);
  CHECK(oracle_argmax_binplane(signs, alpha, x, M, N, K, 128, P, NULL, out, idx, zmax, amax, zs) == 0);
  uint8_t *blob = xmalloc(oracle_int4_blob_bytes(N, K));
  CHECK(oracle_pack_int4(codes, scales, N, K, blob) == 0);
  free(blob);
  blob = xmalloc(oracle_binplane_blob_bytes(N, K, P));
  CHECK(oracle_pack_binplane(signs, alpha, N, K, P, blob) == 0);
  free(blob);
  if (K % 256 == 0) {
    blob = xmalloc(oracle_sa_blob_bytes(N, K, G, P));
    CHECK(oracle_pack_sa(signs, sacodes, d, N, K, G, P, blob) == 0);
    free(blob);
  }
  CHECK(oracle_requant_int4(w, scales, N, K, 128, codes) == 0);
  for (int64_t i = 0; i < N * K; ++i) CHECK(codes[i] >= -8 && codes[i] <= 7);
  double *a64 = xmalloc(8 * P * N * (K / G));
  uint16_t *a16 = xmalloc(2 * P * N * (K / G));
  CHECK(oracle_fit_planes(w, N, K, G, P, 5, signs, a64, a16) == 0);
  if (K % 256 == 0) CHECK(oracle_snap_sa(a16, N, K, G, P, sacodes, d) == 0);
  int32_t t[5] = {3, 4, 5, 6, 7}, dr[4] = {3, 4, 9, 6};
  CHECK(oracle_verify_greedy(t, dr, 5) == 3);
  free(codes); free(signs); free(scales); free(alpha); free(x); free(w); free(d); free(sacodes);
  free(y); free(a); free(out); free(idx); free(zmax); free(amax); free(zs); free(a64); free(a16);
}

int main(void) {
  static const int64_t shapes[][5] = {{1, 1, 128, 1, 128}, {3, 17, 256, 2, 64},  {2, 33, 512, 3, 128},
                                      {5, 16, 768, 6, 256}, {1, 40, 1024, 4, 64}, {4, 7, 384, 5, 128}};
  for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i)
    run_case(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], shapes[i][4]);
  if (fails) fprintf(stderr, "%d checks failed\n", fails);
  else printf("oracle checks passed\n");
  return fails ? 1 : 0;
}
