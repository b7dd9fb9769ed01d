/* A plain C99 client of include/svq.h: checks that the header compiles as C,
 * that the library links and resolves its declarations from C, and that the
 * INT4 and sign-plane blob layouts the header documents are the bytes the
 * host packers write.  Host calls and argument checks only: nothing here
 * touches a GPU.  Prints "abi_from_c OK" on success, exits 1 on the first
 * failure. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "svq.h"

static int fails = 0;
#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      fprintf(stderr, "FAIL: " __VA_ARGS__); \
      fprintf(stderr, "\n");             \
      fails++;                           \
      return;                            \
    }                                    \
  } while (0)

/* INT4 blob, N = 20 (two row tiles, the second ragged), K = 256. */
static void int4_layout(void) {
  const int64_t N = 20, K = 256, N16 = 32, KT = 2, KT4 = 4;
  const size_t bytes = svq_int4_packed_bytes(N, K, 128);
  CHECK(bytes == (size_t)(N16 * K / 2 + N16 * KT4 * 2), "int4 packed bytes %zu", bytes);
  int8_t* c = malloc((size_t)(N * K));
  uint16_t* s = malloc((size_t)(N * KT) * 2);
  uint8_t* p = malloc(bytes);
  int8_t* c2 = malloc((size_t)(N * K));
  uint16_t* s2 = malloc((size_t)(N * KT) * 2);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) c[n * K + k] = (int8_t)((n * 7 + k * 3) % 16 - 8);
  for (int64_t i = 0; i < N * KT; ++i) s[i] = (uint16_t)(0x3F80 + i);
  memset(p, 0xAB, bytes);
  CHECK(pack_int4_grouped(c, s, N, K, 128, p) == SVQ_OK, "pack_int4_grouped: %s", svq_last_error());
  /* Every code at the position the header states. */
  for (int64_t n = 0; n < N16; ++n)
    for (int64_t k = 0; k < K; ++k) {
      const int64_t rt = n / 16, r = n % 16, kt = k / 128, t = (k % 128) / 32, q = (k % 32) / 8, j = k % 8;
      const int64_t lane = 16 * q + r;
      const uint8_t* dw = p + (rt * KT + kt) * 1024 + 16 * lane + 4 * t;
      const uint32_t w = (uint32_t)dw[0] | (uint32_t)dw[1] << 8 | (uint32_t)dw[2] << 16 | (uint32_t)dw[3] << 24;
      const int bit = (j % 2 == 0) ? 4 * (int)(j / 2) : 16 + 4 * (int)(j / 2);
      const int u = (int)((w >> bit) & 15u);
      const int want = n < N ? c[n * K + k] + 8 : 8; /* padding rows hold c = 0 */
      CHECK(u == want, "int4 code (n=%lld, k=%lld): nibble %d, want %d", (long long)n, (long long)k, u, want);
    }
  /* Scales at N16*K/2 + 2*(n*KT4 + g), zero past KT and in padding rows. */
  for (int64_t n = 0; n < N16; ++n)
    for (int64_t g = 0; g < KT4; ++g) {
      const uint8_t* e = p + N16 * K / 2 + 2 * (n * KT4 + g);
      const uint16_t v = (uint16_t)(e[0] | e[1] << 8);
      const uint16_t want = (n < N && g < KT) ? s[n * KT + g] : 0;
      CHECK(v == want, "int4 scale (n=%lld, g=%lld): %04x, want %04x", (long long)n, (long long)g, v, want);
    }
  CHECK(unpack_int4_grouped(p, N, K, 128, c2, s2) == SVQ_OK, "unpack_int4_grouped: %s", svq_last_error());
  CHECK(memcmp(c, c2, (size_t)(N * K)) == 0 && memcmp(s, s2, (size_t)(N * KT) * 2) == 0, "int4 round trip");
  /* A code outside [-8, 7] is refused and named. */
  c[5 * K + 17] = 8;
  CHECK(pack_int4_grouped(c, s, N, K, 128, p) == SVQ_ERR_RANGE, "out-of-range code accepted");
  CHECK(strlen(svq_last_error()) > 0, "no message for SVQ_ERR_RANGE");
  free(c), free(s), free(p), free(c2), free(s2);
}

/* Binary-plane blob, N = 16, K = 128, P = 2. */
static void plane_layout(void) {
  const int64_t N = 16, K = 128, P = 2, N16 = 16, KT4 = 4;
  const size_t bytes = svq_binplane_packed_bytes(N, K, 128, (int32_t)P);
  CHECK(bytes == (size_t)(N16 * K / 8 * P + P * N16 * KT4 * 2), "plane packed bytes %zu", bytes);
  int8_t* b = malloc((size_t)(P * N * K));
  uint16_t* a = malloc((size_t)(P * N) * 2);
  uint8_t* p = malloc(bytes);
  for (int64_t i = 0; i < P * N * K; ++i) b[i] = ((i * 2654435761u) >> 7) & 1 ? -1 : 1;
  for (int64_t i = 0; i < P * N; ++i) a[i] = (uint16_t)(0x3C00 + i);
  CHECK(pack_binary_planes(b, a, N, K, 128, (int32_t)P, p) == SVQ_OK, "pack_binary_planes: %s", svq_last_error());
  for (int64_t pl = 0; pl < P; ++pl)
    for (int64_t n = 0; n < N; ++n)
      for (int64_t k = 0; k < K; ++k) {
        const int64_t r = n % 16, t = k / 32, q = (k % 32) / 8, j = k % 8, lane = 16 * q + r;
        const uint8_t* dw = p + 256 * pl + 4 * lane;
        const uint32_t w = (uint32_t)dw[0] | (uint32_t)dw[1] << 8 | (uint32_t)dw[2] << 16 | (uint32_t)dw[3] << 24;
        const int bit = (j % 2 == 0) ? 4 * (int)t + (int)(j / 2) : 16 + 4 * (int)t + (int)(j / 2);
        const int set = (int)((w >> bit) & 1u);
        CHECK(set == (b[(pl * N + n) * K + k] < 0), "sign (p=%lld, n=%lld, k=%lld)", (long long)pl, (long long)n,
              (long long)k);
      }
  for (int64_t pl = 0; pl < P; ++pl)
    for (int64_t n = 0; n < N16; ++n) {
      const uint8_t* e = p + N16 * K / 8 * P + 2 * ((pl * N16 + n) * KT4 + 0);
      CHECK((uint16_t)(e[0] | e[1] << 8) == a[pl * N + n], "alpha (p=%lld, n=%lld)", (long long)pl, (long long)n);
    }
  free(b), free(a), free(p);
}

/* Device entry points refuse bad arguments before any HIP call. */
static void argument_checks(void) {
  uint16_t y[16] = {0};
  CHECK(gemv_w4a16(NULL, y, y, 16, 128, 128, NULL) == SVQ_ERR_NULL, "gemv_w4a16 took a NULL blob");
  CHECK(strlen(svq_last_error()) > 0, "no message for SVQ_ERR_NULL");
  CHECK(gemm_smallm_binplane((const uint8_t*)y, y, y, 1, 16, 100, 128, 3, NULL) == SVQ_ERR_SHAPE,
        "gemm_smallm_binplane took K = 100");
  CHECK(svq_int4_packed_bytes(16, 100, 128) == 0, "packed bytes for K = 100");
  CHECK(svq_lmhead_workspace_bytes(16) > 0, "head workspace bytes");
}

int main(void) {
  int4_layout();
  plane_layout();
  argument_checks();
  if (fails) return 1;
  printf("abi_from_c OK\n");
  return 0;
}
