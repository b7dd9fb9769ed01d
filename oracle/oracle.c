/*
 * oracle.c -- plain fp64 CPU statement of the low-bit linear layers.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load this
 * library: only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
 * bench.py call it.  It includes no header and shares no helper, table or
 * constant with the HIP library under speculative_verify_amd/csrc; it is
 * written from the definitions below, not from that code.
 *
 * Sources (the pages these definitions come from):
 *  - "Efficient Qwen Competition" tech report, sec. 2.1 (target model QAD):
 *    the served weight is the INT4 code matrix W_q times frozen symmetric
 *    per-group scales s (no zero point), packed as W4A16; sec. 3.3 fixes the
 *    group size at 128 along the input dimension.
 *  - ShiftAddQwen README, intro and "Method / Format": every weight group is a
 *    sum of sign planes, w = sum_p alpha_p * b_p with b_p in {-1,+1} and one
 *    scale per (plane, group) along the input dimension; the mat-vec is a
 *    signed add per plane followed by one multiply per plane and group.
 *  - ShiftAddQwen README, "Method / Format" (the sa* types): inside a
 *    super-block of 256 weights of one row along the input dimension, each
 *    sign plane has one unsigned 8-bit scale code a per group of G in
 *    {64, 128, 256} weights, and the super-block has one fp16 scale d; the
 *    plane's scale for that group is alpha = d * a.
 *  - The same pages for the offline steps: the report's sec. 2.1 rounds the
 *    updated weights back onto the frozen INT4 grid at packing time; the
 *    README's "Output-aware fit" fits the planes by greedy initialisation
 *    and alternating least squares with exhaustive code choice, and its
 *    "Scale distillation" snaps the scales onto the u8 grid.
 *  - DFlash summary, sec. 4.1 and the tech report sec. 2.2: the target
 *    verifies a drafted block in one parallel pass, and greedy (temperature 0)
 *    decoding takes the argmax of the target's logits.
 *  - small-vocabulary MTP study, sec. 3.3: a trimmed 32,768-row head whose
 *    row index can be mapped back to a token id.
 *
 * Everything is evaluated in fp64 with no blocking or reordering beyond the
 * group structure the definitions state.  Output rows are independent, so
 * the loop over output rows n is split across OpenMP threads; each row's sum
 * runs in the order written.
 *
 * Packed layouts (oracle_pack_*): the pages name the formats but not a byte
 * layout; the layout is this project's own, stated here element by element
 * (the same statement is in the repository's design notes):
 *
 *   INT4 blob.  N16 = N rounded up to 16, KT = K/128.
 *     code tile (rt, kt) starts at byte (rt*KT + kt)*1024; inside it,
 *     lane = 16*q + r owns the 16 bytes at 16*lane, dword t (t = 0..3) at
 *     16*lane + 4*t (little endian).  That dword holds the codes of row
 *     n = 16*rt + r at k = 128*kt + 32*t + 8*q + j, j = 0..7: even j = 2i in
 *     bits [4i, 4i+4), odd j = 2i+1 in bits [16+4i, 20+4i).  A nibble holds
 *     u = c + 8.  Rows n >= N hold c = 0.
 *     Then bf16 scales: row n (n < N16) holds s[n][g] at entry n*KT4 + g,
 *     KT4 = KT rounded up to 4; entries g >= KT and padded rows are 0.
 *   Binary-plane blob (P planes).
 *     tile (rt, kt) starts at byte (rt*KT + kt)*256*P; plane p of the tile
 *     occupies bytes [256*p, 256*p + 256), where lane = 16*q + r owns the
 *     dword at 256*p + 4*lane.  That dword holds the signs of plane p, row
 *     n = 16*rt + r, k = 128*kt + 32*t + 8*q + j:
 *     even j = 2i at bit 4t + i, odd j = 2i+1 at bit 16 + 4t + i.  Bit set
 *     means b = -1.  Rows n >= N hold b = +1.
 *     Then fp16 alphas: alpha[p][n][g] at entry (p*N16 + n)*KT4 + g; entries
 *     g >= KT and padded rows are 0.
 *   sa blob (P planes, group G in {64, 128, 256}, K a multiple of 256).
 *     The sign section is the binary-plane blob's, byte for byte.
 *     Then u8 codes: a[p][n][g] at byte (p*N16 + n)*CG + g of the code
 *     section, CG = KT4*128/G (a row spans KT4 128-wide column tiles);
 *     entries g >= K/G and padded rows are 0.
 *     Then fp16 d: d[n][j] (super-block j = k/256) at entry n*KS2 + j of
 *     the last section, KS2 = KT4/2; entries j >= K/256 and padded rows are 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* bfloat16 is the upper 16 bits of an IEEE-754 binary32; widening is exact. */
double oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits; exponent field 0 encodes subnormals f * 2^-24. */
double oracle_f16_value(uint16_t bits) {
  int sign = bits >> 15;
  int e = (bits >> 10) & 0x1f;
  int f = bits & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(1024.0 + (double)f, e - 25);
  return sign ? -v : v;
}

void oracle_bf16_values(const uint16_t* bits, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_value(bits[i]);
}

void oracle_f16_values(const uint16_t* bits, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_value(bits[i]);
}

static double* decode_bf16_array(const uint16_t* bits, int64_t n) {
  double* v = (double*)malloc((size_t)n * sizeof(double));
  if (v) oracle_bf16_values(bits, n, v);
  return v;
}

/*
 * W4A16 linear layer (tech report sec. 2.1, 3.3):
 *   y[m][n] = sum_g s[n][g] * ( sum_{k in group g} c[n][k] * x[m][k] )
 *   a[m][n] = sum_k | s[n][g(k)] * c[n][k] * x[m][k] |   (tolerance scale)
 * codes [N][K] int8, scales [N][K/G] bf16 bits, x [M][K] bf16 bits,
 * y and a [M][N] fp64.  Returns 0, or -1 on bad sizes / no memory.
 */
int oracle_linear_w4a16(const int8_t* codes, const uint16_t* scales,
                        const uint16_t* x, int64_t M, int64_t N, int64_t K,
                        int64_t G, double* y, double* a) {
  if (M < 1 || N < 1 || K < 1 || G < 1 || K % G) return -1;
  const int64_t ng = K / G;
  double* xv = decode_bf16_array(x, M * K);
  if (!xv) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t m = 0; m < M; ++m) {
      double total = 0.0, total_abs = 0.0;
      for (int64_t g = 0; g < ng; ++g) {
        const double s = oracle_bf16_value(scales[n * ng + g]);
        double inner = 0.0, inner_abs = 0.0;
        for (int64_t k = g * G; k < (g + 1) * G; ++k) {
          const double p = (double)codes[n * K + k] * xv[m * K + k];
          inner += p;
          inner_abs += fabs(p);
        }
        total += s * inner;
        total_abs += fabs(s) * inner_abs;
      }
      y[m * N + n] = total;
      a[m * N + n] = total_abs;
    }
  }
  free(xv);
  return 0;
}

/*
 * Binary-plane linear layer (ShiftAddQwen README, intro and "Format"):
 *   y[m][n] = sum_g sum_p alpha[p][n][g] * ( sum_{k in g} b[p][n][k] * x[m][k] )
 *   a[m][n] = sum_k | w[n][k] * x[m][k] |,  w[n][k] = sum_p alpha[p][n][g(k)] b[p][n][k]
 * signs [P][N][K] int8 in {-1,+1}, alpha [P][N][K/G] fp16 bits.
 */
int oracle_linear_binplane(const int8_t* signs, const uint16_t* alpha,
                           const uint16_t* x, int64_t M, int64_t N, int64_t K,
                           int64_t G, int64_t P, double* y, double* a) {
  if (M < 1 || N < 1 || K < 1 || G < 1 || P < 1 || K % G) return -1;
  const int64_t ng = K / G;
  double* xv = decode_bf16_array(x, M * K);
  if (!xv) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t m = 0; m < M; ++m) {
      double total = 0.0, total_abs = 0.0;
      for (int64_t g = 0; g < ng; ++g) {
        for (int64_t p = 0; p < P; ++p) {
          const double al = oracle_f16_value(alpha[(p * N + n) * ng + g]);
          double inner = 0.0;
          for (int64_t k = g * G; k < (g + 1) * G; ++k)
            inner += (double)signs[(p * N + n) * K + k] * xv[m * K + k];
          total += al * inner;
        }
        for (int64_t k = g * G; k < (g + 1) * G; ++k) {
          double w = 0.0;
          for (int64_t p = 0; p < P; ++p)
            w += oracle_f16_value(alpha[(p * N + n) * ng + g]) *
                 (double)signs[(p * N + n) * K + k];
          total_abs += fabs(w * xv[m * K + k]);
        }
      }
      y[m * N + n] = total;
      a[m * N + n] = total_abs;
    }
  }
  free(xv);
  return 0;
}

/*
 * sa* ShiftAdd layer (ShiftAddQwen README, "Method / Format"): the planes'
 * scales are stored as alpha[p][n][g] = d[n][j] * a[p][n][g], j the
 * super-block (256 weights) holding group g:
 *   y[m][n] = sum_g sum_p d[n][g*G/256] * a[p][n][g] * ( sum_{k in g} b[p][n][k] * x[m][k] )
 *   a_tol[m][n] = sum_k | w[n][k] * x[m][k] |,  w[n][k] = sum_p alpha[p][n][g(k)] b[p][n][k]
 * signs [P][N][K] in {-1,+1}, codes [P][N][K/G] u8, d [N][K/256] fp16 bits.
 * d * a is exact in fp64 (11 by 8 significant bits).  Requires K % 256 == 0
 * and G dividing 256.
 */
int oracle_linear_sa(const int8_t* signs, const uint8_t* codes, const uint16_t* d,
                     const uint16_t* x, int64_t M, int64_t N, int64_t K,
                     int64_t G, int64_t P, double* y, double* a) {
  if (M < 1 || N < 1 || K < 256 || K % 256 || G < 1 || 256 % G || P < 1) return -1;
  const int64_t ng = K / G, ns = K / 256;
  double* xv = decode_bf16_array(x, M * K);
  if (!xv) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t m = 0; m < M; ++m) {
      double total = 0.0, total_abs = 0.0;
      for (int64_t g = 0; g < ng; ++g) {
        const double dj = oracle_f16_value(d[n * ns + (g * G) / 256]);
        for (int64_t p = 0; p < P; ++p) {
          const double al = dj * (double)codes[(p * N + n) * ng + g];
          double inner = 0.0;
          for (int64_t k = g * G; k < (g + 1) * G; ++k)
            inner += (double)signs[(p * N + n) * K + k] * xv[m * K + k];
          total += al * inner;
        }
        for (int64_t k = g * G; k < (g + 1) * G; ++k) {
          double w = 0.0;
          for (int64_t p = 0; p < P; ++p)
            w += dj * (double)codes[(p * N + n) * ng + g] * (double)signs[(p * N + n) * K + k];
          total_abs += fabs(w * xv[m * K + k]);
        }
      }
      y[m * N + n] = total;
      a[m * N + n] = total_abs;
    }
  }
  free(xv);
  return 0;
}

/*
 * Greedy verification on a (possibly trimmed) W4A16 head (DFlash summary
 * sec. 4.1; tech report sec. 2.2; MTP study sec. 3.3):
 *   z[m][n]   = W4A16 logits as in oracle_linear_w4a16
 *   idx[m]    = smallest n with z[m][n] == max_n z[m][n]
 *   out[m]    = row_ids ? row_ids[idx[m]] : idx[m]
 *   zmax[m]   = z[m][idx[m]],  amax[m] = a[m][idx[m]]
 *   zsecond[m]= max over n != idx[m] of z[m][n]  (-inf when N == 1)
 * The logits are materialised here on purpose: this is the slow statement.
 */
/* First-occurrence argmax of each row of logits z [M][N] (see above). */
static void argmax_rows(const double* z, const double* a, int64_t M, int64_t N,
                        const int32_t* row_ids, int32_t* out, int32_t* idx,
                        double* zmax, double* amax, double* zsecond) {
  for (int64_t m = 0; m < M; ++m) {
    int64_t best = 0;
    for (int64_t n = 1; n < N; ++n)
      if (z[m * N + n] > z[m * N + best]) best = n;
    double second = -INFINITY;
    for (int64_t n = 0; n < N; ++n)
      if (n != best && z[m * N + n] > second) second = z[m * N + n];
    idx[m] = (int32_t)best;
    out[m] = row_ids ? row_ids[best] : (int32_t)best;
    zmax[m] = z[m * N + best];
    amax[m] = a[m * N + best];
    zsecond[m] = second;
  }
}

int oracle_argmax_w4a16(const int8_t* codes, const uint16_t* scales,
                        const uint16_t* x, int64_t M, int64_t N, int64_t K,
                        int64_t G, const int32_t* row_ids, int32_t* out,
                        int32_t* idx, double* zmax, double* amax,
                        double* zsecond) {
  double* z = (double*)malloc((size_t)(M * N) * sizeof(double));
  double* a = (double*)malloc((size_t)(M * N) * sizeof(double));
  if (!z || !a) {
    free(z);
    free(a);
    return -1;
  }
  int rc = oracle_linear_w4a16(codes, scales, x, M, N, K, G, z, a);
  if (rc == 0) argmax_rows(z, a, M, N, row_ids, out, idx, zmax, amax, zsecond);
  free(z);
  free(a);
  return rc;
}

/*
 * The same greedy decision for a head stored as P sign planes (ShiftAddQwen
 * README, Method/Format): z[m][n] is oracle_linear_binplane's logit.
 */
int oracle_argmax_binplane(const int8_t* signs, const uint16_t* alpha,
                           const uint16_t* x, int64_t M, int64_t N, int64_t K,
                           int64_t G, int64_t P, const int32_t* row_ids,
                           int32_t* out, int32_t* idx, double* zmax,
                           double* amax, double* zsecond) {
  double* z = (double*)malloc((size_t)(M * N) * sizeof(double));
  double* a = (double*)malloc((size_t)(M * N) * sizeof(double));
  if (!z || !a) {
    free(z);
    free(a);
    return -1;
  }
  int rc = oracle_linear_binplane(signs, alpha, x, M, N, K, G, P, z, a);
  if (rc == 0) argmax_rows(z, a, M, N, row_ids, out, idx, zmax, amax, zsecond);
  free(z);
  free(a);
  return rc;
}

/*
 * Greedy acceptance of a verified block (DFlash summary sec. 4.1: the draft
 * proposes gamma tokens, the target verifies them in one parallel pass and
 * tau in [1, gamma + 1] tokens are accepted per cycle; greedy decoding keeps
 * the target's argmax).  The block has M = gamma + 1 rows: the anchor, then
 * the drafted tokens d_1 .. d_{M-1} (draft[0 .. M-2]).  target[j] is the
 * target's greedy token for the position after row j.  Walking the drafts in
 * order, draft d_{j+1} is accepted when every earlier draft was accepted and
 * it equals target[j]; tau counts the accepted drafts plus the one token the
 * target contributes after them.  A target id of -1 (no valid maximum) is
 * never equal to a draft, as drafted ids are token ids >= 0.
 */
int oracle_verify_greedy(const int32_t* target, const int32_t* draft, int64_t M) {
  int64_t accepted = 0;
  for (int64_t j = 0; j + 1 < M; ++j) {
    if (target[j] < 0 || target[j] != draft[j]) break;
    accepted += 1;
  }
  return (int)(accepted + 1);
}

/* ---- packed layouts, stated one element at a time (see header) ---- */

static void or_dword(uint8_t* blob, int64_t byte_off, uint32_t v) {
  for (int b = 0; b < 4; ++b) blob[byte_off + b] |= (uint8_t)(v >> (8 * b));
}

int64_t oracle_int4_blob_bytes(int64_t N, int64_t K) {
  const int64_t N16 = (N + 15) / 16 * 16, KT4 = (K / 128 + 3) / 4 * 4;
  return N16 * (K / 2) + N16 * KT4 * 2;
}

int oracle_pack_int4(const int8_t* codes, const uint16_t* scales, int64_t N,
                     int64_t K, uint8_t* blob) {
  if (N < 1 || K < 128 || K % 128) return -1;
  const int64_t N16 = (N + 15) / 16 * 16, KT = K / 128, ng = K / 128;
  memset(blob, 0, (size_t)oracle_int4_blob_bytes(N, K));
  for (int64_t n = 0; n < N16; ++n) {
    for (int64_t k = 0; k < K; ++k) {
      const int c = n < N ? codes[n * K + k] : 0;
      if (c < -8 || c > 7) return -2;
      const uint32_t u = (uint32_t)(c + 8);
      const int64_t rt = n / 16, r = n % 16, kt = k / 128, kk = k % 128;
      const int64_t t = kk / 32, q = (kk % 32) / 8, j = kk % 8;
      const int64_t lane = 16 * q + r;
      const int64_t off = (rt * KT + kt) * 1024 + 16 * lane + 4 * t;
      const int bit = (j % 2) ? 16 + 4 * (int)(j / 2) : 4 * (int)(j / 2);
      or_dword(blob, off, u << bit);
    }
  }
  const int64_t soff = (N16 / 16) * KT * 1024, KT4 = (KT + 3) / 4 * 4;
  for (int64_t n = 0; n < N16; ++n)
    for (int64_t g = 0; g < ng; ++g) {
      const uint16_t s = n < N ? scales[n * ng + g] : 0;
      blob[soff + 2 * (n * KT4 + g)] = (uint8_t)(s & 0xff);
      blob[soff + 2 * (n * KT4 + g) + 1] = (uint8_t)(s >> 8);
    }
  return 0;
}

int64_t oracle_binplane_blob_bytes(int64_t N, int64_t K, int64_t P) {
  const int64_t N16 = (N + 15) / 16 * 16, KT4 = (K / 128 + 3) / 4 * 4;
  return N16 * (K / 8) * P + P * N16 * KT4 * 2;
}

/* Sign section shared by the binary-plane and sa blobs: returns -2 on a
 * sign outside {-1, +1}.  The blob must be zeroed. */
static int put_sign_planes(const int8_t* signs, int64_t N, int64_t K, int64_t P,
                           uint8_t* blob) {
  const int64_t N16 = (N + 15) / 16 * 16, KT = K / 128;
  for (int64_t p = 0; p < P; ++p)
    for (int64_t n = 0; n < N16; ++n)
      for (int64_t k = 0; k < K; ++k) {
        const int b = n < N ? signs[(p * N + n) * K + k] : 1;
        if (b != 1 && b != -1) return -2;
        if (b == 1) continue;
        const int64_t rt = n / 16, r = n % 16, kt = k / 128, kk = k % 128;
        const int64_t t = kk / 32, q = (kk % 32) / 8, j = kk % 8;
        const int64_t lane = 16 * q + r;
        const int64_t off = (rt * KT + kt) * 256 * P + 256 * p + 4 * lane;
        const int bit = (j % 2) ? 16 + 4 * (int)t + (int)(j / 2)
                                : 4 * (int)t + (int)(j / 2);
        or_dword(blob, off, 1u << bit);
      }
  return 0;
}

int oracle_pack_binplane(const int8_t* signs, const uint16_t* alpha, int64_t N,
                         int64_t K, int64_t P, uint8_t* blob) {
  if (N < 1 || K < 128 || K % 128 || P < 1) return -1;
  const int64_t N16 = (N + 15) / 16 * 16, KT = K / 128, ng = K / 128;
  memset(blob, 0, (size_t)oracle_binplane_blob_bytes(N, K, P));
  if (put_sign_planes(signs, N, K, P, blob)) return -2;
  const int64_t aoff = (N16 / 16) * KT * 256 * P, KT4 = (KT + 3) / 4 * 4;
  for (int64_t p = 0; p < P; ++p)
    for (int64_t n = 0; n < N16; ++n)
      for (int64_t g = 0; g < ng; ++g) {
        const uint16_t a = n < N ? alpha[(p * N + n) * ng + g] : 0;
        const int64_t e = (p * N16 + n) * KT4 + g;
        blob[aoff + 2 * e] = (uint8_t)(a & 0xff);
        blob[aoff + 2 * e + 1] = (uint8_t)(a >> 8);
      }
  return 0;
}

int64_t oracle_sa_blob_bytes(int64_t N, int64_t K, int64_t G, int64_t P) {
  const int64_t N16 = (N + 15) / 16 * 16, KT4 = (K / 128 + 3) / 4 * 4;
  return N16 * (K / 8) * P + P * N16 * (KT4 * 128 / G) + N16 * (KT4 / 2) * 2;
}

int oracle_pack_sa(const int8_t* signs, const uint8_t* codes, const uint16_t* d,
                   int64_t N, int64_t K, int64_t G, int64_t P, uint8_t* blob) {
  if (N < 1 || K < 256 || K % 256 || (G != 64 && G != 128 && G != 256) || P < 1) return -1;
  const int64_t N16 = (N + 15) / 16 * 16, KT4 = (K / 128 + 3) / 4 * 4;
  const int64_t ng = K / G, ns = K / 256, CG = KT4 * 128 / G, KS2 = KT4 / 2;
  memset(blob, 0, (size_t)oracle_sa_blob_bytes(N, K, G, P));
  if (put_sign_planes(signs, N, K, P, blob)) return -2;
  const int64_t coff = N16 * (K / 8) * P, doff = coff + P * N16 * CG;
  for (int64_t p = 0; p < P; ++p)
    for (int64_t n = 0; n < N; ++n)
      for (int64_t g = 0; g < ng; ++g)
        blob[coff + (p * N16 + n) * CG + g] = codes[(p * N + n) * ng + g];
  for (int64_t n = 0; n < N; ++n)
    for (int64_t j = 0; j < ns; ++j) {
      const uint16_t v = d[n * ns + j];
      blob[doff + 2 * (n * KS2 + j)] = (uint8_t)(v & 0xff);
      blob[doff + 2 * (n * KS2 + j) + 1] = (uint8_t)(v >> 8);
    }
  return 0;
}

/* ---- host quantizers ------------------------------------------------------ */

/* fp64 -> IEEE binary16 bits, round to nearest, ties to even (overflow to
 * infinity, gradual underflow to subnormals), from the format's definition. */
uint16_t oracle_f16_bits(double v) {
  uint16_t sign = 0;
  if (signbit(v)) {
    sign = 0x8000;
    v = -v;
  }
  if (isnan(v)) return (uint16_t)(sign | 0x7e00);
  if (v >= 65520.0) return (uint16_t)(sign | 0x7c00); /* >= max + half an ulp */
  /* quantum of the binade holding v (subnormal quantum 2^-24) */
  int e;
  frexp(v, &e);             /* v = m * 2^e, m in [0.5, 1) */
  int q = e - 11;           /* 11 significant bits: quantum 2^(e-11) */
  if (q < -24) q = -24;
  double units = ldexp(v, -q); /* exact: a power-of-two scaling */
  double fl = floor(units), rem = units - fl;
  double n = fl;
  if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;
  double r = ldexp(n, q);   /* rounded value */
  if (r >= 65520.0) return (uint16_t)(sign | 0x7c00);
  if (r == 0.0) return sign;
  int re;
  frexp(r, &re);
  int exp_field = re - 1 + 15; /* r = 1.f * 2^(re-1) */
  if (exp_field <= 0)           /* subnormal: r = f * 2^-24 */
    return (uint16_t)(sign | (uint16_t)ldexp(r, 24));
  uint16_t frac = (uint16_t)(ldexp(r, -(re - 1)) * 1024.0 - 1024.0);
  return (uint16_t)(sign | (uint16_t)(exp_field << 10) | frac);
}

/* Round half to even of an fp64 value to an integer-valued fp64. */
static double rne(double v) {
  double fl = floor(v), rem = v - fl;
  if (rem > 0.5) return fl + 1.0;
  if (rem < 0.5) return fl;
  return fmod(fl, 2.0) == 0.0 ? fl : fl + 1.0;
}

/*
 * Frozen-grid requantisation (tech report sec. 2.1): at packing time the
 * updated bf16 weights are rounded back onto the original grid, i.e. the
 * code of w under its frozen group scale s is the nearest grid point:
 *   c[n][k] = clamp(rne(w[n][k] / s[n][g(k)]), -8, 7);  s == 0 gives c = 0.
 * w [N][K] and s [N][K/G] are bf16 bits; the quotient is taken in fp64,
 * where an exact half-way case stays exact.
 */
int oracle_requant_int4(const uint16_t* w, const uint16_t* s, int64_t N,
                        int64_t K, int64_t G, int8_t* codes) {
  if (N < 1 || K < 1 || G < 1 || K % G) return -1;
  const int64_t ng = K / G;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      const double sv = oracle_bf16_value(s[n * ng + k / G]);
      double c = 0.0;
      if (sv != 0.0) {
        c = rne(oracle_bf16_value(w[n * K + k]) / sv);
        if (c < -8.0) c = -8.0;
        if (c > 7.0) c = 7.0;
      }
      codes[n * K + k] = (int8_t)c;
    }
  return 0;
}

/* sum_p alpha_p b_p for the sign vector of candidate c (bit p of c set means
 * b_p = -1), summed in plane order. */
static double candidate_value(const double* alpha, int64_t P, int64_t c) {
  double v = 0.0;
  for (int64_t p = 0; p < P; ++p) v += ((c >> p) & 1) ? -alpha[p] : alpha[p];
  return v;
}

/* Least-squares plane scales for fixed signs: solve (B B^T) a = B w by
 * Cholesky.  Returns 0, or -1 when B B^T is singular (a plane equal to or the
 * negation of a combination of the others over the group), leaving a alone. */
static int ls_scales(const double* w, const int8_t* b, int64_t P, int64_t G,
                     double* a) {
  double A[36], r[6], L[36];
  for (int64_t p = 0; p < P; ++p) {
    r[p] = 0.0;
    for (int64_t k = 0; k < G; ++k) r[p] += (double)b[p * G + k] * w[k];
    for (int64_t q = 0; q < P; ++q) {
      double acc = 0.0;
      for (int64_t k = 0; k < G; ++k) acc += (double)(b[p * G + k] * b[q * G + k]);
      A[p * P + q] = acc;
    }
  }
  for (int64_t i = 0; i < P; ++i)
    for (int64_t j = 0; j <= i; ++j) {
      double acc = A[i * P + j];
      for (int64_t t = 0; t < j; ++t) acc -= L[i * P + t] * L[j * P + t];
      if (i == j) {
        if (acc <= 1e-9 * (double)G) return -1;
        L[i * P + i] = sqrt(acc);
      } else {
        L[i * P + j] = acc / L[j * P + j];
      }
    }
  double y[6];
  for (int64_t i = 0; i < P; ++i) {
    double acc = r[i];
    for (int64_t t = 0; t < i; ++t) acc -= L[i * P + t] * y[t];
    y[i] = acc / L[i * P + i];
  }
  for (int64_t i = P - 1; i >= 0; --i) {
    double acc = y[i];
    for (int64_t t = i + 1; t < P; ++t) acc -= L[t * P + i] * a[t];
    a[i] = acc / L[i * P + i];
  }
  return 0;
}

/*
 * Binary-coding fit of one group (ShiftAddQwen README, "Output-aware fit":
 * greedy initialisation, then alternating least squares with exhaustive code
 * choice; here on the plain weight error, without the Hessian weighting):
 *   greedy:  r = w; for p = 1..P: b_p = sign(r) (sign(0) = +1),
 *            alpha_p = mean_k |r_k|, r -= alpha_p b_p
 *   a round: every weight takes the sign vector whose sum_p alpha_p b_p is
 *            nearest to it (lowest candidate index on ties), then alpha is
 *            re-solved by least squares for those signs (kept when the
 *            system is singular)
 * After `iters` rounds every plane with alpha_p < 0 is flipped (alpha_p and
 * b_p negated, the same weights).  w has G values; b is [P][G]; a is [P].
 */
static void fit_group(const double* w, int64_t G, int64_t P, int64_t iters,
                      int8_t* b, double* a) {
  double r[256];
  for (int64_t k = 0; k < G; ++k) r[k] = w[k];
  for (int64_t p = 0; p < P; ++p) {
    double m = 0.0;
    for (int64_t k = 0; k < G; ++k) {
      b[p * G + k] = r[k] < 0.0 ? -1 : 1;
      m += fabs(r[k]);
    }
    a[p] = m / (double)G;
    for (int64_t k = 0; k < G; ++k) r[k] -= a[p] * (double)b[p * G + k];
  }
  for (int64_t it = 0; it < iters; ++it) {
    const int64_t nc = (int64_t)1 << P;
    for (int64_t k = 0; k < G; ++k) {
      int64_t best = 0;
      double bd = fabs(w[k] - candidate_value(a, P, 0));
      for (int64_t c = 1; c < nc; ++c) {
        const double dd = fabs(w[k] - candidate_value(a, P, c));
        if (dd < bd) {
          bd = dd;
          best = c;
        }
      }
      for (int64_t p = 0; p < P; ++p) b[p * G + k] = ((best >> p) & 1) ? -1 : 1;
    }
    ls_scales(w, b, P, G, a);
  }
  for (int64_t p = 0; p < P; ++p)
    if (a[p] < 0.0) {
      a[p] = -a[p];
      for (int64_t k = 0; k < G; ++k) b[p * G + k] = (int8_t)-b[p * G + k];
    }
}

/*
 * The fit for every (row, group) of bf16 weights w [N][K]:
 * signs [P][N][K], alpha [P][N][K/G] as fp64 (alpha64, unrounded) and as
 * fp16 bits (round to nearest even).  G <= 256, 1 <= P <= 6.
 */
int oracle_fit_planes(const uint16_t* w, int64_t N, int64_t K, int64_t G,
                      int64_t P, int64_t iters, int8_t* signs, double* alpha64,
                      uint16_t* alpha16) {
  if (N < 1 || K < 1 || G < 1 || G > 256 || K % G || P < 1 || P > 6 || iters < 0) return -1;
  const int64_t ng = K / G;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    double wv[256], a[6];
    int8_t b[6 * 256];
    for (int64_t g = 0; g < ng; ++g) {
      for (int64_t k = 0; k < G; ++k) wv[k] = oracle_bf16_value(w[n * K + g * G + k]);
      fit_group(wv, G, P, iters, b, a);
      for (int64_t p = 0; p < P; ++p) {
        alpha64[(p * N + n) * ng + g] = a[p];
        alpha16[(p * N + n) * ng + g] = oracle_f16_bits(a[p]);
        for (int64_t k = 0; k < G; ++k) signs[(p * N + n) * K + g * G + k] = b[p * G + k];
      }
    }
  }
  return 0;
}

/*
 * Snap fp16 plane scales onto the sa* grid (ShiftAddQwen README, "Format":
 * alpha = d * a with u8 codes a and one fp16 d per 256-weight super-block;
 * "Scale distillation": scales end snapped to the u8 grid).  Per (row,
 * super-block j): m = the largest alpha over its planes and groups,
 * d = fp16(m / 255), and a = min(rne(alpha / d), 255) (a = 0 when
 * d == 0).  Negative alphas are not representable and are rejected (-2).
 * alpha [P][N][K/G] fp16 bits -> codes [P][N][K/G], d [N][K/256].
 */
int oracle_snap_sa(const uint16_t* alpha, int64_t N, int64_t K, int64_t G,
                   int64_t P, uint8_t* codes, uint16_t* d) {
  if (N < 1 || K < 256 || K % 256 || G < 1 || 256 % G || P < 1) return -1;
  const int64_t ng = K / G, ns = K / 256, gps = 256 / G;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t j = 0; j < ns; ++j) {
      double m = 0.0;
      for (int64_t p = 0; p < P; ++p)
        for (int64_t g = j * gps; g < (j + 1) * gps; ++g) {
          const double v = oracle_f16_value(alpha[(p * N + n) * ng + g]);
          if (v < 0.0) return -2;
          if (v > m) m = v;
        }
      const uint16_t db = oracle_f16_bits(m / 255.0);
      const double dv = oracle_f16_value(db);
      d[n * ns + j] = db;
      for (int64_t p = 0; p < P; ++p)
        for (int64_t g = j * gps; g < (j + 1) * gps; ++g) {
          double c = 0.0;
          if (dv > 0.0) {
            c = rne(oracle_f16_value(alpha[(p * N + n) * ng + g]) / dv);
            if (c > 255.0) c = 255.0;
          }
          codes[(p * N + n) * ng + g] = (uint8_t)c;
        }
    }
  return 0;
}
