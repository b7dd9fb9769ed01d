// Host-side packers for the INT4, binary-plane and sa blobs (layouts in svq.h).
//
// Packing is offline work: the report (sec. 2.1) rounds the trained weights
// back onto the frozen INT4 grid "at packing time", and the ShiftAddQwen
// pipeline writes its sign planes once into its own container.  These
// routines therefore run on the CPU, synchronously, and validate every code.
#include <cstdint>
#include <cstring>
#include <string>

#include "svq.h"
#include "svq_internal.h"

namespace {

inline void store_u32(uint8_t* p, uint32_t v) { std::memcpy(p, &v, 4); }
inline uint32_t load_u32(const uint8_t* p) {
  uint32_t v;
  std::memcpy(&v, p, 4);
  return v;
}

int check_common(int64_t N, int64_t K, int32_t G) {
  if (N < 1) return svq::fail(SVQ_ERR_SHAPE, "N must be >= 1 (got %lld)", (long long)N);
  if (G != SVQ_GROUP) return svq::fail(SVQ_ERR_SHAPE, "group size G must be 128 (got %d)", G);
  if (K < SVQ_GROUP || K % SVQ_GROUP)
    return svq::fail(SVQ_ERR_SHAPE, "K must be a positive multiple of 128 (got %lld)", (long long)K);
  return SVQ_OK;
}

// Sign section shared by the binary-plane and sa blobs (layout in svq.h).
void put_signs(const int8_t* signs, int64_t N, int64_t K, int32_t P, uint8_t* packed) {
  const int64_t N16 = svq::round16(N), KT = K / 128, NT = N16 / 16;
  svq::parallel_for(NT, [&](int64_t lo, int64_t hi) {
    for (int64_t rt = lo; rt < hi; ++rt)
      for (int64_t kt = 0; kt < KT; ++kt) {
        uint8_t* tile = packed + (rt * KT + kt) * 256 * P;
        for (int lane = 0; lane < 64; ++lane) {
          const int q = lane >> 4, r = lane & 15;
          const int64_t n = rt * 16 + r;
          for (int p = 0; p < P; ++p) {
            uint32_t w = 0;
            if (n < N) {
              const int8_t* b = signs + ((int64_t)p * N + n) * K + kt * 128 + q * 8;
              for (int t = 0; t < 4; ++t)
                for (int i = 0; i < 4; ++i) {
                  w |= (uint32_t)(b[32 * t + 2 * i] < 0) << (4 * t + i);
                  w |= (uint32_t)(b[32 * t + 2 * i + 1] < 0) << (16 + 4 * t + i);
                }
            }
            store_u32(tile + 256 * p + 4 * lane, w);
          }
        }
      }
  });
}

void get_signs(const uint8_t* packed, int64_t N, int64_t K, int32_t P, int8_t* signs) {
  const int64_t N16 = svq::round16(N), KT = K / 128, NT = N16 / 16;
  svq::parallel_for(NT, [&](int64_t lo, int64_t hi) {
    for (int64_t rt = lo; rt < hi; ++rt)
      for (int64_t kt = 0; kt < KT; ++kt) {
        const uint8_t* tile = packed + (rt * KT + kt) * 256 * P;
        for (int lane = 0; lane < 64; ++lane) {
          const int q = lane >> 4, r = lane & 15;
          const int64_t n = rt * 16 + r;
          if (n >= N) continue;
          for (int p = 0; p < P; ++p) {
            const uint32_t w = load_u32(tile + 256 * p + 4 * lane);
            int8_t* b = signs + ((int64_t)p * N + n) * K + kt * 128 + q * 8;
            for (int t = 0; t < 4; ++t)
              for (int i = 0; i < 4; ++i) {
                b[32 * t + 2 * i] = (w >> (4 * t + i)) & 1 ? -1 : 1;
                b[32 * t + 2 * i + 1] = (w >> (16 + 4 * t + i)) & 1 ? -1 : 1;
              }
          }
        }
      }
  });
}

// Sign check shared by the plane packers: SVQ_OK or SVQ_ERR_RANGE naming the
// first sign outside {-1, +1}.
int check_signs(const char* fn, const int8_t* signs, int64_t N, int64_t K, int32_t P) {
  const int64_t total = (int64_t)P * N * K;
  for (int64_t i = 0; i < total; ++i)
    if (signs[i] != 1 && signs[i] != -1)
      return svq::fail(SVQ_ERR_RANGE, "%s: sign %d at (p=%lld, n=%lld, k=%lld) is not +-1", fn, (int)signs[i],
                       (long long)(i / (N * K)), (long long)((i / K) % N), (long long)(i % K));
  return SVQ_OK;
}

int check_sa(int64_t N, int64_t K, int32_t G, int32_t P) {
  if (N < 1) return svq::fail(SVQ_ERR_SHAPE, "N must be >= 1 (got %lld)", (long long)N);
  if (G != 64 && G != 128 && G != 256) return svq::fail(SVQ_ERR_SHAPE, "G must be 64, 128 or 256 (got %d)", G);
  if (K < 256 || K % 256) return svq::fail(SVQ_ERR_SHAPE, "K must be a positive multiple of 256 (got %lld)", (long long)K);
  if (P < 2 || P > SVQ_MAX_P) return svq::fail(SVQ_ERR_SHAPE, "P must be in 2..6 (got %d)", P);
  return SVQ_OK;
}

}  // namespace

extern "C" {

size_t svq_int4_packed_bytes(int64_t N, int64_t K, int32_t G) {
  if (N < 1 || G != SVQ_GROUP || K < SVQ_GROUP || K % SVQ_GROUP) return 0;
  const int64_t N16 = svq::round16(N);
  return (size_t)(N16 * (K / 2) + N16 * svq::round4(K / G) * 2);
}

size_t svq_binplane_packed_bytes(int64_t N, int64_t K, int32_t G, int32_t P) {
  if (N < 1 || G != SVQ_GROUP || K < SVQ_GROUP || K % SVQ_GROUP || P < 1 || P > SVQ_MAX_P) return 0;
  const int64_t N16 = svq::round16(N);
  return (size_t)(N16 * (K / 8) * P + (int64_t)P * N16 * svq::round4(K / G) * 2);
}

size_t svq_sa_packed_bytes(int64_t N, int64_t K, int32_t G, int32_t P) {
  if (N < 1 || (G != 64 && G != 128 && G != 256) || K < 256 || K % 256 || P < 2 || P > SVQ_MAX_P) return 0;
  const int64_t N16 = svq::round16(N), KT4 = svq::round4(K / 128);
  return (size_t)(N16 * (K / 8) * P + (int64_t)P * N16 * (KT4 * 128 / G) + N16 * (KT4 / 2) * 2);
}

int pack_int4_grouped(const int8_t* codes, const uint16_t* scales_bf16, int64_t N, int64_t K,
                      int32_t G, uint8_t* packed) {
  svq::clear_error();
  if (!codes || !scales_bf16 || !packed) return svq::fail(SVQ_ERR_NULL, "pack_int4_grouped: NULL pointer");
  if (int rc = check_common(N, K, G)) return rc;
  for (int64_t i = 0; i < N * K; ++i)
    if (codes[i] < -8 || codes[i] > 7)
      return svq::fail(SVQ_ERR_RANGE, "pack_int4_grouped: code %d at (n=%lld, k=%lld) outside [-8, 7]",
                       (int)codes[i], (long long)(i / K), (long long)(i % K));
  const int64_t N16 = svq::round16(N), KT = K / 128, NT = N16 / 16, ng = K / G;
  svq::parallel_for(NT, [&](int64_t lo, int64_t hi) {
    static const int8_t zero_row[32] = {0};
    for (int64_t rt = lo; rt < hi; ++rt)
      for (int64_t kt = 0; kt < KT; ++kt) {
        uint8_t* tile = packed + (rt * KT + kt) * 1024;
        for (int lane = 0; lane < 64; ++lane) {
          const int q = lane >> 4, r = lane & 15;
          const int64_t n = rt * 16 + r;
          for (int t = 0; t < 4; ++t) {
            const int8_t* c = n < N ? codes + n * K + kt * 128 + t * 32 + q * 8 : zero_row;
            uint32_t w = 0;
            for (int i = 0; i < 4; ++i) {
              w |= (uint32_t)(c[2 * i] + 8) << (4 * i);
              w |= (uint32_t)(c[2 * i + 1] + 8) << (16 + 4 * i);
            }
            store_u32(tile + 16 * lane + 4 * t, w);
          }
        }
      }
  });
  // Scale rows are KT4 = round4(K/G) entries long; the tail entries and the
  // padding rows are zero.
  uint16_t* s = reinterpret_cast<uint16_t*>(packed + N16 * (K / 2));
  const int64_t KT4 = svq::round4(ng);
  std::memset(s, 0, (size_t)(N16 * KT4 * 2));
  for (int64_t n = 0; n < N; ++n) std::memcpy(s + n * KT4, scales_bf16 + n * ng, (size_t)(ng * 2));
  return SVQ_OK;
}

int unpack_int4_grouped(const uint8_t* packed, int64_t N, int64_t K, int32_t G, int8_t* codes,
                        uint16_t* scales_bf16) {
  svq::clear_error();
  if (!codes || !scales_bf16 || !packed) return svq::fail(SVQ_ERR_NULL, "unpack_int4_grouped: NULL pointer");
  if (int rc = check_common(N, K, G)) return rc;
  const int64_t N16 = svq::round16(N), KT = K / 128, NT = N16 / 16, ng = K / G;
  svq::parallel_for(NT, [&](int64_t lo, int64_t hi) {
    for (int64_t rt = lo; rt < hi; ++rt)
      for (int64_t kt = 0; kt < KT; ++kt) {
        const uint8_t* tile = packed + (rt * KT + kt) * 1024;
        for (int lane = 0; lane < 64; ++lane) {
          const int q = lane >> 4, r = lane & 15;
          const int64_t n = rt * 16 + r;
          if (n >= N) continue;
          for (int t = 0; t < 4; ++t) {
            const uint32_t w = load_u32(tile + 16 * lane + 4 * t);
            int8_t* c = codes + n * K + kt * 128 + t * 32 + q * 8;
            for (int i = 0; i < 4; ++i) {
              c[2 * i] = (int8_t)(((w >> (4 * i)) & 15) - 8);
              c[2 * i + 1] = (int8_t)(((w >> (16 + 4 * i)) & 15) - 8);
            }
          }
        }
      }
  });
  const uint16_t* s = reinterpret_cast<const uint16_t*>(packed + N16 * (K / 2));
  const int64_t KT4 = svq::round4(ng);
  for (int64_t n = 0; n < N; ++n) std::memcpy(scales_bf16 + n * ng, s + n * KT4, (size_t)(ng * 2));
  return SVQ_OK;
}

int pack_binary_planes(const int8_t* signs, const uint16_t* alpha_f16, int64_t N, int64_t K, int32_t G,
                       int32_t P, uint8_t* packed) {
  svq::clear_error();
  if (!signs || !alpha_f16 || !packed) return svq::fail(SVQ_ERR_NULL, "pack_binary_planes: NULL pointer");
  if (int rc = check_common(N, K, G)) return rc;
  if (P < 1 || P > SVQ_MAX_P) return svq::fail(SVQ_ERR_SHAPE, "P must be in 1..6 (got %d)", P);
  if (int rc = check_signs("pack_binary_planes", signs, N, K, P)) return rc;
  const int64_t N16 = svq::round16(N), ng = K / G;
  put_signs(signs, N, K, P, packed);
  uint16_t* a = reinterpret_cast<uint16_t*>(packed + N16 * (K / 8) * P);
  const int64_t KT4 = svq::round4(ng);
  std::memset(a, 0, (size_t)(P * N16 * KT4 * 2));
  for (int p = 0; p < P; ++p)
    for (int64_t n = 0; n < N; ++n)
      std::memcpy(a + ((int64_t)p * N16 + n) * KT4, alpha_f16 + ((int64_t)p * N + n) * ng, (size_t)(ng * 2));
  return SVQ_OK;
}

int unpack_binary_planes(const uint8_t* packed, int64_t N, int64_t K, int32_t G, int32_t P, int8_t* signs,
                         uint16_t* alpha_f16) {
  svq::clear_error();
  if (!signs || !alpha_f16 || !packed) return svq::fail(SVQ_ERR_NULL, "unpack_binary_planes: NULL pointer");
  if (int rc = check_common(N, K, G)) return rc;
  if (P < 1 || P > SVQ_MAX_P) return svq::fail(SVQ_ERR_SHAPE, "P must be in 1..6 (got %d)", P);
  const int64_t N16 = svq::round16(N), ng = K / G;
  get_signs(packed, N, K, P, signs);
  const uint16_t* a = reinterpret_cast<const uint16_t*>(packed + N16 * (K / 8) * P);
  const int64_t KT4 = svq::round4(ng);
  for (int p = 0; p < P; ++p)
    for (int64_t n = 0; n < N; ++n)
      std::memcpy(alpha_f16 + ((int64_t)p * N + n) * ng, a + ((int64_t)p * N16 + n) * KT4, (size_t)(ng * 2));
  return SVQ_OK;
}

// sa blob: the sign section, then the code rows (CG bytes each), then the d
// rows (KS2 fp16 entries each); padding is zero.
int pack_sa(const int8_t* signs, const uint8_t* codes, const uint16_t* d_f16, int64_t N, int64_t K, int32_t G,
            int32_t P, uint8_t* packed) {
  svq::clear_error();
  if (!signs || !codes || !d_f16 || !packed) return svq::fail(SVQ_ERR_NULL, "pack_sa: NULL pointer");
  if (int rc = check_sa(N, K, G, P)) return rc;
  if (int rc = check_signs("pack_sa", signs, N, K, P)) return rc;
  const int64_t N16 = svq::round16(N), KT4 = svq::round4(K / 128), ng = K / G, ns = K / 256;
  const int64_t CG = KT4 * 128 / G, KS2 = KT4 / 2;
  put_signs(signs, N, K, P, packed);
  uint8_t* a = packed + N16 * (K / 8) * P;
  std::memset(a, 0, (size_t)(P * N16 * CG));
  for (int p = 0; p < P; ++p)
    for (int64_t n = 0; n < N; ++n) std::memcpy(a + ((int64_t)p * N16 + n) * CG, codes + ((int64_t)p * N + n) * ng, (size_t)ng);
  uint16_t* d = reinterpret_cast<uint16_t*>(a + P * N16 * CG);
  std::memset(d, 0, (size_t)(N16 * KS2 * 2));
  for (int64_t n = 0; n < N; ++n) std::memcpy(d + n * KS2, d_f16 + n * ns, (size_t)(ns * 2));
  return SVQ_OK;
}

int unpack_sa(const uint8_t* packed, int64_t N, int64_t K, int32_t G, int32_t P, int8_t* signs, uint8_t* codes,
              uint16_t* d_f16) {
  svq::clear_error();
  if (!signs || !codes || !d_f16 || !packed) return svq::fail(SVQ_ERR_NULL, "unpack_sa: NULL pointer");
  if (int rc = check_sa(N, K, G, P)) return rc;
  const int64_t N16 = svq::round16(N), KT4 = svq::round4(K / 128), ng = K / G, ns = K / 256;
  const int64_t CG = KT4 * 128 / G, KS2 = KT4 / 2;
  get_signs(packed, N, K, P, signs);
  const uint8_t* a = packed + N16 * (K / 8) * P;
  for (int p = 0; p < P; ++p)
    for (int64_t n = 0; n < N; ++n) std::memcpy(codes + ((int64_t)p * N + n) * ng, a + ((int64_t)p * N16 + n) * CG, (size_t)ng);
  const uint16_t* d = reinterpret_cast<const uint16_t*>(a + P * N16 * CG);
  for (int64_t n = 0; n < N; ++n) std::memcpy(d_f16 + n * ns, d + n * KS2, (size_t)(ns * 2));
  return SVQ_OK;
}

}  // extern "C"
