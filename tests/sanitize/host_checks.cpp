// Host code of the library (packers, unpackers, quantizers) on seeded small
// inputs with ragged shapes, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers.py.  Every packer is
// checked by its round trip, every quantizer for its output ranges, and the
// argument checks by their error codes.  Exit status 0 means every check
// passed and no sanitizer fired.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "svq.h"

namespace svq {
// The library's per-thread error message (defined with the device entry
// points in the full build).
char* error_buffer() {
  static thread_local char buf[512];
  return buf;
}
}  // namespace svq

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}

int g_fail = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

uint16_t bf16_of(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

void int4_round_trip(int64_t N, int64_t K) {
  std::vector<int8_t> codes(N * K), codes2(N * K);
  std::vector<uint16_t> scales(N * (K / 128)), scales2(scales.size());
  for (auto& c : codes) c = (int8_t)((int)(next_u32() % 16) - 8);
  for (auto& s : scales) s = bf16_of(0.005f + 0.015f * (next_u32() % 1000) / 1000.f);
  std::vector<uint8_t> blob(svq_int4_packed_bytes(N, K, 128));
  CHECK(pack_int4_grouped(codes.data(), scales.data(), N, K, 128, blob.data()) == SVQ_OK);
  CHECK(unpack_int4_grouped(blob.data(), N, K, 128, codes2.data(), scales2.data()) == SVQ_OK);
  CHECK(codes == codes2 && scales == scales2);
  codes[N * K - 1] = 8;  // out of range: rejected
  CHECK(pack_int4_grouped(codes.data(), scales.data(), N, K, 128, blob.data()) == SVQ_ERR_RANGE);
}

void planes_round_trip(int64_t N, int64_t K, int32_t P) {
  std::vector<int8_t> signs(P * N * K), signs2(signs.size());
  std::vector<uint16_t> alpha(P * N * (K / 128)), alpha2(alpha.size());
  for (auto& b : signs) b = (next_u32() & 1) ? 1 : -1;
  for (auto& a : alpha) a = (uint16_t)(0x2000 + next_u32() % 0x1000);
  std::vector<uint8_t> blob(svq_binplane_packed_bytes(N, K, 128, P));
  CHECK(pack_binary_planes(signs.data(), alpha.data(), N, K, 128, P, blob.data()) == SVQ_OK);
  CHECK(unpack_binary_planes(blob.data(), N, K, 128, P, signs2.data(), alpha2.data()) == SVQ_OK);
  CHECK(signs == signs2 && alpha == alpha2);
}

void sa_round_trip(int64_t N, int64_t K, int32_t G, int32_t P) {
  std::vector<int8_t> signs(P * N * K), signs2(signs.size());
  std::vector<uint8_t> codes(P * N * (K / G)), codes2(codes.size());
  std::vector<uint16_t> d(N * (K / 256)), d2(d.size());
  for (auto& b : signs) b = (next_u32() & 1) ? 1 : -1;
  for (auto& c : codes) c = (uint8_t)next_u32();
  for (auto& v : d) v = (uint16_t)(0x0400 + next_u32() % 0x3000);
  std::vector<uint8_t> blob(svq_sa_packed_bytes(N, K, G, P));
  CHECK(pack_sa(signs.data(), codes.data(), d.data(), N, K, G, P, blob.data()) == SVQ_OK);
  CHECK(unpack_sa(blob.data(), N, K, G, P, signs2.data(), codes2.data(), d2.data()) == SVQ_OK);
  CHECK(signs == signs2 && codes == codes2 && d == d2);
}

void quantizers(int64_t N, int64_t K, int32_t G, int32_t P) {
  std::vector<uint16_t> w(N * K), scales(N * (K / G));
  for (auto& v : w) v = bf16_of(((int)(next_u32() % 2001) - 1000) * 4e-5f);
  for (auto& s : scales) s = bf16_of(0.005f + 0.015f * (next_u32() % 1000) / 1000.f);
  std::vector<int8_t> codes(N * K);
  CHECK(quantize_int4_frozen(w.data(), scales.data(), N, K, G, codes.data()) == SVQ_OK);
  for (int8_t c : codes) CHECK(c >= -8 && c <= 7);
  std::vector<int8_t> signs(P * N * K);
  std::vector<uint16_t> alpha(P * N * (K / G));
  CHECK(fit_binary_planes(w.data(), N, K, G, P, 6, signs.data(), alpha.data()) == SVQ_OK);
  for (int8_t b : signs) CHECK(b == 1 || b == -1);
  if (K % 256 == 0) {
    std::vector<uint8_t> sc(alpha.size());
    std::vector<uint16_t> d(N * (K / 256));
    CHECK(snap_sa_scales(alpha.data(), N, K, G, P, sc.data(), d.data()) == SVQ_OK);
  }
  CHECK(fit_binary_planes(w.data(), N, K, G, 7, 1, signs.data(), alpha.data()) == SVQ_ERR_SHAPE);
}

}  // namespace

int main() {
  for (int64_t N : {1, 15, 16, 17, 33})
    for (int64_t K : {128, 384, 1024}) {
      int4_round_trip(N, K);
      for (int32_t P : {1, 3, 6}) planes_round_trip(N, K, P);
    }
  for (int64_t N : {1, 17, 40})
    for (int64_t K : {256, 768})
      for (int32_t G : {64, 128, 256})
        for (int32_t P : {2, 3, 6}) sa_round_trip(N, K, G, P);
  for (int64_t N : {3, 70})
    for (int32_t G : {64, 128, 256}) quantizers(N, 512, G, G == 64 ? 4 : 3);
  CHECK(pack_int4_grouped(nullptr, nullptr, 1, 128, 128, nullptr) == SVQ_ERR_NULL);
  CHECK(svq_int4_packed_bytes(1, 100, 128) == 0);
  if (g_fail) std::fprintf(stderr, "%d checks failed\n", g_fail);
  else std::printf("host checks passed\n");
  return g_fail ? 1 : 0;
}
