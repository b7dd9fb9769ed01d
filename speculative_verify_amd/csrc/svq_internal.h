// Internal helpers shared by the library's host translation units.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <thread>
#include <vector>

namespace svq {

// Per-thread message behind svq_last_error().
char* error_buffer();

inline void clear_error() { error_buffer()[0] = '\0'; }

// Record a message for the calling thread and return `code`.
__attribute__((format(printf, 2, 3))) inline int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(error_buffer(), 512, fmt, ap);
  va_end(ap);
  return code;
}

// One-token sign-plane LM head (arguments already checked): launches the
// mat-vec kernel with fused argmax.  Defined with the mat-vec kernels so that
// their instantiations stay in one translation unit.
int launch_binplane_head_m1(const char* fn, const uint8_t* packed, const uint16_t* x, int64_t N, int64_t K,
                            int32_t P, const int32_t* row_ids, int32_t* argmax, float* maxlogit, void* workspace,
                            void* stream);

// Host helpers of the packers and quantizers.
// Split [0, n) over the host's threads; each chunk is independent.
template <class F>
inline void parallel_for(int64_t n, F f) {
  int nt = (int)std::thread::hardware_concurrency();
  if (nt < 1) nt = 1;
  if (nt > 32) nt = 32;
  if (n < 64 || nt == 1) {
    f((int64_t)0, n);
    return;
  }
  std::vector<std::thread> th;
  const int64_t chunk = (n + nt - 1) / nt;
  for (int i = 0; i < nt; ++i) {
    const int64_t lo = i * chunk, hi = lo + chunk < n ? lo + chunk : n;
    if (lo >= hi) break;
    th.emplace_back([=] { f(lo, hi); });
  }
  for (auto& t : th) t.join();
}

inline int64_t round16(int64_t n) { return (n + 15) / 16 * 16; }
inline int64_t round4(int64_t n) { return (n + 3) / 4 * 4; }

}  // namespace svq
