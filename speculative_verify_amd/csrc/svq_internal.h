// Internal helpers shared by the library's host translation units.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>

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

inline int64_t round16(int64_t n) { return (n + 15) / 16 * 16; }
inline int64_t round4(int64_t n) { return (n + 3) / 4 * 4; }

}  // namespace svq
