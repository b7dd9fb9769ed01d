// svq_sa_gemv.hip -- M = 1 device entry point for the sa* storage of sign
// planes (ShiftAddQwen README, "Method / Format": per 256-weight super-block
// of a row, u8 scale codes a per plane and group of G in {64, 128, 256} and
// one fp16 d, alpha = d * a): the decode mat-vec.
//   y = sum_j d[n][j] * sum_{g in j} sum_p a[p][n][g] * sum_{k in g} b[p][n][k] x[k]
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"
#include "launch.h"
#include "svq.h"
#include "svq_internal.h"

extern "C" {

int gemv_sa(const uint8_t* packed, const uint16_t* x, uint16_t* y, int64_t N, int64_t K, int32_t G, int32_t P,
            void* stream) {
  if (int rc = check_sa("gemv_sa", packed, x, y, 1, N, K, G, P)) return rc;
  Shape sh;
  if (int rc = plan(N, K, 1, kPrefGemv, &sh)) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint32_t* xw = reinterpret_cast<const uint32_t*>(x);
  dispatch_group(G, [&](auto Gc) {
    dispatch_p(P, [&](auto Pc) {
      if constexpr (decltype(Pc)::value >= 2) {
        using F = SaFmt<decltype(Pc)::value, decltype(Gc)::value>;
        dispatch<kMaxDepthSa>(sh, [&](auto G, auto W, auto D) {
          hipLaunchKernelGGL((k_gemv_planes<SVQ_KARGS_F(F, G, W, D), false>), dim3(sh.grid), dim3(64 * sh.waves), 0,
                             st, packed, xw, y, (uint8_t*)nullptr, HeadOut{}, (int)N, sh.KT, sh.NT);
        });
      }
    });
  });
  return launched("gemv_sa");
}

}  // extern "C"
