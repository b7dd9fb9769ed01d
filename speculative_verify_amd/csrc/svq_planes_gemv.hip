// svq_planes_gemv.hip -- M = 1 device entry points for binary-plane weights
// (P sign planes, one fp16 scale per plane, row and group of 128): the decode
// mat-vec and the one-token LM head with fused argmax.
//   y = sum_g sum_p alpha[p][n][g] * sum_{k in g} b[p][n][k] x[k]
//   (ShiftAddQwen README, intro and "Method / Format")
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"
#include "launch.h"
#include "svq.h"
#include "svq_internal.h"

namespace svq {

int launch_binplane_head_m1(const char* fn, const uint8_t* packed, const uint16_t* x, int64_t N, int64_t K,
                            int32_t P, const int32_t* row_ids, int32_t* argmax, float* maxlogit, void* workspace,
                            void* stream) {
  Shape sh;
  if (int rc = plan(N, K, 1, kPrefHeadM1, &sh)) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint32_t* xw = reinterpret_cast<const uint32_t*>(x);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  const HeadOut ho = with_levels(HeadOut{row_ids, argmax, maxlogit, nullptr, nullptr, 0}, sh);
  dispatch_p(P, [&](auto Pc) {
    using F = PlaneFmt<decltype(Pc)::value>;
    dispatch(sh, [&](auto G, auto W, auto D) {
      hipLaunchKernelGGL((k_gemv_planes<SVQ_KARGS_F(F, G, W, D), true>), dim3(sh.grid), dim3(64 * sh.waves), 0,
                         st, packed, xw, (uint16_t*)nullptr, ws, ho, (int)N, sh.KT, sh.NT);
    });
  });
  return launched(fn);
}

}  // namespace svq

extern "C" {

int gemv_binplane(const uint8_t* packed, const uint16_t* x, uint16_t* y, int64_t N, int64_t K, int32_t G, int32_t P,
                  void* stream) {
  if (P == 0) return svq::fail(SVQ_ERR_SHAPE, "gemv_binplane: P=0 must be in 1..6");
  if (int rc = check_linear("gemv_binplane", packed, x, y, 1, N, K, G, P)) return rc;
  Shape sh;
  if (int rc = plan(N, K, 1, kPrefGemv, &sh)) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint32_t* xw = reinterpret_cast<const uint32_t*>(x);
  dispatch_p(P, [&](auto Pc) {
    using F = PlaneFmt<decltype(Pc)::value>;
    dispatch(sh, [&](auto G, auto W, auto D) {
      hipLaunchKernelGGL((k_gemv_planes<SVQ_KARGS_F(F, G, W, D), false>), dim3(sh.grid),
                         dim3(64 * sh.waves), 0, st, packed, xw, y, (uint8_t*)nullptr, HeadOut{}, (int)N,
                         sh.KT, sh.NT);
    });
  });
  return launched("gemv_binplane");
}

}  // extern "C"
