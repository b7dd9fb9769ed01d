// svq_planes_gemm.hip -- small-M device entry points for binary-plane
// weights (P sign planes, one fp16 scale per plane, row and group of 128):
// the verify mat-mul and the LM head with fused argmax, whose one-token case
// launches the mat-vec kernel of svq_planes_gemv.hip.
//   Y = X W^T with W[n][k] = sum_p alpha[p][n][k/128] * b[p][n][k]
//   (ShiftAddQwen README, intro and "Method / Format")
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"
#include "launch.h"
#include "mmq_planes.h"
#include "svq.h"
#include "svq_internal.h"

extern "C" {

int gemm_smallm_binplane(const uint8_t* packed, const uint16_t* X, uint16_t* Y, int32_t M, int64_t N, int64_t K,
                         int32_t G, int32_t P, void* stream) {
  if (P == 0) return svq::fail(SVQ_ERR_SHAPE, "gemm_smallm_binplane: P=0 must be in 1..6");
  if (int rc = check_linear("gemm_smallm_binplane", packed, X, Y, M, N, K, G, P, SVQ_MAX_M_GEMM)) return rc;
  if (M > SVQ_BLOCK_M) {
    // Consecutive launches of at most SVQ_BLOCK_M rows, each reading the
    // weights once.
    for (int32_t m0 = 0; m0 < M; m0 += SVQ_BLOCK_M) {
      const int32_t Mb = M - m0 < SVQ_BLOCK_M ? M - m0 : SVQ_BLOCK_M;
      if (int rc = gemm_smallm_binplane(packed, X + (size_t)m0 * K, Y + (size_t)m0 * N, Mb, N, K, G, P, stream))
        return rc;
    }
    return SVQ_OK;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  bool two = false;
  if (M > SVQ_MAX_M && K <= 4096)
    if (int rc = use_two_mtiles(N, M, P <= 4, &two)) return rc;
  if (M > SVQ_MAX_M && K <= 4096 && !two) {
    // The block as ceil(M / 16) m-tiles of the M <= 16 kernel in one launch.
    Shape sh;
    int ms = 1;
    if (int rc = plan_msplit(N, K, M, kPrefGemmPlanes, &sh, &ms)) return rc;
    const uint32_t* Xw = reinterpret_cast<const uint32_t*>(X);
    dispatch_p(P, [&](auto Pc) {
      using F = PlaneFmt<decltype(Pc)::value>;
      dispatch<kMaxDepthPlanesGemm>(sh, [&](auto G, auto W, auto D) {
        hipLaunchKernelGGL((k_gemm_planes<SVQ_KARGS_F(F, G, W, D), false>), dim3(sh.grid), dim3(64 * sh.waves), 0,
                           st, packed, Xw, Y, (uint8_t*)nullptr, HeadOut{}, M, (int)N, sh.KT, sh.NT, ms);
      });
    });
    return launched("gemm_smallm_binplane");
  }
  if (two) {
    // Two m-tiles held in registers: the M <= 16 kernel's eight-wave shape,
    // each decoded weight feeding both m-tiles.
    Shape sh;
    if (int rc = plan(N, K, 4, kPrefGemmPlanes, &sh)) return rc;
    dispatch_p(P, [&](auto Pc) {
      if constexpr (decltype(Pc)::value <= 4) {
        using F = PlaneFmt<decltype(Pc)::value>;
        auto go = [&](auto Gc) {
          hipLaunchKernelGGL((k_gemm_planes_x2<F, decltype(Gc)::value, 1>), dim3(sh.grid), dim3(64 * sh.waves), 0,
                             st, packed, X, Y, M, (int)N, sh.KT, sh.NT);
        };
        if (sh.gpw == 1) go(ic<1>{});
        else if (sh.gpw == 2) go(ic<2>{});
        else go(ic<4>{});
      }
    });
    return launched("gemm_smallm_binplane");
  }
  if (M > SVQ_MAX_M) {
    // Blocks of 17..64 rows above K = 4096: the weights are read and decoded
    // once for the whole block (mmq_planes.h).
    int rc = SVQ_OK;
    dispatch_p(P, [&](auto Pc) {
      rc = launch_mmq_planes<MmqPlanes<decltype(Pc)::value>>("gemm_smallm_binplane", packed, X, Y, M, N, K, st);
    });
    return rc;
  }
  Shape sh;
  if (int rc = plan(N, K, 4, kPrefGemmPlanes, &sh)) return rc;
  const uint32_t* Xw = reinterpret_cast<const uint32_t*>(X);
  dispatch_p(P, [&](auto Pc) {
    using F = PlaneFmt<decltype(Pc)::value>;
    dispatch<kMaxDepthPlanesGemm>(sh, [&](auto G, auto W, auto D) {
      hipLaunchKernelGGL((k_gemm_planes<SVQ_KARGS_F(F, G, W, D), false>), dim3(sh.grid), dim3(64 * sh.waves), 0, st,
                         packed, Xw, Y, (uint8_t*)nullptr, HeadOut{}, M, (int)N, sh.KT, sh.NT, 1);
    });
  });
  return launched("gemm_smallm_binplane");
}

int lmhead_argmax_binplane(const uint8_t* packed, const uint16_t* X, int32_t M, int64_t N, int64_t K, int32_t G,
                           int32_t P, const int32_t* row_ids, int32_t* argmax, float* maxlogit, void* workspace,
                           size_t workspace_bytes, void* stream) {
  svq::clear_error();
  if (P < 1 || P > SVQ_MAX_P) return svq::fail(SVQ_ERR_SHAPE, "lmhead_argmax_binplane: P=%d must be in 1..6", P);
  const char* fn = "lmhead_argmax_binplane";
  const HeadOut ho{row_ids, argmax, maxlogit, nullptr, nullptr};
  if (int rc = check_head(fn, packed, X, M, N, K, G, P, ho, workspace, workspace_bytes)) return rc;
  if (M == 1)
    return svq::launch_binplane_head_m1(fn, packed, X, N, K, P, row_ids, argmax, maxlogit, workspace, stream);
  Shape sh;
  if (int rc = plan(N, K, 4, kPrefGemmPlanes, &sh)) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint32_t* Xw = reinterpret_cast<const uint32_t*>(X);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  dispatch_p(P, [&](auto Pc) {
    using F = PlaneFmt<decltype(Pc)::value>;
    dispatch<kMaxDepthPlanesGemm>(sh, [&](auto G, auto W, auto D) {
      hipLaunchKernelGGL((k_gemm_planes<SVQ_KARGS_F(F, G, W, D), true>), dim3(sh.grid), dim3(64 * sh.waves), 0,
                         st, packed, Xw, (uint16_t*)nullptr, ws, with_levels(ho, sh), M, (int)N, sh.KT, sh.NT, 1);
    });
  });
  return launched(fn);
}

}  // extern "C"
