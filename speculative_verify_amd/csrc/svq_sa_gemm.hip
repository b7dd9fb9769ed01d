// svq_sa_gemm.hip -- small-M device entry point for the sa* storage of sign
// planes (ShiftAddQwen README, "Method / Format"): the verify mat-mul over a
// drafted block of M <= 16 rows on 16x16x32 bf16 MFMA, and blocks of up to
// 64 rows on the same kernel (or the streaming kernel of mmq_planes.h above
// K = 4096).
//   Y = X W^T with W[n][k] = d[n][k/256] * sum_p a[p][n][k/G] * b[p][n][k]
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"
#include "launch.h"
#include "mmq_planes.h"
#include "svq.h"
#include "svq_internal.h"

extern "C" {

int gemm_smallm_sa(const uint8_t* packed, const uint16_t* X, uint16_t* Y, int32_t M, int64_t N, int64_t K,
                   int32_t G, int32_t P, void* stream) {
  if (int rc = check_sa("gemm_smallm_sa", packed, X, Y, M, N, K, G, P, SVQ_MAX_M_GEMM)) return rc;
  if (M > SVQ_BLOCK_M) {
    // Consecutive launches of at most SVQ_BLOCK_M rows, each reading the
    // weights once.
    for (int32_t m0 = 0; m0 < M; m0 += SVQ_BLOCK_M) {
      const int32_t Mb = M - m0 < SVQ_BLOCK_M ? M - m0 : SVQ_BLOCK_M;
      if (int rc = gemm_smallm_sa(packed, X + (size_t)m0 * K, Y + (size_t)m0 * N, Mb, N, K, G, P, stream)) return rc;
    }
    return SVQ_OK;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint32_t* Xw = reinterpret_cast<const uint32_t*>(X);
  // The M <= 16 kernel over ms m-tiles of 16 rows (ms = 1 for M <= 16).
  auto launch_tiles = [&](const Shape& sh, int ms) {
    dispatch_group(G, [&](auto Gc) {
      dispatch_p(P, [&](auto Pc) {
        if constexpr (decltype(Pc)::value >= 2) {
          using F = SaFmt<decltype(Pc)::value, decltype(Gc)::value>;
          dispatch<kMaxDepthSa>(sh, [&](auto G, auto W, auto D) {
            hipLaunchKernelGGL((k_gemm_planes<SVQ_KARGS_F(F, G, W, D), false>), dim3(sh.grid), dim3(64 * sh.waves),
                               0, st, packed, Xw, Y, (uint8_t*)nullptr, HeadOut{}, M, (int)N, sh.KT, sh.NT, ms);
          });
        }
      });
    });
    return launched("gemm_smallm_sa");
  };
  bool two = false;
  if (M > SVQ_MAX_M && K <= 4096)
    if (int rc = use_two_mtiles(N, M, P <= 4 && G != 64, &two)) return rc;
  if (M > SVQ_MAX_M && K <= 4096 && !two) {
    // The block as ceil(M / 16) m-tiles of the M <= 16 kernel in one launch.
    Shape sh;
    int ms = 1;
    if (int rc = plan_msplit(N, K, M, kPrefGemmPlanes, &sh, &ms)) return rc;
    return launch_tiles(sh, ms);
  }
  if (two) {
    // Two m-tiles held in registers (k_gemm_planes_x2), each decoded weight
    // feeding both m-tiles.
    Shape sh;
    if (int rc = plan(N, K, 4, kPrefGemmPlanes, &sh)) return rc;
    dispatch_group(G, [&](auto Gc) {
      dispatch_p(P, [&](auto Pc) {
        constexpr int Pv = decltype(Pc)::value, Gv = decltype(Gc)::value;
        if constexpr (Pv >= 2 && Pv <= 4 && Gv != 64) {
          using F = SaFmt<Pv, Gv>;
          auto go = [&](auto GPWc) {
            hipLaunchKernelGGL((k_gemm_planes_x2<F, decltype(GPWc)::value, 1>), dim3(sh.grid), dim3(64 * sh.waves),
                               0, st, packed, X, Y, M, (int)N, sh.KT, sh.NT);
          };
          if (sh.gpw == 1) go(ic<1>{});
          else if (sh.gpw == 2) go(ic<2>{});
          else go(ic<4>{});
        }
      });
    });
    return launched("gemm_smallm_sa");
  }
  if (M > SVQ_MAX_M) {
    // Blocks of 17..64 rows above K = 4096: the weights are read and decoded
    // once for the whole block (mmq_planes.h).
    int rc = SVQ_OK;
    dispatch_group(G, [&](auto Gc) {
      dispatch_p(P, [&](auto Pc) {
        if constexpr (decltype(Pc)::value >= 2)
          rc = launch_mmq_planes<MmqSa<decltype(Pc)::value, decltype(Gc)::value>>("gemm_smallm_sa", packed, X, Y, M, N,
                                                                                   K, st);
      });
    });
    return rc;
  }
  Shape sh;
  if (int rc = plan(N, K, 4, kPrefGemmPlanes, &sh)) return rc;
  return launch_tiles(sh, 1);
}

}  // extern "C"
