// svq_int4.hip -- device entry points for W4A16 weights (symmetric INT4
// codes, one bf16 scale per group of 128): decode mat-vec, small-M verify
// mat-mul, and the LM head with fused argmax and greedy acceptance.
//   y = sum_g s[n][g] * sum_{k in g} c[n][k] x[k]
//   (Efficient Qwen Competition report, sec. 2.1 and 3.3)
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kernels.h"
#include "launch.h"
#include "mmq.h"
#include "svq.h"
#include "svq_internal.h"

namespace {

// Launch of the W4A16 head once its arguments are checked.
int launch_head_w4a16(const char* fn, const uint8_t* packed, const uint16_t* X, int32_t M, int64_t N, int64_t K,
                      int32_t G, const HeadOut& ho, void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = check_head(fn, packed, X, M, N, K, G, 0, ho, workspace, workspace_bytes)) return rc;
  Shape sh;
  if (int rc = plan(N, K, M == 1 ? 1 : 4, M == 1 ? kPrefHeadM1 : kPrefHeadM16, &sh)) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint32_t* Xw = reinterpret_cast<const uint32_t*>(X);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  const HeadOut h = with_levels(ho, sh);
  if (M == 1) {
    dispatch<6, 2>(sh, [&](auto G, auto W, auto D) {
      hipLaunchKernelGGL((k_gemv_w4a16<SVQ_KARGS(G, W, D), true>), dim3(sh.grid), dim3(64 * sh.waves), 0, st,
                         packed, Xw, (uint16_t*)nullptr, ws, h, (int)N, sh.KT, sh.NT);
    });
  } else {
    dispatch(sh, [&](auto G, auto W, auto D) {
      hipLaunchKernelGGL((k_gemm_w4a16<SVQ_KARGS(G, W, D), true>), dim3(sh.grid), dim3(64 * sh.waves), 0, st,
                         packed, Xw, (uint16_t*)nullptr, ws, h, M, (int)N, sh.KT, sh.NT, 1);
    });
  }
  return launched(fn);
}

// Scratch of lmhead_argmax_noalloc: the argmax completion state (per-row
// keys and counters, the layout of a head workspace) in device memory the
// library owns, one copy per GPU, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device, and that pointer is what the
// kernels receive.
constexpr size_t kScratchBytes = kWsBytes;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void __launch_bounds__(256) k_clear_scratch(uint4* __restrict__ p, int n16) {
  for (int i = threadIdx.x; i < n16; i += blockDim.x) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// The current device's scratch address.  On the first call on a device the
// address is looked up and the scratch is cleared by a kernel on `st`,
// ordered before the caller's launch; every head launch leaves it zero again.
int device_scratch(const char* fn, hipStream_t st, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return svq::fail(SVQ_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return svq::fail(SVQ_ERR_HIP, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return svq::fail(SVQ_ERR_HIP, "%s: hipGetSymbolAddress: %s", fn, hipGetErrorString(e));
    hipLaunchKernelGGL(k_clear_scratch, dim3(1), dim3(256), 0, st, reinterpret_cast<uint4*>(p),
                       (int)(kScratchBytes / 16));
    if (int rc = launched(fn)) return rc;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SVQ_OK;
}

}  // namespace

extern "C" {

int gemv_w4a16(const uint8_t* packed, const uint16_t* x, uint16_t* y, int64_t N, int64_t K, int32_t G,
               void* stream) {
  if (int rc = check_linear("gemv_w4a16", packed, x, y, 1, N, K, G, 0)) return rc;
  Shape sh;
  if (int rc = plan(N, K, 1, kPrefGemvW4, &sh)) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint32_t* xw = reinterpret_cast<const uint32_t*>(x);
  dispatch<6, 2>(sh, [&](auto G, auto W, auto D) {
    hipLaunchKernelGGL((k_gemv_w4a16<SVQ_KARGS(G, W, D), false>), dim3(sh.grid), dim3(64 * sh.waves), 0, st,
                       packed, xw, y, (uint8_t*)nullptr, HeadOut{}, (int)N, sh.KT, sh.NT);
  });
  return launched("gemv_w4a16");
}

int gemm_smallm_w4a16(const uint8_t* packed, const uint16_t* X, uint16_t* Y, int32_t M, int64_t N, int64_t K,
                      int32_t G, void* stream) {
  if (int rc = check_linear("gemm_smallm_w4a16", packed, X, Y, M, N, K, G, 0, SVQ_MAX_M_GEMM)) return rc;
  if (M > SVQ_BLOCK_M) {
    // Consecutive launches of at most SVQ_BLOCK_M rows (the exact-operand
    // kernels below; each reads the weights once).
    for (int32_t m0 = 0; m0 < M; m0 += SVQ_BLOCK_M) {
      const int32_t Mb = M - m0 < SVQ_BLOCK_M ? M - m0 : SVQ_BLOCK_M;
      if (int rc = gemm_smallm_w4a16(packed, X + (size_t)m0 * K, Y + (size_t)m0 * N, Mb, N, K, G, stream)) return rc;
    }
    return SVQ_OK;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  bool two = false;
  if (M > SVQ_MAX_M && K <= 4096)
    if (int rc = use_two_mtiles(N, M, true, &two)) return rc;
  if (M > SVQ_MAX_M && K <= 4096 && !two) {
    // The block as ceil(M / 16) m-tiles of the M <= 16 kernel in one launch.
    Shape sh;
    int ms = 1;
    if (int rc = plan_msplit(N, K, M, kPrefGemmW4, &sh, &ms)) return rc;
    const uint32_t* Xw = reinterpret_cast<const uint32_t*>(X);
    dispatch(sh, [&](auto G, auto W, auto D) {
      hipLaunchKernelGGL((k_gemm_w4a16<SVQ_KARGS(G, W, D), false>), dim3(sh.grid), dim3(64 * sh.waves), 0, st,
                         packed, Xw, Y, (uint8_t*)nullptr, HeadOut{}, M, (int)N, sh.KT, sh.NT, ms);
    });
    return launched("gemm_smallm_w4a16");
  }
  if (two) {
    // Two m-tiles held in registers: the M <= 16 kernel's eight-wave shape.
    Shape sh;
    if (int rc = plan(N, K, 4, kPrefGemmW4, &sh)) return rc;
    auto launch = [&](auto Gc, auto Dc) {
      hipLaunchKernelGGL((k_gemm_w4a16_x2<decltype(Gc)::value, decltype(Dc)::value>), dim3(sh.grid),
                         dim3(64 * sh.waves), 0, st, packed, X, Y, M, (int)N, sh.KT, sh.NT);
    };
    auto by_depth = [&](auto Gc) {
      // At four groups a wave the two m-tiles' activations leave registers
      // for a one-tile ring only.
      if constexpr (decltype(Gc)::value < 4) {
        if (sh.depth >= 2) return launch(Gc, ic<2>{});
      }
      launch(Gc, ic<1>{});
    };
    if (sh.gpw == 1) by_depth(ic<1>{});
    else if (sh.gpw == 2) by_depth(ic<2>{});
    else by_depth(ic<4>{});
    return launched("gemm_smallm_w4a16");
  }
  if (M > SVQ_MAX_M) {
    // Blocks of 17..64 rows above K = 4096: X streams with the weights.
    MmqShape sh;
    if (int rc = plan_mmq(N, M, &sh)) return rc;
    const int KT = (int)(K / 128), NT = (int)((N + 15) / 16);
    // Every workgroup runs a multiple of CK steps (CK column tiles per wave
    // and block), and the unrolled ring loop runs whole rounds of D steps:
    // a depth of 3 is kept only where CK is a multiple of 3 (or of neither 2
    // nor 3), so no round ends in steps on empty tiles.
    const int CK = (KT + kMmqWaves - 1) / kMmqWaves;
    const bool three = CK % 3 == 0 || CK % 2 != 0;
    auto launch = [&](auto MTc, auto Rc, auto Dc) {
      hipLaunchKernelGGL((k_gemm_mmq_w4a16<decltype(MTc)::value, decltype(Rc)::value, decltype(Dc)::value>),
                         dim3(sh.grid), dim3(64 * kMmqWaves), 0, st, packed, X, Y, M, (int)N, (int)K, KT, NT);
    };
    dispatch_r(sh.R, [&](auto Rc) {
      constexpr int R = decltype(Rc)::value;
      // The deepest weight ring that stays in registers for the block height
      // (3 tiles, or 2), where the step count allows it.
      if (M <= 32) {
        if (R != 4 && three) launch(ic<2>{}, Rc, ic<3>{});
        else launch(ic<2>{}, Rc, ic<2>{});
      } else {
        constexpr int R3 = R < 4 ? R : 3;
        auto by_m = [&](auto MTc) {
          if (R < 3 && three) launch(MTc, ic<R3>{}, ic<3>{});
          else launch(MTc, ic<R3>{}, ic<2>{});
        };
        if (M <= 48) by_m(ic<3>{});
        else by_m(ic<4>{});
      }
    });
    return launched("gemm_smallm_w4a16");
  }
  Shape sh;
  if (int rc = plan(N, K, 4, kPrefGemmW4, &sh)) return rc;
  const uint32_t* Xw = reinterpret_cast<const uint32_t*>(X);
  dispatch(sh, [&](auto G, auto W, auto D) {
    hipLaunchKernelGGL((k_gemm_w4a16<SVQ_KARGS(G, W, D), false>), dim3(sh.grid), dim3(64 * sh.waves), 0, st,
                       packed, Xw, Y, (uint8_t*)nullptr, HeadOut{}, M, (int)N, sh.KT, sh.NT, 1);
  });
  return launched("gemm_smallm_w4a16");
}

int lmhead_argmax(const uint8_t* packed, const uint16_t* X, int32_t M, int64_t N, int64_t K, int32_t G,
                  const int32_t* row_ids, int32_t* argmax, float* maxlogit, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return launch_head_w4a16("lmhead_argmax", packed, X, M, N, K, G, HeadOut{row_ids, argmax, maxlogit, nullptr, nullptr},
                     workspace, workspace_bytes, stream);
}

int lmhead_argmax_noalloc(const uint8_t* packed, const uint16_t* X, int32_t M, int64_t N, int64_t K, int32_t G,
                          const int32_t* row_ids, int32_t* argmax, float* maxlogit, void* stream) {
  const char* fn = "lmhead_argmax_noalloc";
  svq::clear_error();
  if (M < 1 || M > SVQ_MAX_M || svq_lmhead_workspace_bytes(M) > kScratchBytes)
    return svq::fail(SVQ_ERR_SHAPE, "%s: M=%d must be in 1..%d (the static scratch holds %zu bytes of argmax state)",
                     fn, M, SVQ_MAX_M, kScratchBytes);
  // Every argument check runs before the scratch is touched.
  const HeadOut ho{row_ids, argmax, maxlogit, nullptr, nullptr};
  if (int rc = check_head_args(fn, packed, X, M, N, K, G, 0, ho)) return rc;
  void* ws = nullptr;
  if (int rc = device_scratch(fn, reinterpret_cast<hipStream_t>(stream), &ws)) return rc;
  return launch_head_w4a16(fn, packed, X, M, N, K, G, ho, ws, kScratchBytes, stream);
}

int lmhead_verify_greedy(const uint8_t* packed, const uint16_t* X, int32_t M, int64_t N, int64_t K, int32_t G,
                         const int32_t* row_ids, const int32_t* draft_ids, int32_t* argmax, float* maxlogit,
                         int32_t* accept_len, void* workspace, size_t workspace_bytes, void* stream) {
  svq::clear_error();
  if (!accept_len || (M > 1 && !draft_ids))
    return svq::fail(SVQ_ERR_NULL, "lmhead_verify_greedy: NULL accept_len or draft_ids");
  if (misaligned(accept_len, 4) || (draft_ids && misaligned(draft_ids, 4)))
    return svq::fail(SVQ_ERR_ALIGN, "lmhead_verify_greedy: accept_len and draft_ids must be 4-byte aligned");
  return launch_head_w4a16("lmhead_verify_greedy", packed, X, M, N, K, G,
                           HeadOut{row_ids, argmax, maxlogit, draft_ids, accept_len}, workspace, workspace_bytes, stream);
}

}  // extern "C"
