// launch.h -- host-side helpers shared by the device entry points:
// argument checks, launch shapes and compile-time dispatch.
#pragma once

#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <type_traits>

#include "kernels.h"
#include "svq.h"
#include "svq_internal.h"

namespace {

inline std::atomic<int> g_cus[64];

inline int device_cus(int* cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return svq::fail(SVQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev >= 0 && dev < 64) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return SVQ_OK;
    }
  }
  int v = 0;
  e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return svq::fail(SVQ_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
  if (v < 1) v = 1;
  if (dev >= 0 && dev < 64) g_cus[dev].store(v, std::memory_order_relaxed);
  *cus = v;
  return SVQ_OK;
}

inline bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

inline int check_linear(const char* fn, const void* packed, const void* x, const void* y, int32_t M, int64_t N, int64_t K,
                        int32_t G, int32_t P, int32_t max_m = SVQ_MAX_M) {
  svq::clear_error();
  if (!packed || !x || !y) return svq::fail(SVQ_ERR_NULL, "%s: NULL pointer", fn);
  if (N < 1 || N > (int64_t)INT_MAX - 16) return svq::fail(SVQ_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
  if (G != SVQ_GROUP) return svq::fail(SVQ_ERR_SHAPE, "%s: group size must be 128 (got %d)", fn, G);
  if (K < SVQ_GROUP || K % SVQ_GROUP || K > SVQ_MAX_K)
    return svq::fail(SVQ_ERR_SHAPE, "%s: K=%lld must be a multiple of 128 in [128, %d]", fn, (long long)K, SVQ_MAX_K);
  if (M < 1 || M > max_m) return svq::fail(SVQ_ERR_SHAPE, "%s: M=%d must be in 1..%d", fn, M, max_m);
  if (P != 0 && (P < 1 || P > SVQ_MAX_P)) return svq::fail(SVQ_ERR_SHAPE, "%s: P=%d must be in 1..6", fn, P);
  const int64_t N16 = (N + 15) / 16 * 16;
  if (N16 * K / 2 >= ((int64_t)1 << 31) || (P != 0 && N16 * K / 8 * P >= ((int64_t)1 << 31)))
    return svq::fail(SVQ_ERR_SHAPE, "%s: packed weights must be smaller than 2 GiB (N=%lld, K=%lld)", fn,
                     (long long)N, (long long)K);
  if (misaligned(packed, 16)) return svq::fail(SVQ_ERR_ALIGN, "%s: packed weights must be 16-byte aligned", fn);
  if (misaligned(x, 16)) return svq::fail(SVQ_ERR_ALIGN, "%s: activations must be 16-byte aligned", fn);
  if (misaligned(y, 2)) return svq::fail(SVQ_ERR_ALIGN, "%s: output must be 2-byte aligned", fn);
  return SVQ_OK;
}

struct Shape {
  int KT, NT, gpw, waves, grid, depth;
};

inline int env_int(const char* name, int lo, int hi, int dflt) {
  const char* s = std::getenv(name);
  const int x = s ? std::atoi(s) : 0;
  return x >= lo && x <= hi ? x : dflt;
}

// Launch shape.  A workgroup owns one 16-row tile at a time and splits K
// across its waves (gpw groups each); the grid is one or a few workgroups per
// CU walking the row tiles in grid-stride order; the ring depth is the number
// of tiles whose loads each wave keeps in flight, at most the number of tiles
// every workgroup owns (so the pipeline tail stays short).
// wave_quantum: the M <= 16 kernels finish the tiles of a chunk one wave per
// tile (up to four tiles), so their workgroups carry a multiple of four waves.
// Measured on MI355X (rocprofv3 kernel traces of the decode, verify and head
// shapes at K = 4096, sweeping both knobs): the sign-plane and sa* mat-vecs
// run best at two workgroups per CU while the row tiles number at most three
// per CU and at one above (interleaved A/B, five rounds: N = 12288 3.4%
// slower at one, N = 8192 alike, N = 16384 and 28672 6-8% faster), the
// W4A16 mat-vec at one at every size (3-14% faster than at two for
// N = 8192..28672, K = 2048..8192), everything else at one workgroup per
// CU, all with a ring of <= 2 tiles; a ring of 2 tiles already keeps more bytes in flight
// than the memory system's bandwidth-latency product, and deeper rings were
// slower (the M = 16 sign-plane head at 32768 rows, eight tiles a
// workgroup: 26.4 us at a ring of 2, 28.7 at 3).  Workgroups of the M <= 16
// mat-muls that own at most `shallow` tiles run without a ring (depth 1).
// Interleaved A/B runs of ring 2 against no ring (six rounds each, since a
// partial last round of the ring no longer steps through empty tiles) gave:
// * three tiles a workgroup (N = 12288): the ring wins (W4A16 -2.6%, sign
//   planes -0.7%, sa* -1.4 to -4.5%);
// * two tiles (N = 8192): no ring wins (the ring costs +1.1%, +2.7% and
//   +3.4 to +4.6%), as the prefetch of the second tile delays the first
//   tile's activations and weights.
// K up to 4096 runs on eight waves of four column tiles.  Sixteen waves of
// two column tiles (the full-register form at 128 registers a lane) were
// measured and dropped: every M <= 16 mat-mul ran 7-16% slower (interleaved
// A/B runs after a 50 ms warm-up, W4A16, sign planes and sa* at N = 4096 and
// 12288): VALU and MFMA already keep the SIMDs busy once the data arrives,
// and twice the waves double the per-wave prologue and the cross-wave sums.
struct LaunchPref {
  int wgs_per_cu, max_depth, shallow;
  // Above wide_tiles row tiles per CU, wide_wgs workgroups per CU instead
  // (0: no such rule).
  int wide_tiles = 0, wide_wgs = 0;
};
constexpr LaunchPref kPrefGemv = {2, 2, 0, 3, 1};
constexpr LaunchPref kPrefGemvW4 = {1, 2, 0};
constexpr LaunchPref kPrefGemmW4 = {1, 2, 2};
constexpr LaunchPref kPrefGemmPlanes = {1, 2, 2};
constexpr LaunchPref kPrefHeadM1 = {1, 2, 0};
constexpr LaunchPref kPrefHeadM16 = {1, 2, 0};

inline int plan(int64_t N, int64_t K, int wave_quantum, LaunchPref pref, Shape* s) {
  int cus = 0;
  if (int rc = device_cus(&cus)) return rc;
  s->KT = (int)(K / 128);
  s->NT = (int)((N + 15) / 16);
  s->gpw = s->KT <= 8 ? 1 : s->KT <= 16 ? 2 : 4;
  s->waves = (s->KT + s->gpw - 1) / s->gpw;
  s->waves = (s->waves + wave_quantum - 1) / wave_quantum * wave_quantum;
  // SVQ_WG_PER_CU / SVQ_PIPE_DEPTH / SVQ_GRID_MAX override the preferences
  // (for tuning runs).
  const int wpc = pref.wide_tiles > 0 && s->NT > pref.wide_tiles * cus ? pref.wide_wgs : pref.wgs_per_cu;
  int want = cus * env_int("SVQ_WG_PER_CU", 1, 8, wpc);
  const int gmax = env_int("SVQ_GRID_MAX", 1, 1 << 20, want);
  if (gmax < want) want = gmax;
  s->grid = s->NT < want ? s->NT : want;
  const int tmin = s->NT / s->grid;
  const int dmax = env_int("SVQ_PIPE_DEPTH", 1, 6, pref.max_depth);
  const bool shallow = tmin <= pref.shallow && env_int("SVQ_PIPE_DEPTH", 1, 6, 0) == 0;
  s->depth = tmin < 1 || shallow ? 1 : tmin > dmax ? dmax : tmin;
  return SVQ_OK;
}

// Launch shape of a block of 16 < M <= 64 rows run as ms = ceil(M / 16)
// m-tiles on the M <= 16 kernels in one launch (TileWalk in kernels.h):
// ms * gper workgroups, gper a multiple of 8 of at most CUs / ms that does
// not exceed the row tiles rounded up to 8; the ring depth follows the row
// tiles each workgroup owns, as in plan().
inline int plan_msplit(int64_t N, int64_t K, int32_t M, LaunchPref pref, Shape* s, int* ms) {
  if (int rc = plan(N, K, 4, pref, s)) return rc;
  int cus = 0;
  if (int rc = device_cus(&cus)) return rc;
  *ms = (M + 15) / 16;
  const int sets = (s->NT + 7) / 8;
  int per = cus / (8 * *ms);
  per = per < 1 ? 1 : per > sets ? sets : per;
  const int gper = 8 * per;
  s->grid = gper * *ms;
  const int tmin = s->NT / gper;
  const int dmax = env_int("SVQ_PIPE_DEPTH", 1, 6, pref.max_depth);
  const bool shallow = tmin <= pref.shallow && env_int("SVQ_PIPE_DEPTH", 1, 6, 0) == 0;
  s->depth = tmin < 1 || shallow ? 1 : tmin > dmax ? dmax : tmin;
  return SVQ_OK;
}

// Kernel choice for a block of 16 < M <= 64 rows at K <= 4096 (interleaved
// A/B runs on MI355X, K = 4096 unless noted, against the streaming kernels
// of mmq.h / mmq_planes.h that read X with the weights):
// * the m-split (plan_msplit) was faster wherever it replaced them:
//   W4A16 M = 48 and 64 by 10-31% (N = 4096 and 12288; M = 64 at K = 2048
//   by 12%), sign planes and sa* M = 48 and 64 by 8-20%, P = 6 and sa* at
//   G = 64 by 8-24% (M = 32 and 64);
// * against the two-m-tile kernel (k_gemm_w4a16_x2, k_gemm_planes_x2:
//   M <= 32, P <= 4, sa* G >= 128), which decodes each weight tile once for
//   both m-tiles, the m-split won only where every workgroup owns a single
//   row tile (W4A16 M = 32, N = 4096: -10%) and lost where they own several
//   (N = 32768: +8% W4A16, +14% sign planes; N = 12288: +1-6% at M = 24 and
//   32 for sign planes and sa*, within noise for W4A16).
// So the two-m-tile kernel takes M <= 32 when the row tiles outnumber the
// CUs and the m-split takes every other block.
inline int use_two_mtiles(int64_t N, int32_t M, bool applies, bool* out) {
  int cus = 0;
  if (int rc = device_cus(&cus)) return rc;
  *out = applies && M <= 2 * SVQ_MAX_M && (N + 15) / 16 > cus;
  return SVQ_OK;
}

// Set by dispatch() when a planned launch is wider than every kernel shape it
// may instantiate (the launch is then skipped); reported by launched().
inline thread_local bool g_shape_mismatch = false;

inline int launched(const char* fn) {
  if (g_shape_mismatch) {
    g_shape_mismatch = false;
    return svq::fail(SVQ_ERR_SHAPE, "%s: no kernel shape for the planned launch", fn);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return svq::fail(SVQ_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return SVQ_OK;
}

template <int V>
using ic = std::integral_constant<int, V>;

// Launch shape of the 16 < M <= 64 kernels: R row tiles per block, so that
// about one block lands on each CU (at most four tiles, three above M = 32:
// a wave holds R x ceil(M / 16) accumulator tiles), and a grid of at most
// one workgroup per CU walking the blocks.
struct MmqShape {
  int R, grid;
};

inline int plan_mmq(int64_t N, int32_t M, MmqShape* s) {
  int cus = 0;
  if (int rc = device_cus(&cus)) return rc;
  const int NT = (int)((N + 15) / 16);
  const int rmax = M > 32 ? 3 : 4;  // the accumulators of R x ceil(M / 16) tiles must stay in registers
  int R = (NT + cus - 1) / cus;
  R = R < 1 ? 1 : R > rmax ? rmax : R;
  const int NB = (NT + R - 1) / R;
  s->R = R;
  s->grid = NB < cus ? NB : cus;
  return SVQ_OK;
}

// Calls launch(ic<R>) for the block height of a 16 < M <= 64 launch.
template <class L>
void dispatch_r(int R, L&& launch) {
  switch (R) {
    case 1: launch(ic<1>{}); break;
    case 2: launch(ic<2>{}); break;
    case 3: launch(ic<3>{}); break;
    default: launch(ic<4>{}); break;
  }
}

// Calls launch(ic<GPW>, ic<MAXW>, ic<D>) for the shape's compile-time
// parameters.  Depths above 2 are instantiated only for the 8-wave shapes,
// and none above MAXD (a shallower ring is launched instead).  The 16-wave
// shapes (K > 4096, 128 registers a lane) get a ring of at most MAXD16
// tiles: a second slot spills every kernel but the W4A16 mat-vec, which
// cost far more than the ring hides (measured at K = 8192, N = 32768, eight
// tiles a workgroup: without the ring the W4A16 verify mat-mul ran 32%
// faster, its head 17%, the P = 6 sign-plane kernels 31-35%, the P = 3 ones
// 2-6%, while the W4A16 mat-vec, which does not spill, ran 2% slower).
template <int MAXD = 6, int MAXD16 = 1, class L>
void dispatch(const Shape& sh, L&& launch) {
  auto depth = [&](auto G, auto W, auto DM) {
    if (sh.waves > decltype(W)::value) {  // the kernel's launch bounds would not hold
      g_shape_mismatch = true;
      return;
    }
    constexpr int dm = decltype(DM)::value < MAXD ? decltype(DM)::value : MAXD;
    if constexpr (dm >= 6)
      if (sh.depth >= 6) return launch(G, W, ic<6>{});
    if constexpr (dm >= 5)
      if (sh.depth >= 5) return launch(G, W, ic<5>{});
    if constexpr (dm >= 4)
      if (sh.depth >= 4) return launch(G, W, ic<4>{});
    if constexpr (dm >= 3)
      if (sh.depth >= 3) return launch(G, W, ic<3>{});
    if constexpr (dm >= 2)
      if (sh.depth >= 2) return launch(G, W, ic<2>{});
    launch(G, W, ic<1>{});
  };
  if (sh.gpw == 1)
    depth(ic<1>{}, ic<8>{}, ic<2>{});
  else if (sh.gpw == 2)
    depth(ic<2>{}, ic<8>{}, ic<2>{});
  else if (sh.waves <= 8)
    depth(ic<4>{}, ic<8>{}, ic<6>{});
  else
    depth(ic<4>{}, ic<16>{}, ic<MAXD16 < 2 ? MAXD16 : 2>{});
}

template <class L>
void dispatch_p(int P, L&& launch) {
  switch (P) {
    case 1: launch(ic<1>{}); break;
    case 2: launch(ic<2>{}); break;
    case 3: launch(ic<3>{}); break;
    case 4: launch(ic<4>{}); break;
    case 5: launch(ic<5>{}); break;
    default: launch(ic<6>{}); break;
  }
}

// Calls launch(ic<G>) for a group size of the sa* storage (64, 128 or 256).
template <class L>
void dispatch_group(int G, L&& launch) {
  switch (G) {
    case 64: launch(ic<64>{}); break;
    case 128: launch(ic<128>{}); break;
    default: launch(ic<256>{}); break;
  }
}

#define SVQ_KARGS(G, W, D) decltype(G)::value, decltype(W)::value, decltype(D)::value

// Deepest ring the sign-plane kernels keep in registers without spilling:
// a slot holds P sign dwords and P scale runs per group.  The sixteen-wave
// shapes (K above 4096) take MAXD16 (one slot).
constexpr int max_depth_planes(int P, int W) { return W > 8 ? 1 : P <= 4 ? 6 : P == 5 ? 5 : 4; }
// Template arguments of the sign-plane kernels for format F.
#define SVQ_KARGS_F(F, G, W, D)                                                                     \
  F, decltype(G)::value, decltype(W)::value,                                                       \
      (decltype(D)::value < max_depth_planes(F::P, decltype(W)::value)                            \
           ? decltype(D)::value                                                                     \
           : max_depth_planes(F::P, decltype(W)::value))

// The sa* kernels and the sign-plane mat-muls are instantiated with rings of
// at most three tiles (deeper rings would spill registers); the launch
// preferences above choose at most two, three stays reachable through
// SVQ_PIPE_DEPTH.
constexpr int kMaxDepthSa = 3;
constexpr int kMaxDepthPlanesGemm = 3;

// Argument checks of the sa* entry points; the rest as check_linear.
inline int check_sa(const char* fn, const void* packed, const void* x, const void* y, int32_t M, int64_t N,
                    int64_t K, int32_t G, int32_t P, int32_t max_m = SVQ_MAX_M) {
  svq::clear_error();
  if (G != 64 && G != 128 && G != 256)
    return svq::fail(SVQ_ERR_SHAPE, "%s: group size must be 64, 128 or 256 (got %d)", fn, G);
  if (K % 256) return svq::fail(SVQ_ERR_SHAPE, "%s: K=%lld must be a multiple of 256", fn, (long long)K);
  if (P < 2 || P > SVQ_MAX_P) return svq::fail(SVQ_ERR_SHAPE, "%s: P=%d must be in 2..6", fn, P);
  return check_linear(fn, packed, x, y, M, N, K, SVQ_GROUP, P, max_m);
}

// Argument checks shared by the head entry points (P = 0: INT4 weights;
// P >= 1: P sign planes).
// Argmax completion form for a head launch (see HeadOut::levels): two
// levels where every workgroup owns at most kArgmaxSplitMaxTiles row tiles
// (their completions arrive together), one level otherwise.  Measured on
// MI355X (K = 4096, 256 workgroups, medians of three interleaved rounds):
// two levels were 1-6% faster at 8 tiles a workgroup (N = 32768, W4A16 and
// sign-plane heads, M = 1 and 16) and 0.3-1.3% slower at 16, 32 and 61
// (N = 65536, 131072, 248320).  SVQ_ARGMAX_LEVELS = 1 or 2 overrides it (for
// tuning runs).
constexpr int kArgmaxSplitMaxTiles = 8;
inline HeadOut with_levels(HeadOut ho, const Shape& sh) {
  const int tmax = (sh.NT + sh.grid - 1) / sh.grid;
  ho.levels = env_int("SVQ_ARGMAX_LEVELS", 1, 2, tmax <= kArgmaxSplitMaxTiles ? 2 : 1);
  return ho;
}

// The head's arguments other than its workspace.
inline int check_head_args(const char* fn, const uint8_t* packed, const uint16_t* X, int32_t M, int64_t N, int64_t K,
                           int32_t G, int32_t P, const HeadOut& ho) {
  if (int rc = check_linear(fn, packed, X, ho.idx, M, N, K, G, P)) return rc;
  if (!ho.max) return svq::fail(SVQ_ERR_NULL, "%s: NULL maxlogit", fn);
  if (misaligned(ho.idx, 4) || misaligned(ho.max, 4) || (ho.row_ids && misaligned(ho.row_ids, 4)))
    return svq::fail(SVQ_ERR_ALIGN, "%s: argmax, maxlogit and row_ids must be 4-byte aligned", fn);
  return SVQ_OK;
}

inline int check_head(const char* fn, const uint8_t* packed, const uint16_t* X, int32_t M, int64_t N, int64_t K,
                      int32_t G, int32_t P, const HeadOut& ho, void* workspace, size_t workspace_bytes) {
  if (int rc = check_head_args(fn, packed, X, M, N, K, G, P, ho)) return rc;
  if (!workspace || workspace_bytes < svq_lmhead_workspace_bytes(M))
    return svq::fail(SVQ_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu)", fn, svq_lmhead_workspace_bytes(M),
                     workspace ? workspace_bytes : (size_t)0);
  if (misaligned(workspace, 16)) return svq::fail(SVQ_ERR_ALIGN, "%s: workspace must be 16-byte aligned", fn);
  return SVQ_OK;
}

}  // namespace
