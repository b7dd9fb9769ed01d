// svq.hip -- gfx950 (CDNA4) kernels behind the device entry points of svq.h.
//
// What is computed (see svq.h for the full statements and citations):
//   W4A16         y = sum_g s[n][g] * sum_{k in g} c[n][k] x[k]
//                 (Efficient Qwen Competition report, sec. 2.1 and 3.3)
//   binary planes y = sum_g sum_p alpha[p][n][g] * sum_{k in g} b[p][n][k] x[k]
//                 (ShiftAddQwen README, intro and "Method / Format")
//   greedy head   argmax over W4A16 logits, lowest index on ties
//                 (DFlash summary sec. 4.1; small-vocabulary MTP study sec. 3.3)
//
// Work decomposition shared by every kernel.  A workgroup owns one 16-row
// tile at a time (grid-stride over row tiles) and splits K across its waves:
// wave w owns groups [w*GPW, (w+1)*GPW).  A lane (q = lane/16, r = lane%16)
// of a tile owns row r and the k sub-ranges 32t + 8q + [0, 8), t = 0..3, of
// every group; the packed layout stores exactly that lane's data as one
// contiguous 16-byte (INT4) or 4P-byte (sign planes) chunk, so one wave load
// moves a whole 1 KiB INT4 tile.  The activations of the wave's K range stay
// in registers for the whole kernel; each tile's per-wave partial sums meet
// in LDS and one thread per output row finishes the sum.
//
// Exact operands.  A nibble u = c + 8 becomes the bf16 value 128 + u with one
// AND-OR (the high bits 0x43 form 2^7, the nibble fills the mantissa), so the
// dot products see 136 + c exactly; the group sum of x times 136 is taken
// back out before the group scale is applied in fp32.  A sign bit becomes the
// bf16 value +1 or -1 (0x3F80 with the sign bit set for b = -1) with one
// shift and one AND-OR.  Neither s*c nor sum_p alpha_p b_p is ever rounded to
// bf16; the scales are applied per group in fp32, and the output is rounded
// to bf16 once, to nearest even.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cfloat>
#include <climits>
#include <cstdint>
#include <cstdlib>

#include "svq.h"
#include "svq_internal.h"

namespace svq {
char* error_buffer() {
  static thread_local char buf[512];
  return buf;
}
}  // namespace svq

extern "C" const char* svq_last_error(void) { return svq::error_buffer(); }

namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

constexpr uint32_t kInt4Magic = 0x43004300u;  // bf16 pair (128, 128)
constexpr float kInt4Bias = 136.0f;           // 128 + 8: decoded value = 136 + c
constexpr uint32_t kOnePair = 0x3F803F80u;    // bf16 pair (1, 1)
constexpr int kMaxWaves = 16;
constexpr int kLmheadMaxWg = 1024;

struct ArgBest {
  float v;
  int idx;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         c, false);
}

// bf16 pair (136 + c_even, 136 + c_odd) for pair i (k = 2i, 2i+1) of a code dword.
__device__ __forceinline__ uint32_t int4_pair(uint32_t w, int i) {
  return ((w >> (4 * i)) & 0x000F000Fu) | kInt4Magic;
}

// bf16 pair (b_even, b_odd) in {-1, +1} for pair ip = 4t + i of a sign dword.
__device__ __forceinline__ uint32_t sign_pair(uint32_t w, int ip) {
  return ((w << (15 - ip)) & 0x80008000u) | kOnePair;
}

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint32_t* a, const uint32_t* b, f32x4_t c) {
  u32x4_t av = {a[0], a[1], a[2], a[3]};
  u32x4_t bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                 __builtin_bit_cast(bf16x8_t, bv), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Activation staging: lane (q, r) keeps the bf16 pairs of row `row` at
// k = 128g + 32t + 8q + [0, 8) for the wave's GPW groups: xp[gi][4t + i] is
// the pair (k, k+1), k = 128g + 32t + 8q + 2i.  Zero outside [0, KT) / rows.
template <int GPW>
__device__ __forceinline__ void load_x_pairs(const uint32_t* __restrict__ xrow, bool row_ok, int g0, int KT, int q,
                                             uint32_t (&xp)[GPW][16]) {
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = g0 + gi;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (row_ok && g < KT) v = *reinterpret_cast<const uint4*>(xrow + 64 * g + 16 * t + 4 * q);
      xp[gi][4 * t + 0] = v.x;
      xp[gi][4 * t + 1] = v.y;
      xp[gi][4 * t + 2] = v.z;
      xp[gi][4 * t + 3] = v.w;
    }
  }
}

// Sum of the 32 activations a lane holds for each of its groups.
template <int GPW>
__device__ __forceinline__ void lane_group_sums(const uint32_t (&xp)[GPW][16], float (&xs)[GPW]) {
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s = dot2(xp[gi][j], kOnePair, s);
    xs[gi] = s;
  }
}

// ---------------------------------------------------------------------------
// M = 1 mat-vec cores.  Each returns the lane's partial sum for row r over its
// k sub-ranges of the wave's groups.
template <int GPW>
__device__ __forceinline__ float w4a16_tile_partial(const uint4 (&c)[GPW], const uint16_t (&s)[GPW],
                                                    const uint32_t (&xp)[GPW][16], const float (&xs)[GPW]) {
  float part = 0.f;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const uint32_t w[4] = {c[gi].x, c[gi].y, c[gi].z, c[gi].w};
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = dot2(int4_pair(w[t], i), xp[gi][4 * t + i], acc);
    part = fmaf(bf16_to_f32(s[gi]), fmaf(-kInt4Bias, xs[gi], acc), part);
  }
  return part;
}

template <int GPW, int P>
__device__ __forceinline__ float binplane_tile_partial(const uint32_t (&w)[GPW][P], const uint16_t (&al)[GPW][P],
                                                       const uint32_t (&xp)[GPW][16]) {
  float part = 0.f;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float acc = 0.f;
#pragma unroll
      for (int ip = 0; ip < 16; ++ip) acc = dot2(sign_pair(w[gi][p], ip), xp[gi][ip], acc);
      part = fmaf(f16_to_f32(al[gi][p]), acc, part);
    }
  return part;
}

// ---------------------------------------------------------------------------
// Tile loaders (global -> registers).
template <int GPW>
__device__ __forceinline__ void load_int4_tile(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                               int rt, int g0, int KT, int lane, int r, uint4 (&c)[GPW],
                                               uint16_t (&s)[GPW]) {
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = g0 + gi;
    if (g < KT) {
      c[gi] = *reinterpret_cast<const uint4*>(codes + ((size_t)rt * KT + g) * 1024 + 16 * lane);
      s[gi] = scales[(size_t)(16 * rt + r) * KT + g];
    } else {
      c[gi] = make_uint4(0u, 0u, 0u, 0u);
      s[gi] = 0;
    }
  }
}

template <int GPW, int P>
__device__ __forceinline__ void load_sign_tile(const uint8_t* __restrict__ bits, const uint16_t* __restrict__ alpha,
                                               int rt, int g0, int KT, int N16, int lane, int r,
                                               uint32_t (&w)[GPW][P], uint16_t (&al)[GPW][P]) {
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = g0 + gi;
    const uint32_t* src =
        reinterpret_cast<const uint32_t*>(bits + ((size_t)rt * KT + g) * 256 * P + 4 * P * lane);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (g < KT) {
        w[gi][p] = src[p];
        al[gi][p] = alpha[((size_t)p * N16 + 16 * rt + r) * KT + g];
      } else {
        w[gi][p] = 0u;
        al[gi][p] = 0;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// gemv_w4a16 / lmhead (M = 1).  ARGMAX selects the epilogue.
template <int GPW, int MAXW, bool ARGMAX>
__global__ void __launch_bounds__(64 * MAXW)
    k_gemv_w4a16(const uint8_t* __restrict__ blob, const uint32_t* __restrict__ xw, uint16_t* __restrict__ y,
                 ArgBest* __restrict__ ws, int N, int KT, int NT) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int g0 = wave * GPW;
  const uint8_t* codes = blob;
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(blob + (size_t)NT * KT * 1024);

  uint32_t xp[GPW][16];
  float xs[GPW];
  load_x_pairs<GPW>(xw, true, g0, KT, q, xp);
  lane_group_sums<GPW>(xp, xs);

  __shared__ float red[2][kMaxWaves][16];
  float best_v = -FLT_MAX;
  int best_i = INT_MAX;

  uint4 cur[GPW], nxt[GPW];
  uint16_t scur[GPW], snxt[GPW];
  int rt = blockIdx.x;
  if (rt < NT) load_int4_tile<GPW>(codes, scales, rt, g0, KT, lane, r, cur, scur);
  for (int it = 0; rt < NT; rt += gridDim.x, ++it) {
    const int rn = rt + gridDim.x;
    if (rn < NT) load_int4_tile<GPW>(codes, scales, rn, g0, KT, lane, r, nxt, snxt);
    float part = w4a16_tile_partial<GPW>(cur, scur, xp, xs);
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    if (q == 0) red[it & 1][wave][r] = part;
    __syncthreads();
    if (threadIdx.x < 16) {
      float v = 0.f;
      for (int w2 = 0; w2 < nwaves; ++w2) v += red[it & 1][w2][threadIdx.x];
      const int n = 16 * rt + threadIdx.x;
      if (n < N) {
        if constexpr (ARGMAX) {
          if (v > best_v) {  // rows arrive in increasing n per thread
            best_v = v;
            best_i = n;
          }
        } else {
          y[n] = f32_to_bf16_rne(v);
        }
      }
    }
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      cur[gi] = nxt[gi];
      scur[gi] = snxt[gi];
    }
  }
  if constexpr (ARGMAX) {
    if (threadIdx.x < 64) {
      for (int off = 8; off > 0; off >>= 1) {
        const float ov = __shfl_xor(best_v, off);
        const int oi = __shfl_xor(best_i, off);
        if (better(ov, oi, best_v, best_i)) {
          best_v = ov;
          best_i = oi;
        }
      }
      if (threadIdx.x == 0) ws[blockIdx.x] = ArgBest{best_v, best_i};
    }
  }
}

// gemv_binplane (M = 1).
template <int GPW, int MAXW, int P>
__global__ void __launch_bounds__(64 * MAXW)
    k_gemv_binplane(const uint8_t* __restrict__ blob, const uint32_t* __restrict__ xw, uint16_t* __restrict__ y,
                    int N, int KT, int NT) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int g0 = wave * GPW;
  const int N16 = NT * 16;
  const uint8_t* bits = blob;
  const uint16_t* alpha = reinterpret_cast<const uint16_t*>(blob + (size_t)NT * KT * 256 * P);

  uint32_t xp[GPW][16];
  load_x_pairs<GPW>(xw, true, g0, KT, q, xp);

  __shared__ float red[2][kMaxWaves][16];
  uint32_t cur[GPW][P], nxt[GPW][P];
  uint16_t acur[GPW][P], anxt[GPW][P];
  int rt = blockIdx.x;
  if (rt < NT) load_sign_tile<GPW, P>(bits, alpha, rt, g0, KT, N16, lane, r, cur, acur);
  for (int it = 0; rt < NT; rt += gridDim.x, ++it) {
    const int rn = rt + gridDim.x;
    if (rn < NT) load_sign_tile<GPW, P>(bits, alpha, rn, g0, KT, N16, lane, r, nxt, anxt);
    float part = binplane_tile_partial<GPW, P>(cur, acur, xp);
    part += __shfl_xor(part, 16);
    part += __shfl_xor(part, 32);
    if (q == 0) red[it & 1][wave][r] = part;
    __syncthreads();
    if (threadIdx.x < 16) {
      float v = 0.f;
      for (int w2 = 0; w2 < nwaves; ++w2) v += red[it & 1][w2][threadIdx.x];
      const int n = 16 * rt + threadIdx.x;
      if (n < N) y[n] = f32_to_bf16_rne(v);
    }
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        cur[gi][p] = nxt[gi][p];
        acur[gi][p] = anxt[gi][p];
      }
  }
}

// ---------------------------------------------------------------------------
// M <= 16 verify kernels on v_mfma_f32_16x16x32_bf16.  Per 32-wide k block t,
// A = X[m = r][k = 32t + 8q + 0..7] (lane q, r) and B = W^T[k][n = r] from the
// tile's dword t; D lands as D[m = 4q + i][n = r], i = 0..3.

// Group sums of X per (row m, group g) into LDS, computed by the owning wave.
template <int GPW>
__device__ __forceinline__ void x_group_sums_to_lds(const uint32_t (&xa)[GPW][16], int g0, int KT, int q, int r,
                                                    float (*xs_sh)[65]) {
  float xs[GPW];
  lane_group_sums<GPW>(xa, xs);
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    float s = xs[gi];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (q == 0 && g0 + gi < KT) xs_sh[r][g0 + gi] = s;
  }
}

// Per-tile epilogue: the WG's waves' 16x16 partials meet in LDS.  Thread
// tid < 256 owns (m = tid/16, n = tid%16) and returns the finished sum.
__device__ __forceinline__ float reduce_tile_16x16(float (*red)[256], const float (&yv)[4], int wave, int nwaves,
                                                   int q, int r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][(4 * q + i) * 16 + r] = yv[i];
  __syncthreads();
  float v = 0.f;
  if (threadIdx.x < 256)
    for (int w2 = 0; w2 < nwaves; ++w2) v += red[w2][threadIdx.x];
  return v;
}

template <int GPW, int MAXW, bool ARGMAX>
__global__ void __launch_bounds__(64 * MAXW)
    k_gemm_w4a16(const uint8_t* __restrict__ blob, const uint32_t* __restrict__ Xw, uint16_t* __restrict__ Y,
                 ArgBest* __restrict__ ws, int M, int N, int KT, int NT) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int g0 = wave * GPW;
  const uint8_t* codes = blob;
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(blob + (size_t)NT * KT * 1024);

  __shared__ float xs_sh[16][65];
  __shared__ float red[2][kMaxWaves][256];

  uint32_t xa[GPW][16];
  load_x_pairs<GPW>(Xw + (size_t)r * KT * 64, r < M, g0, KT, q, xa);
  // Every (row, group) entry read below is written by the wave owning the group.
  x_group_sums_to_lds<GPW>(xa, g0, KT, q, r, xs_sh);
  __syncthreads();
  float xsv[GPW][4];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
    for (int i = 0; i < 4; ++i) xsv[gi][i] = g0 + gi < KT ? xs_sh[4 * q + i][g0 + gi] : 0.f;

  float best_v = -FLT_MAX;
  int best_i = INT_MAX;
  const int mo = threadIdx.x >> 4, no = threadIdx.x & 15;  // output owned by this thread (tid < 256)

  uint4 cur[GPW], nxt[GPW];
  uint16_t scur[GPW], snxt[GPW];
  int rt = blockIdx.x;
  if (rt < NT) load_int4_tile<GPW>(codes, scales, rt, g0, KT, lane, r, cur, scur);
  for (int it = 0; rt < NT; rt += gridDim.x, ++it) {
    const int rn = rt + gridDim.x;
    if (rn < NT) load_int4_tile<GPW>(codes, scales, rn, g0, KT, lane, r, nxt, snxt);
    float yv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      const uint32_t w[4] = {cur[gi].x, cur[gi].y, cur[gi].z, cur[gi].w};
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t b[4] = {int4_pair(w[t], 0), int4_pair(w[t], 1), int4_pair(w[t], 2), int4_pair(w[t], 3)};
        c = mfma16x16x32(&xa[gi][4 * t], b, c);
      }
      const float s = bf16_to_f32(scur[gi]);
#pragma unroll
      for (int i = 0; i < 4; ++i) yv[i] = fmaf(s, fmaf(-kInt4Bias, xsv[gi][i], c[i]), yv[i]);
    }
    const float v = reduce_tile_16x16(red[it & 1], yv, wave, nwaves, q, r);
    const int n = 16 * rt + no;
    if (threadIdx.x < 256 && mo < M && n < N) {
      if constexpr (ARGMAX) {
        if (v > best_v) {
          best_v = v;
          best_i = n;
        }
      } else {
        Y[(size_t)mo * N + n] = f32_to_bf16_rne(v);
      }
    }
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) {
      cur[gi] = nxt[gi];
      scur[gi] = snxt[gi];
    }
  }
  if constexpr (ARGMAX) {
    if (threadIdx.x < 256) {
      for (int off = 8; off > 0; off >>= 1) {
        const float ov = __shfl_xor(best_v, off);
        const int oi = __shfl_xor(best_i, off);
        if (better(ov, oi, best_v, best_i)) {
          best_v = ov;
          best_i = oi;
        }
      }
      if (no == 0 && mo < M) ws[(size_t)mo * gridDim.x + blockIdx.x] = ArgBest{best_v, best_i};
    }
  }
}

template <int GPW, int MAXW, int P>
__global__ void __launch_bounds__(64 * MAXW)
    k_gemm_binplane(const uint8_t* __restrict__ blob, const uint32_t* __restrict__ Xw, uint16_t* __restrict__ Y,
                    int M, int N, int KT, int NT) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int g0 = wave * GPW;
  const int N16 = NT * 16;
  const uint8_t* bits = blob;
  const uint16_t* alpha = reinterpret_cast<const uint16_t*>(blob + (size_t)NT * KT * 256 * P);

  __shared__ float red[2][kMaxWaves][256];
  uint32_t xa[GPW][16];
  load_x_pairs<GPW>(Xw + (size_t)r * KT * 64, r < M, g0, KT, q, xa);
  const int mo = threadIdx.x >> 4, no = threadIdx.x & 15;

  uint32_t cur[GPW][P], nxt[GPW][P];
  uint16_t acur[GPW][P], anxt[GPW][P];
  int rt = blockIdx.x;
  if (rt < NT) load_sign_tile<GPW, P>(bits, alpha, rt, g0, KT, N16, lane, r, cur, acur);
  for (int it = 0; rt < NT; rt += gridDim.x, ++it) {
    const int rn = rt + gridDim.x;
    if (rn < NT) load_sign_tile<GPW, P>(bits, alpha, rn, g0, KT, N16, lane, r, nxt, anxt);
    float yv[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t b[4] = {sign_pair(cur[gi][p], 4 * t + 0), sign_pair(cur[gi][p], 4 * t + 1),
                                 sign_pair(cur[gi][p], 4 * t + 2), sign_pair(cur[gi][p], 4 * t + 3)};
          c = mfma16x16x32(&xa[gi][4 * t], b, c);
        }
        const float a = f16_to_f32(acur[gi][p]);
#pragma unroll
        for (int i = 0; i < 4; ++i) yv[i] = fmaf(a, c[i], yv[i]);
      }
    const float v = reduce_tile_16x16(red[it & 1], yv, wave, nwaves, q, r);
    const int n = 16 * rt + no;
    if (threadIdx.x < 256 && mo < M && n < N) Y[(size_t)mo * N + n] = f32_to_bf16_rne(v);
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        cur[gi][p] = nxt[gi][p];
        acur[gi][p] = anxt[gi][p];
      }
  }
}

// Combine the per-workgroup bests of lmhead_argmax: block m reduces row m.
__global__ void __launch_bounds__(256)
    k_argmax_finalize(const ArgBest* __restrict__ ws, int nwg, int N, const int32_t* __restrict__ row_ids,
                      int32_t* __restrict__ out_idx, float* __restrict__ out_max) {
  const int m = blockIdx.x;
  float bv = -FLT_MAX;
  int bi = INT_MAX;
  for (int j = threadIdx.x; j < nwg; j += blockDim.x) {
    const ArgBest e = ws[(size_t)m * nwg + j];
    if (better(e.v, e.idx, bv, bi)) {
      bv = e.v;
      bi = e.idx;
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  __shared__ ArgBest part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ArgBest{bv, bi};
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w)
      if (better(part[w].v, part[w].idx, bv, bi)) {
        bv = part[w].v;
        bi = part[w].idx;
      }
    // No row compared greater than -FLT_MAX only if every logit was NaN.
    const bool found = bi >= 0 && bi < N;
    out_idx[m] = !found ? -1 : row_ids ? row_ids[bi] : bi;
    out_max[m] = found ? bv : __builtin_nanf("");
  }
}

// Streaming-read ceiling: 16-byte loads over `n16` chunks, one checksum per WG.
__global__ void __launch_bounds__(256) k_stream_read(const uint4* __restrict__ src, size_t n16,
                                                     uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// ---------------------------------------------------------------------------
// Host side: validation, launch shapes, dispatch.

std::atomic<int> g_cus[64];

int device_cus(int* cus) {
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

int wgs_per_cu() {
  static const int v = [] {
    const char* s = std::getenv("SVQ_WG_PER_CU");
    const int x = s ? std::atoi(s) : 0;
    return x >= 1 && x <= 8 ? x : 2;
  }();
  return v;
}

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

int check_linear(const char* fn, const void* packed, const void* x, const void* y, int32_t M, int64_t N, int64_t K,
                 int32_t G, int32_t P) {
  svq::clear_error();
  if (!packed || !x || !y) return svq::fail(SVQ_ERR_NULL, "%s: NULL pointer", fn);
  if (N < 1 || N > (int64_t)INT_MAX - 16) return svq::fail(SVQ_ERR_SHAPE, "%s: N=%lld out of range", fn, (long long)N);
  if (G != SVQ_GROUP) return svq::fail(SVQ_ERR_SHAPE, "%s: group size must be 128 (got %d)", fn, G);
  if (K < SVQ_GROUP || K % SVQ_GROUP || K > SVQ_MAX_K)
    return svq::fail(SVQ_ERR_SHAPE, "%s: K=%lld must be a multiple of 128 in [128, %d]", fn, (long long)K, SVQ_MAX_K);
  if (M < 1 || M > SVQ_MAX_M) return svq::fail(SVQ_ERR_SHAPE, "%s: M=%d must be in 1..16", fn, M);
  if (P != 0 && (P < 1 || P > SVQ_MAX_P)) return svq::fail(SVQ_ERR_SHAPE, "%s: P=%d must be in 1..6", fn, P);
  if (misaligned(packed, 16)) return svq::fail(SVQ_ERR_ALIGN, "%s: packed weights must be 16-byte aligned", fn);
  if (misaligned(x, 16)) return svq::fail(SVQ_ERR_ALIGN, "%s: activations must be 16-byte aligned", fn);
  if (misaligned(y, 2)) return svq::fail(SVQ_ERR_ALIGN, "%s: output must be 2-byte aligned", fn);
  return SVQ_OK;
}

struct Shape {
  int KT, NT, gpw, waves, grid;
};

// min_waves: the M <= 16 kernels finish a 16x16 output tile with 256
// threads, so their workgroups always carry at least four waves.
int plan(int64_t N, int64_t K, int min_waves, Shape* s) {
  int cus = 0;
  if (int rc = device_cus(&cus)) return rc;
  s->KT = (int)(K / 128);
  s->NT = (int)((N + 15) / 16);
  s->gpw = s->KT <= 8 ? 1 : s->KT <= 16 ? 2 : 4;
  s->waves = (s->KT + s->gpw - 1) / s->gpw;
  if (s->waves < min_waves) s->waves = min_waves;
  const int want = cus * wgs_per_cu();
  s->grid = s->NT < want ? s->NT : want;
  return SVQ_OK;
}

int launched(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return svq::fail(SVQ_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return SVQ_OK;
}

#define SVQ_DISPATCH_GPW(sh, BODY)                         \
  do {                                                     \
    if ((sh).gpw == 1) {                                   \
      constexpr int GPW = 1, MAXW = 8;                     \
      BODY;                                                \
    } else if ((sh).gpw == 2) {                            \
      constexpr int GPW = 2, MAXW = 8;                     \
      BODY;                                                \
    } else if ((sh).waves <= 8) {                          \
      constexpr int GPW = 4, MAXW = 8;                     \
      BODY;                                                \
    } else {                                               \
      constexpr int GPW = 4, MAXW = 16;                    \
      BODY;                                                \
    }                                                      \
  } while (0)

#define SVQ_DISPATCH_P(Pv, BODY)        \
  switch (Pv) {                         \
    case 1: { constexpr int P = 1; BODY; } break; \
    case 2: { constexpr int P = 2; BODY; } break; \
    case 3: { constexpr int P = 3; BODY; } break; \
    case 4: { constexpr int P = 4; BODY; } break; \
    case 5: { constexpr int P = 5; BODY; } break; \
    default: { constexpr int P = 6; BODY; } break; \
  }

}  // namespace

extern "C" {

size_t svq_lmhead_workspace_bytes(int32_t M) {
  if (M < 1 || M > SVQ_MAX_M) return 0;
  return (size_t)kLmheadMaxWg * (size_t)M * sizeof(ArgBest);
}

int gemv_w4a16(const uint8_t* packed, const uint16_t* x, uint16_t* y, int64_t N, int64_t K, int32_t G,
               void* stream) {
  if (int rc = check_linear("gemv_w4a16", packed, x, y, 1, N, K, G, 0)) return rc;
  Shape sh;
  if (int rc = plan(N, K, 1, &sh)) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint32_t* xw = reinterpret_cast<const uint32_t*>(x);
  SVQ_DISPATCH_GPW(sh, hipLaunchKernelGGL((k_gemv_w4a16<GPW, MAXW, false>), dim3(sh.grid), dim3(64 * sh.waves), 0,
                                          st, packed, xw, y, (ArgBest*)nullptr, (int)N, sh.KT, sh.NT));
  return launched("gemv_w4a16");
}

int gemv_binplane(const uint8_t* packed, const uint16_t* x, uint16_t* y, int64_t N, int64_t K, int32_t G, int32_t P,
                  void* stream) {
  if (P == 0) return svq::fail(SVQ_ERR_SHAPE, "gemv_binplane: P=0 must be in 1..6");
  if (int rc = check_linear("gemv_binplane", packed, x, y, 1, N, K, G, P)) return rc;
  Shape sh;
  if (int rc = plan(N, K, 1, &sh)) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint32_t* xw = reinterpret_cast<const uint32_t*>(x);
  SVQ_DISPATCH_P(P, SVQ_DISPATCH_GPW(sh, hipLaunchKernelGGL((k_gemv_binplane<GPW, MAXW, P>), dim3(sh.grid),
                                                            dim3(64 * sh.waves), 0, st, packed, xw, y, (int)N,
                                                            sh.KT, sh.NT)));
  return launched("gemv_binplane");
}

int gemm_smallm_w4a16(const uint8_t* packed, const uint16_t* X, uint16_t* Y, int32_t M, int64_t N, int64_t K,
                      int32_t G, void* stream) {
  if (int rc = check_linear("gemm_smallm_w4a16", packed, X, Y, M, N, K, G, 0)) return rc;
  Shape sh;
  if (int rc = plan(N, K, 4, &sh)) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint32_t* Xw = reinterpret_cast<const uint32_t*>(X);
  SVQ_DISPATCH_GPW(sh, hipLaunchKernelGGL((k_gemm_w4a16<GPW, MAXW, false>), dim3(sh.grid), dim3(64 * sh.waves), 0,
                                          st, packed, Xw, Y, (ArgBest*)nullptr, M, (int)N, sh.KT, sh.NT));
  return launched("gemm_smallm_w4a16");
}

int gemm_smallm_binplane(const uint8_t* packed, const uint16_t* X, uint16_t* Y, int32_t M, int64_t N, int64_t K,
                         int32_t G, int32_t P, void* stream) {
  if (P == 0) return svq::fail(SVQ_ERR_SHAPE, "gemm_smallm_binplane: P=0 must be in 1..6");
  if (int rc = check_linear("gemm_smallm_binplane", packed, X, Y, M, N, K, G, P)) return rc;
  Shape sh;
  if (int rc = plan(N, K, 4, &sh)) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint32_t* Xw = reinterpret_cast<const uint32_t*>(X);
  SVQ_DISPATCH_P(P, SVQ_DISPATCH_GPW(sh, hipLaunchKernelGGL((k_gemm_binplane<GPW, MAXW, P>), dim3(sh.grid),
                                                            dim3(64 * sh.waves), 0, st, packed, Xw, Y, M, (int)N,
                                                            sh.KT, sh.NT)));
  return launched("gemm_smallm_binplane");
}

int lmhead_argmax(const uint8_t* packed, const uint16_t* X, int32_t M, int64_t N, int64_t K, int32_t G,
                  const int32_t* row_ids, int32_t* argmax, float* maxlogit, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (int rc = check_linear("lmhead_argmax", packed, X, argmax, M, N, K, G, 0)) return rc;
  if (!maxlogit) return svq::fail(SVQ_ERR_NULL, "lmhead_argmax: NULL maxlogit");
  if (misaligned(argmax, 4) || misaligned(maxlogit, 4) || (row_ids && misaligned(row_ids, 4)))
    return svq::fail(SVQ_ERR_ALIGN, "lmhead_argmax: argmax, maxlogit and row_ids must be 4-byte aligned");
  if (!workspace || workspace_bytes < svq_lmhead_workspace_bytes(M))
    return svq::fail(SVQ_ERR_WORKSPACE, "lmhead_argmax: workspace needs %zu bytes (got %zu)",
                     svq_lmhead_workspace_bytes(M), workspace ? workspace_bytes : (size_t)0);
  if (misaligned(workspace, 16)) return svq::fail(SVQ_ERR_ALIGN, "lmhead_argmax: workspace must be 16-byte aligned");
  Shape sh;
  if (int rc = plan(N, K, M == 1 ? 1 : 4, &sh)) return rc;
  if (sh.grid > kLmheadMaxWg) sh.grid = kLmheadMaxWg;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint32_t* Xw = reinterpret_cast<const uint32_t*>(X);
  ArgBest* ws = reinterpret_cast<ArgBest*>(workspace);
  if (M == 1) {
    SVQ_DISPATCH_GPW(sh, hipLaunchKernelGGL((k_gemv_w4a16<GPW, MAXW, true>), dim3(sh.grid), dim3(64 * sh.waves), 0,
                                            st, packed, Xw, (uint16_t*)nullptr, ws, (int)N, sh.KT, sh.NT));
  } else {
    SVQ_DISPATCH_GPW(sh, hipLaunchKernelGGL((k_gemm_w4a16<GPW, MAXW, true>), dim3(sh.grid), dim3(64 * sh.waves), 0,
                                            st, packed, Xw, (uint16_t*)nullptr, ws, M, (int)N, sh.KT, sh.NT));
  }
  if (int rc = launched("lmhead_argmax")) return rc;
  hipLaunchKernelGGL(k_argmax_finalize, dim3(M), dim3(256), 0, st, ws, sh.grid, (int)N, row_ids, argmax, maxlogit);
  return launched("lmhead_argmax(finalize)");
}

int svq_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  svq::clear_error();
  if (!src || !sink) return svq::fail(SVQ_ERR_NULL, "svq_stream_read: NULL pointer");
  if (bytes == 0 || bytes % 16) return svq::fail(SVQ_ERR_SHAPE, "svq_stream_read: bytes must be a positive multiple of 16");
  if (misaligned(src, 16) || misaligned(sink, 4)) return svq::fail(SVQ_ERR_ALIGN, "svq_stream_read: misaligned pointer");
  int cus = 0;
  if (int rc = device_cus(&cus)) return rc;
  int grid = cus * 8;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(k_stream_read, dim3(grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const uint4*>(src), bytes / 16, sink);
  return launched("svq_stream_read");
}

}  // extern "C"
