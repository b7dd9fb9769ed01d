// mmq_planes.h -- gfx950 mat-mul for blocks of 16 < M <= 64 activation rows
// over sign-plane weights: the fp16-alpha binary-plane blob and the sa*
// blob (u8 scale codes per plane and group, one fp16 d per 256-weight
// super-block).
//   Y[m][n] = sum_g sum_p alpha[p][n][g] * sum_{k in g} b[p][n][k] * X[m][k]
//   (ShiftAddQwen README, intro and "Method / Format"; the README places
//   batches below 64 in its quantized mat-mul regime)
// Blocks at K <= 4096 run on the M <= 16 kernel instead (see mmq.h); this
// kernel serves K above 4096.
//
// The decomposition is the W4A16 streaming kernel's (mmq.h): a workgroup owns
// R consecutive 16-row weight tiles (a block) at a time, its 8 waves split K,
// and a step of a wave covers one 128-wide column tile for the block's R row
// tiles and all MT 16-row m-tiles of X.  What differs is the weight side,
// which costs far more instructions per byte: every sign dword is decoded
// once per step into MFMA operands (one AND-OR per bf16 pair, see
// plane_operands in kernels.h) and each decoded operand feeds the MFMAs of
// all MT m-tiles, so a block of 64 rows decodes its weights once instead of
// four times (once per 16-row pass of the M <= 16 kernel) and reads them once.
//
// Exact operands.  A decoded operand is c + 2 bit with c a power of two fixed
// per k position (or the plain +-1 at two positions whose activations enter
// negated), so every product is exact in fp32.  A plane's chain starts at
// -Z, Z = sum_k (1 + c_k) X[m][k] over the column tile, and ends at minus the
// plane's signed sum; Z is itself an MFMA chain of X against the constant
// operand (1 + c_k), formed once per step and m-tile and shared by every row
// tile and plane (over each half of the tile for sa* at G = 64, whose halves
// carry their own codes).
//
// Data movement per step.  The A fragments of all MT m-tiles are read from
// the wave's LDS buffer at the start of the step; the buffer is then free,
// and the next step's X arrives through registers in two halves of at most
// two m-tiles, the first stored after the first half of the step's
// computation and the second at its end, so each half's load latency is
// covered by computation.  Weight tiles run in a ring D - 1 steps ahead.
#pragma once

#include "kernels.h"
#include "launch.h"
#include "mmq.h"

namespace {

// fp16-alpha binary planes.
template <int P_>
struct MmqPlanes {
  static constexpr int P = P_;
  static constexpr bool kHalves = false;
  using View = BlobView;
  template <int R>
  struct Slot {
    uint32_t w[R][P];  // the lane's sign dword of each (row tile, plane)
    uint32_t s[R][P];  // fp16 alpha of (plane, row 16 rt + r, this column tile) in the low half
  };
  static __device__ __forceinline__ View view(const uint8_t* blob, int KT, int NT) {
    return sign_view(blob, KT, NT, P);
  }
  template <int R>
  static __device__ __forceinline__ void load(Slot<R>& sl, const View& b, uint32_t tile0, uint32_t g, uint32_t oob,
                                              int lane, int r) {
    const uint32_t N16 = (uint32_t)b.NT * 16u;
#pragma unroll
    for (int rt = 0; rt < R; ++rt) {
      const uint32_t tile = tile0 + rt;
      const uint32_t off = (tile * (uint32_t)b.KT + g) * 256u * P + 4u * lane;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        sl.w[rt][p] = ld_stream4(b.w, (off + 256u * p) | oob);
        const uint32_t aoff = (((uint32_t)p * N16 + 16u * tile + r) * (uint32_t)b.KT4 + g) * 2u;
        sl.s[rt][p] = __builtin_amdgcn_raw_buffer_load_b16(b.s, aoff | oob, 0, 0);
      }
    }
  }
  // Row tile rt, plane p: MT chains from -Z, weighted by alpha.
  template <int R, int MT>
  static __device__ __forceinline__ void pair(const Slot<R>& sl, int rt, int p, const uint32_t (&a)[MT][4][4],
                                              const f32x4_t (&nz)[MT][2], const PlaneDecode& d,
                                              f32x4_t (&acc)[R][MT]) {
    const PlaneViews v = plane_views(sl.w[rt][p]);
    f32x4_t c[MT];
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) c[mi] = nz[mi][0];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t bq[4];
      plane_operands_t(v, t, d, bq);
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) c[mi] = mfma16x16x32(a[mi][t], bq, c[mi]);
    }
    const float al = f16_to_f32((uint16_t)sl.s[rt][p]);
#pragma unroll
    for (int mi = 0; mi < MT; ++mi)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[rt][mi][e] = fmaf(al, c[mi][e], acc[rt][mi][e]);
  }
};

// sa*: u8 codes per (plane, row, group of G) and one fp16 d per (row,
// 256-weight super-block); a column tile is half a super-block.
template <int P_, int G>
struct MmqSa {
  static constexpr int P = P_;
  static constexpr bool kHalves = G == 64;
  using View = SaView;
  template <int R>
  struct Slot {
    uint32_t w[R][P];  // sign dwords
    uint32_t a[R][P];  // the tile's code (G = 64: its two codes, first in the low byte)
    uint32_t d[R];     // fp16 d of the super-block holding the tile, low half
  };
  static __device__ __forceinline__ View view(const uint8_t* blob, int KT, int NT) {
    return sa_view<G>(blob, KT, NT, P);
  }
  template <int R>
  static __device__ __forceinline__ void load(Slot<R>& sl, const View& b, uint32_t tile0, uint32_t g, uint32_t oob,
                                              int lane, int r) {
    const uint32_t N16 = (uint32_t)b.NT * 16u;
    const uint32_t CG = (uint32_t)b.KT4 * 128u / G;
#pragma unroll
    for (int rt = 0; rt < R; ++rt) {
      const uint32_t tile = tile0 + rt, row = 16u * tile + r;
      const uint32_t off = (tile * (uint32_t)b.KT + g) * 256u * P + 4u * lane;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        sl.w[rt][p] = ld_stream4(b.w, (off + 256u * p) | oob);
        const uint32_t coff = ((uint32_t)p * N16 + row) * CG + (G == 64 ? 2u * g : G == 128 ? g : g >> 1);
        if constexpr (G == 64)
          sl.a[rt][p] = __builtin_amdgcn_raw_buffer_load_b16(b.a, coff | oob, 0, 0);
        else
          sl.a[rt][p] = __builtin_amdgcn_raw_buffer_load_b8(b.a, coff | oob, 0, 0);
      }
      sl.d[rt] = __builtin_amdgcn_raw_buffer_load_b16(b.d, ((row * ((uint32_t)b.KT4 / 2u) + (g >> 1)) * 2u) | oob, 0, 0);
    }
  }
  // Row tile rt, plane p: chains from -Z (per half at G = 64), each weighted
  // by its alpha = d * a (exact in fp32: an fp16 significand times 8 bits).
  template <int R, int MT>
  static __device__ __forceinline__ void pair(const Slot<R>& sl, int rt, int p, const uint32_t (&a)[MT][4][4],
                                              const f32x4_t (&nz)[MT][2], const PlaneDecode& d,
                                              f32x4_t (&acc)[R][MT]) {
    const PlaneViews v = plane_views(sl.w[rt][p]);
    const float dd = f16_to_f32((uint16_t)sl.d[rt]);
#pragma unroll
    for (int h = 0; h < (kHalves ? 2 : 1); ++h) {
      f32x4_t c[MT];
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) c[mi] = nz[mi][h];
#pragma unroll
      for (int t = kHalves ? 2 * h : 0; t < (kHalves ? 2 * h + 2 : 4); ++t) {
        uint32_t bq[4];
        plane_operands_t(v, t, d, bq);
#pragma unroll
        for (int mi = 0; mi < MT; ++mi) c[mi] = mfma16x16x32(a[mi][t], bq, c[mi]);
      }
      const float al = dd * (float)((sl.a[rt][p] >> (8 * h)) & 0xFFu);
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[rt][mi][e] = fmaf(al, c[mi][e], acc[rt][mi][e]);
    }
  }
};

template <class F, int MT, int R, int D>
__global__ void __launch_bounds__(64 * kMmqWaves)
    k_gemm_mmq_planes(const uint8_t* __restrict__ blob, const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                      int M, int N, int K, int KT, int NT) {
  // m-tiles of the first and second half of the next step's X.
  constexpr int H0 = MT < 2 ? MT : 2;
  constexpr int H1 = MT - H0;
  // The ring's next slot is refilled at the start of a step, so a ring of one
  // slot would overwrite the step's own weights.
  static_assert(D >= 2, "the weight ring needs two slots");
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int q = lane >> 4, r = lane & 15;
  const typename F::View bv = F::view(blob, KT, NT);
  // Rows >= M lie past the end of this range and read zero.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
  const int NB = (NT + R - 1) / R;
  const int CK = (KT + kMmqWaves - 1) / kMmqWaves;
  const int T = ((NB - 1 - (int)blockIdx.x) / (int)gridDim.x + 1) * CK;  // steps of every wave

  __shared__ uint4 xbuf[kMmqWaves][MT * 16 * 16];
  __shared__ float4 red[kMmqWaves][MT][64];
  char* xb = reinterpret_cast<char*>(xbuf[wave]);

  const uint32_t xlane = ((uint32_t)(lane >> 4) * (uint32_t)K + 8u * (lane & 15)) * 2u;
  const uint32_t xrow4 = 4u * (uint32_t)K * 2u;

  // Step order and cursors as in the W4A16 streaming kernel: the block's
  // column tiles w * CK + (c + blockIdx.x) % CK, X one step ahead, weights
  // D - 1 steps ahead.
  struct Cursor {
    int blk, c, rot, i;
  };
  auto advance = [&](Cursor& u) {
    ++u.i;
    u.rot = u.rot + 1 == CK ? 0 : u.rot + 1;
    if (++u.c == CK) {
      u.c = 0;
      u.blk += (int)gridDim.x;
    }
  };
  auto col = [&](const Cursor& u) { return wave * CK + u.rot; };
  auto step_oob = [&](const Cursor& u) { return oob_bit(u.i < T && col(u) < KT); };
  auto load_x = [&](const Cursor& u, int mt0, int nm, uint4 (&xh)[H0][4]) {
    const uint32_t uni = (256u * (uint32_t)col(u)) | step_oob(u);
#pragma unroll
    for (int h = 0; h < H0; ++h)
      if (h < nm)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t off = xlane + (uint32_t)(mt0 + h) * 4u * xrow4 + (uint32_t)v * xrow4;
          const v4u_t t = __builtin_amdgcn_raw_buffer_load_b128(xr, off + uni, 0, 0);
          xh[h][v] = make_uint4(t.x, t.y, t.z, t.w);
        }
  };
  auto store_x = [&](int mt0, int nm, const uint4 (&xh)[H0][4]) {
#pragma unroll
    for (int h = 0; h < H0; ++h)
      if (h < nm)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          *reinterpret_cast<uint4*>(xb + xrow_chunk(16 * (mt0 + h) + 4 * v + (lane >> 4), lane & 15)) = xh[h][v];
  };
  auto load_w = [&](const Cursor& u, typename F::template Slot<R>& w) {
    F::template load<R>(w, bv, (uint32_t)(R * u.blk), (uint32_t)col(u), step_oob(u), lane, r);
  };

  Cursor xc{(int)blockIdx.x, 0, (int)blockIdx.x % CK, 0};
  Cursor wc = xc;
  uint4 xh[H0][4];
  // Prologue: step 0's X into LDS, the first D - 1 steps' weights in flight.
  load_x(xc, 0, H0, xh);
  uint4 xh1[H1 > 0 ? H0 : 1][4];
  if constexpr (H1 > 0) load_x(xc, H0, H1, xh1);
  typename F::template Slot<R> ring[D];
#pragma unroll
  for (int j = 0; j + 1 < D; ++j) {
    load_w(wc, ring[j]);
    advance(wc);
  }
  store_x(0, H0, xh);
  if constexpr (H1 > 0) store_x(H0, H1, xh1);
  advance(xc);

  const PlaneDecode pd = plane_decode();
  uint32_t zlo[4], zhi[4];
  plane_chain_weights(zlo, zhi);
  f32x4_t acc[R][MT];
#pragma unroll
  for (int rt = 0; rt < R; ++rt)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) acc[rt][mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The (row tile, plane) pairs of a step, in two halves: the next step's
  // first X half is stored between them.
  constexpr int NPAIR = R * F::P, PSPLIT = NPAIR / 2;
  int blk = (int)blockIdx.x, cc = 0;
  int i0 = 0;
  do {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int i = i0 + j;
      const bool block_done = cc + 1 == CK;
      // This step's A fragments, all m-tiles; pairs 11 and 15 (the plain
      // +-1 positions) enter negated.
      uint32_t a[MT][4][4];
#pragma unroll
      for (int mi = 0; mi < MT; ++mi)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint4 v = *reinterpret_cast<const uint4*>(xb + xrow_chunk(16 * mi + r, 4 * t + q));
          a[mi][t][0] = v.x;
          a[mi][t][1] = v.y;
          a[mi][t][2] = v.z;
          a[mi][t][3] = v.w ^ (t >= 2 ? 0x80008000u : 0u);
        }
      // The next step's first X half and the weights D - 1 steps ahead.
      load_x(xc, 0, H0, xh);
      load_w(wc, ring[(j + D - 1) % D]);
      advance(wc);
      // Chain starts -Z per m-tile (and half, for sa* at G = 64).
      f32x4_t nz[MT][2];
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        f32x4_t z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
        z0 = mfma16x16x32(a[mi][0], zlo, z0);
        z0 = mfma16x16x32(a[mi][1], zlo, z0);
        if constexpr (F::kHalves) {
          z1 = mfma16x16x32(a[mi][2], zhi, z1);
          z1 = mfma16x16x32(a[mi][3], zhi, z1);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            nz[mi][0][e] = -z0[e];
            nz[mi][1][e] = -z1[e];
          }
        } else {
          z0 = mfma16x16x32(a[mi][2], zhi, z0);
          z0 = mfma16x16x32(a[mi][3], zhi, z0);
#pragma unroll
          for (int e = 0; e < 4; ++e) nz[mi][0][e] = -z0[e];
        }
      }
      const typename F::template Slot<R>& w = ring[j];
      static_for<0, PSPLIT>([&](auto k) {
        constexpr int kk = decltype(k)::value;
        F::template pair<R, MT>(w, kk / F::P, kk % F::P, a, nz, pd, acc);
      });
      store_x(0, H0, xh);
      if constexpr (H1 > 0) load_x(xc, H0, H1, xh);
      static_for<PSPLIT, NPAIR>([&](auto k) {
        constexpr int kk = decltype(k)::value;
        F::template pair<R, MT>(w, kk / F::P, kk % F::P, a, nz, pd, acc);
      });
      if constexpr (H1 > 0) store_x(H0, H1, xh);
      if (block_done) {
        // Uniform: every wave is at the same step.  The partial sums of one
        // row tile at a time meet in LDS; each wave's sum is minus the
        // output (the chains end at minus the signed sums).
        if (i < T) {
#pragma unroll
          for (int rt = 0; rt < R; ++rt) {
#pragma unroll
            for (int mi = 0; mi < MT; ++mi) {
              red[wave][mi][lane] = make_float4(acc[rt][mi][0], acc[rt][mi][1], acc[rt][mi][2], acc[rt][mi][3]);
              acc[rt][mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
            __syncthreads();
            for (int e = threadIdx.x; e < MT * 64; e += 64 * kMmqWaves) {
              const int ln = e & 63, mi = e >> 6;
              float4 tot = red[0][mi][ln];
#pragma unroll
              for (int ww = 1; ww < kMmqWaves; ++ww) {
                const float4 v = red[ww][mi][ln];
                tot.x += v.x;
                tot.y += v.y;
                tot.z += v.z;
                tot.w += v.w;
              }
              const int n = 16 * (R * blk + rt) + (ln & 15);
              const int mb = 16 * mi + 4 * (ln >> 4);
              const float v[4] = {-tot.x, -tot.y, -tot.z, -tot.w};
#pragma unroll
              for (int ii = 0; ii < 4; ++ii)
                if (mb + ii < M && n < N) Y[(size_t)(mb + ii) * N + n] = f32_to_bf16_rne(v[ii]);
            }
            __syncthreads();
          }
        }
        blk += (int)gridDim.x;
        cc = 0;
      } else {
        ++cc;
      }
      advance(xc);
    }
    i0 += D;
  } while (i0 < T);
}

// Host side: the launch of a 16 < M <= 64 sign-plane block (arguments
// already checked).  Block height R: the per-step registers (A fragments of
// MT m-tiles, R x MT accumulator tiles, two ring slots of R x P sign dwords
// and scales) allow R = 3 up to three planes, R = 1 at four m-tiles and six
// planes, else R = 2; within that, R = ceil(row tiles / CUs), so that about
// one block lands on each CU.  At four m-tiles and three planes a block of
// three spills 11 to 18 registers, reloaded at every step, and is still
// 11-13% faster at N = 12288 than blocks of two (768 row tiles: one block a
// CU instead of 384 blocks on 256 CUs); six planes at four m-tiles still
// spill a few registers at R = 1.
constexpr int mmq_planes_rmax(int MT, int P) { return P <= 3 ? 3 : MT >= 4 && P >= 6 ? 1 : 2; }

template <class F>
int launch_mmq_planes(const char* fn, const uint8_t* packed, const uint16_t* X, uint16_t* Y, int32_t M, int64_t N,
                      int64_t K, hipStream_t st) {
  int cus = 0;
  if (int rc = device_cus(&cus)) return rc;
  const int NT = (int)((N + 15) / 16), KT = (int)(K / 128);
  const int MT = (M + 15) / 16;
  const int rmax = mmq_planes_rmax(MT, F::P);
  int R = (NT + cus - 1) / cus;
  R = R < 1 ? 1 : R > rmax ? rmax : R;
  const int NB = (NT + R - 1) / R;
  const int grid = NB < cus ? NB : cus;
  auto go = [&](auto MTc, auto Rc) {
    hipLaunchKernelGGL((k_gemm_mmq_planes<F, decltype(MTc)::value, decltype(Rc)::value, 2>), dim3(grid),
                       dim3(64 * kMmqWaves), 0, st, packed, X, Y, M, (int)N, (int)K, KT, NT);
  };
  auto by_r = [&](auto MTc) {
    constexpr int rm = mmq_planes_rmax(decltype(MTc)::value, F::P);
    if constexpr (rm >= 3)
      if (R == 3) return go(MTc, ic<3>{});
    if constexpr (rm >= 2)
      if (R >= 2) return go(MTc, ic<2>{});
    go(MTc, ic<1>{});
  };
  if (MT <= 2)
    by_r(ic<2>{});
  else if (MT == 3)
    by_r(ic<3>{});
  else
    by_r(ic<4>{});
  return launched(fn);
}

}  // namespace
