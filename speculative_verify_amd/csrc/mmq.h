// mmq.h -- gfx950 mat-mul for blocks of 16 < M <= 64 activation rows (a
// prefill chunk or a long drafted block), W4A16 weights in the INT4 blob.
//   Y[m][n] = sum_g s[n][g] * sum_{k in g} c[n][k] * X[m][k]
//   (Efficient Qwen Competition report, sec. 2.1 and 3.3; the ShiftAddQwen
//   README places batches below 64 in its quantized mat-mul regime)
//
// The M <= 16 kernels keep a wave's whole K slice of X in registers; at
// M = 64 that slice no longer fits, so here X streams with the weights.
// Work decomposition: a workgroup owns R consecutive 16-row weight tiles (a
// block) at a time, grid-stride over blocks.  Its 8 waves form WM groups
// along M (MTW 16-row m-tiles each) times WK = 8 / WM groups along K; wave
// (wm, wk) walks the 128-wide column tiles [wk * CK, (wk + 1) * CK) of the
// block, and each step loads, for one column tile, its rows of X (cached,
// every workgroup reads them) and the block's R weight tiles (non-temporal,
// read once), D steps ahead.  A decoded weight tile feeds MTW MFMA chains
// and an X fragment R chains, so X is reused across the block's rows and the
// weights across the wave's m-tiles.  The partial sums of the WK groups meet
// in LDS once per block.
//
// X staging.  The MFMA A operand gives consecutive lanes consecutive rows,
// so loading it straight from row-major X touches one cache line per lane.
// Instead a quarter-wave loads one row's 256 bytes of the column tile (fully
// coalesced), the wave writes its rows into a private LDS region with the
// 16-byte chunks of row p XOR-swizzled by p mod 16, and reads them back in
// operand order: in both directions the 16 lanes of a quarter-wave touch 16
// distinct chunks of 256 bytes, so neither side has bank conflicts, and as
// the region is the wave's own no barrier is needed.
//
// Exact operands as in the M <= 16 kernel: nibble u = c + 8 decodes to the
// bf16 value 136 + c; the correction -136 * sum_k X[m][k] over the group is
// one MFMA chain per m-tile against the constant bf16 pair (-136, -136),
// shared by the block's R row tiles and exact term by term.
#pragma once

#include "kernels.h"

namespace {

constexpr int kMmqWaves = 8;
constexpr uint32_t kMinus136Pair = 0xC308C308u;  // bf16 pair (-136, -136)

template <int MTW, int R>
struct MmqSlot {
  uint4 x[MTW][4];  // load j = 4 mi + u: row 16 mi + 4 u + lane / 16, k chunk lane % 16
  uint4 c[R];       // the lane's 16 code bytes of each row tile of the block
  uint32_t s[R];    // bf16 scale of (row 16 rt + r, group g) in the low half
};

// Lane-dependent parts of a step's buffer offsets, fixed for the kernel:
// X row 16 (mt0 + mi) + 4 u + lane / 16 at k chunk lane % 16; the lane's 16
// bytes of a weight tile; row r of a scale run.  A step adds one uniform
// value per load (which carries bit 31 when the step reads nothing), so all
// range-relevant offsets stay in the per-lane register, where the buffer
// range check sees them: rows >= M and tiles past NT fall outside their
// sections and read zero.
template <int MTW>
struct MmqLanes {
  uint32_t x[MTW][4];
  uint32_t w, s;
};

template <int MTW>
__device__ __forceinline__ MmqLanes<MTW> mmq_lanes(int K, int KT4, int mt0, int lane) {
  MmqLanes<MTW> o;
#pragma unroll
  for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      o.x[mi][u] = ((uint32_t)(16 * (mt0 + mi) + 4 * u + (lane >> 4)) * (uint32_t)K + 8u * (lane & 15)) * 2u;
  o.w = 16u * lane;
  o.s = (uint32_t)(lane & 15) * (uint32_t)KT4 * 2u;
  return o;
}

// Loads step (blk, g) of a wave; `live` false makes the whole step read zero.
template <int MTW, int R>
__device__ __forceinline__ void load_mmq_step(MmqSlot<MTW, R>& sl, __amdgpu_buffer_rsrc_t xr, const BlobView& b,
                                              const MmqLanes<MTW>& lo, int blk, bool live, int g) {
  const uint32_t oob = oob_bit(live && g < b.KT);
  const uint32_t xs = (256u * g) | oob;
#pragma unroll
  for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const v4u_t v = __builtin_amdgcn_raw_buffer_load_b128(xr, lo.x[mi][u] + xs, 0, 0);
      sl.x[mi][u] = make_uint4(v.x, v.y, v.z, v.w);
    }
#pragma unroll
  for (int rt = 0; rt < R; ++rt) {
    const uint32_t tile = (uint32_t)(R * blk + rt);
    sl.c[rt] = ld_stream16(b.w, lo.w + (((tile * b.KT + g) * 1024u) | oob));
    sl.s[rt] = __builtin_amdgcn_raw_buffer_load_b16(b.s, lo.s + (((16u * tile * b.KT4 + g) * 2u) | oob), 0, 0);
  }
}

// Byte offset of 16-byte chunk c of row p in a wave's staging region.
__device__ __forceinline__ uint32_t mmq_chunk(int p, int c) { return (uint32_t)(p * 256 + ((c ^ (p & 15)) << 4)); }

// The slot's rows of X into the wave's region, then back as MFMA A operands:
// a[mi][t] is lane (q, r)'s X[16 (mt0 + mi) + r][128 g + 32 t + 8 q + 0..7].
template <int MTW>
__device__ __forceinline__ void mmq_stage_x(const uint4 (&x)[MTW][4], char* region, int lane, int q, int r,
                                            uint4 (&a)[MTW][4]) {
#pragma unroll
  for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<uint4*>(region + mmq_chunk(16 * mi + 4 * u + (lane >> 4), lane & 15)) = x[mi][u];
#pragma unroll
  for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
    for (int t = 0; t < 4; ++t)
      a[mi][t] = *reinterpret_cast<const uint4*>(region + mmq_chunk(16 * mi + r, 4 * t + q));
}

template <int MTW, int WM, int R, int D>
__global__ void __launch_bounds__(64 * kMmqWaves)
    k_gemm_mmq_w4a16(const uint8_t* __restrict__ blob, const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                     int M, int N, int K, int KT, int NT) {
  constexpr int WK = kMmqWaves / WM;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int wm = wave % WM, wk = wave / WM;
  const int mt0 = wm * MTW;
  const BlobView bv = int4_view(blob, KT, NT);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
  const int NB = (NT + R - 1) / R;
  const int CK = (KT + WK - 1) / WK;
  const int T = ((NB - 1 - (int)blockIdx.x) / (int)gridDim.x + 1) * CK;  // steps of every wave
  const MmqLanes<MTW> lo = mmq_lanes<MTW>(K, bv.KT4, mt0, lane);
  // Step order: the workgroup's blocks in turn (blockIdx.x, + gridDim.x, ...),
  // within a block the wave's column tiles wk * CK + (c + blockIdx.x) % CK,
  // c = 0 .. CK - 1.  Every workgroup reads all of X; starting each one at a
  // different column tile spreads those reads over the whole of X instead
  // of sending every CU to the same lines at once.  The load cursor runs D
  // steps ahead of the consumer.
  int ld_blk = (int)blockIdx.x, ld_c = 0, ld_rot = (int)blockIdx.x % CK, ld_i = 0;
  auto load_next = [&](MmqSlot<MTW, R>& slot) {
    load_mmq_step<MTW, R>(slot, xr, bv, lo, ld_blk, ld_i < T, wk * CK + ld_rot);
    ++ld_i;
    ld_rot = ld_rot + 1 == CK ? 0 : ld_rot + 1;
    if (++ld_c == CK) {
      ld_c = 0;
      ld_blk += (int)gridDim.x;
    }
  };

  MmqSlot<MTW, R> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    load_next(ring[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
  __shared__ float4 red[WK][WM * R * MTW][64];
  __shared__ uint4 xstage[kMmqWaves][MTW * 16 * 16];  // a wave's rows of one column tile
  char* region = reinterpret_cast<char*>(xstage[wave]);
  const PairDecode magic = int4_decode();
  const uint32_t minus136[4] = {kMinus136Pair, kMinus136Pair, kMinus136Pair, kMinus136Pair};
  f32x4_t acc[R][MTW];
#pragma unroll
  for (int rt = 0; rt < R; ++rt)
#pragma unroll
    for (int mi = 0; mi < MTW; ++mi) acc[rt][mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int blk = (int)blockIdx.x, cc = 0;  // consumer: current block, column tiles done in it
  int i0 = 0;
  do {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int i = i0 + j;
      const MmqSlot<MTW, R>& sl = ring[j];
      uint4 xa[MTW][4];
      mmq_stage_x<MTW>(sl.x, region, lane, q, r, xa);
      // All R x MTW chains advance together, one 32-wide k block at a time,
      // so consecutive MFMAs are independent; the correction chain of each
      // m-tile leads its k block.
      f32x4_t corr[MTW], c[R][MTW];
#pragma unroll
      for (int mi = 0; mi < MTW; ++mi) corr[mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int mi = 0; mi < MTW; ++mi) {
          const uint32_t a[4] = {xa[mi][t].x, xa[mi][t].y, xa[mi][t].z, xa[mi][t].w};
          corr[mi] = mfma16x16x32(a, minus136, corr[mi]);
        }
#pragma unroll
        for (int rt = 0; rt < R; ++rt) {
          const uint32_t wt = t == 0 ? sl.c[rt].x : t == 1 ? sl.c[rt].y : t == 2 ? sl.c[rt].z : sl.c[rt].w;
          const uint32_t bq[4] = {int4_pair(wt, 0, magic), int4_pair(wt, 1, magic), int4_pair(wt, 2, magic),
                                  int4_pair(wt, 3, magic)};
#pragma unroll
          for (int mi = 0; mi < MTW; ++mi) {
            const uint32_t a[4] = {xa[mi][t].x, xa[mi][t].y, xa[mi][t].z, xa[mi][t].w};
            c[rt][mi] = mfma16x16x32(a, bq, t == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : c[rt][mi]);
          }
        }
      }
#pragma unroll
      for (int rt = 0; rt < R; ++rt) {
        const float sc = __uint_as_float(sl.s[rt] << 16);
#pragma unroll
        for (int mi = 0; mi < MTW; ++mi)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[rt][mi][e] = fmaf(sc, c[rt][mi][e] + corr[mi][e], acc[rt][mi][e]);
      }
      // Slot j is refilled only after its last use, so it keeps its registers.
      __builtin_amdgcn_sched_barrier(0);
      load_next(ring[j]);
      // The block's last column tile: every wave is at the same step, so the
      // condition (and the barriers under it) is uniform across the workgroup.
      const bool block_done = ++cc == CK;
      if (block_done) cc = 0;
      if (i < T && block_done) {
#pragma unroll
        for (int rt = 0; rt < R; ++rt)
#pragma unroll
          for (int mi = 0; mi < MTW; ++mi) {
            red[wk][(wm * R + rt) * MTW + mi][lane] =
                make_float4(acc[rt][mi][0], acc[rt][mi][1], acc[rt][mi][2], acc[rt][mi][3]);
            acc[rt][mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
        __syncthreads();
        for (int e = threadIdx.x; e < WM * R * MTW * 64; e += 64 * kMmqWaves) {
          const int ln = e & 63, slot = e >> 6;
          const int mi = slot % MTW, rt = (slot / MTW) % R, wmm = slot / (MTW * R);
          float4 tot = red[0][slot][ln];
#pragma unroll
          for (int w = 1; w < WK; ++w) {
            const float4 v = red[w][slot][ln];
            tot.x += v.x;
            tot.y += v.y;
            tot.z += v.z;
            tot.w += v.w;
          }
          const int n = 16 * (R * blk + rt) + (ln & 15);
          const int mb = 16 * (wmm * MTW + mi) + 4 * (ln >> 4);
          const float v[4] = {tot.x, tot.y, tot.z, tot.w};
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            if (mb + ii < M && n < N) Y[(size_t)(mb + ii) * N + n] = f32_to_bf16_rne(v[ii]);
        }
        __syncthreads();
      }
      if (block_done) blk += (int)gridDim.x;
    }
    i0 += D;
  } while (i0 < T);
}

}  // namespace
