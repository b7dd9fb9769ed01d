// mmq.h -- gfx950 mat-mul for blocks of 16 < M <= 64 activation rows (a
// prefill chunk or a long drafted block), W4A16 weights in the INT4 blob.
//   Y[m][n] = sum_g s[n][g] * sum_{k in g} c[n][k] * X[m][k]
//   (Efficient Qwen Competition report, sec. 2.1 and 3.3; the ShiftAddQwen
//   README places batches below 64 in its quantized mat-mul regime)
//
// The M <= 16 kernels keep a wave's whole K slice of X in registers; at
// M = 64 that slice no longer fits, so here X streams with the weights.
// Blocks at K <= 4096 run on the M <= 16 kernel instead (each 16-row tile on
// workgroups of its own, or two tiles in registers), which measured faster
// for every block height; this kernel serves K above 4096.
// Work decomposition: a workgroup owns R consecutive 16-row weight tiles (a
// block) at a time, grid-stride over blocks; its 8 waves split K, wave w
// walking the 128-wide column tiles [w * CK, (w + 1) * CK) of the block.  A
// step of a wave covers one column tile for all MT 16-row m-tiles of X and
// the block's R weight tiles: the weights are decoded once per step and feed
// MT MFMA chains each, and every X fragment feeds R chains.  The partial
// sums of the 8 waves meet in LDS once per block.
//
// Data movement per step.  Weight tiles (read once, non-temporal) run in a
// register ring D - 1 steps ahead.  X (read by every workgroup, cached) is
// loaded coalesced -- a quarter-wave reads one row's 256 bytes of the column
// tile -- one step ahead, in two halves of at most two m-tiles, and written
// into the wave's private LDS buffer with the 16-byte chunks of row p
// XOR-swizzled by p mod 16; the MFMA fragments are read back from it one
// m-tile at a time (both directions free of bank conflicts).  LDS executes a
// wave's operations in order, so a half of the next step's X is written as
// soon as the current step has read the rows it replaces; no barrier is
// needed until the block ends.
//
// Exact operands as in the M <= 16 kernel: nibble u = c + 8 decodes to the
// bf16 value 136 + c, and the 136 is taken back out per group by subtracting
// the same MFMA chain run on the constant pair (136, 136) (one chain per
// m-tile and step, shared by the block's row tiles), so a group whose codes
// are all zero cancels to exactly 0.
#pragma once

#include "kernels.h"

namespace {

constexpr int kMmqWaves = 8;

// The R weight tiles of one step and their scales.
template <int R>
struct MmqW {
  uint4 c[R];     // the lane's 16 code bytes of each row tile of the block
  uint32_t s[R];  // bf16 scale of (row 16 rt + r, group g) in the low half
};

template <int MT, int R, int D>
__global__ void __launch_bounds__(64 * kMmqWaves)
    k_gemm_mmq_w4a16(const uint8_t* __restrict__ blob, const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                     int M, int N, int K, int KT, int NT) {
  // m-tiles of the first and second half of a step's X: the whole step in
  // one half when the registers allow (one row tile per block).
  constexpr int H0 = (MT < 2 || R == 1) ? MT : 2;
  constexpr int H1 = MT - H0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const BlobView bv = int4_view(blob, KT, NT);
  // Rows >= M lie past the end of this range and read zero; the range check
  // sees the whole offset, which is kept in the per-lane register.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
  const int NB = (NT + R - 1) / R;
  const int CK = (KT + kMmqWaves - 1) / kMmqWaves;
  const int T = ((NB - 1 - (int)blockIdx.x) / (int)gridDim.x + 1) * CK;  // steps of every wave

  // LDS: each wave's X buffer (MT * 16 rows of 256 bytes), then the
  // cross-wave staging of one row tile's partial sums.
  __shared__ uint4 xbuf[kMmqWaves][MT * 16 * 16];
  __shared__ float4 red[kMmqWaves][MT][64];
  char* xb = reinterpret_cast<char*>(xbuf[wave]);

  // Lane-dependent offsets.  X: row 4 u + lane / 16 of an m-tile, chunk
  // lane % 16; the m-tile and the column tile are added per load.
  const uint32_t xlane = ((uint32_t)(lane >> 4) * (uint32_t)K + 8u * (lane & 15)) * 2u;
  const uint32_t xrow4 = 4u * (uint32_t)K * 2u;  // four rows further
  const uint32_t wlane = 16u * lane, slane = (uint32_t)r * (uint32_t)bv.KT4 * 2u;

  // Step order: the workgroup's blocks in turn; within a block the wave's
  // column tiles w * CK + (c + blockIdx.x) % CK, c = 0 .. CK - 1 (every
  // workgroup reads all of X; starting each at a different column tile
  // spreads those reads over X).  Cursors for X (one step ahead) and the
  // weights (D - 1 ahead) advance without division.
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
          const uint32_t off = xlane + (uint32_t)(mt0 + h) * 4u * xrow4 + (uint32_t)v * xrow4;  // row 16 (mt0 + h) + 4 v
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
  auto load_w = [&](const Cursor& u, MmqW<R>& w) {
    const uint32_t oob = step_oob(u);
    const uint32_t g = (uint32_t)col(u);
#pragma unroll
    for (int rt = 0; rt < R; ++rt) {
      const uint32_t tile = (uint32_t)(R * u.blk + rt);
      w.c[rt] = ld_stream16(bv.w, wlane + (((tile * bv.KT + g) * 1024u) | oob));
      w.s[rt] = __builtin_amdgcn_raw_buffer_load_b16(bv.s, slane + (((16u * tile * bv.KT4 + g) * 2u) | oob), 0, 0);
    }
  };

  Cursor xc{(int)blockIdx.x, 0, (int)blockIdx.x % CK, 0};
  Cursor wc = xc;
  uint4 xh[H0][4];
  // Prologue: step 0's X into LDS (both halves requested before either is
  // stored: the accumulators are not live yet, so the second half has
  // registers of its own), the first D - 1 steps' weights in flight.
  load_x(xc, 0, H0, xh);
  uint4 xh1[H1 > 0 ? H0 : 1][4];
  if constexpr (H1 > 0) load_x(xc, H0, H1, xh1);
  MmqW<R> ring[D];
#pragma unroll
  for (int j = 0; j + 1 < D; ++j) {
    load_w(wc, ring[j]);
    advance(wc);
  }
  store_x(0, H0, xh);
  if constexpr (H1 > 0) store_x(H0, H1, xh1);
  advance(xc);

  const PairDecode magic = int4_decode();
  const uint32_t zero_codes[4] = {kInt4ZeroPair, kInt4ZeroPair, kInt4ZeroPair, kInt4ZeroPair};
  f32x4_t acc[R][MT];
#pragma unroll
  for (int rt = 0; rt < R; ++rt)
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) acc[rt][mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int blk = (int)blockIdx.x, cc = 0;  // consumer: current block, column tiles done in it
  int i0 = 0;
  do {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int i = i0 + j;
      const bool block_done = cc + 1 == CK;
      // Next step's X (first half) goes out first.  The weights D - 1 steps
      // ahead (into the slot step i - 1 freed) follow the last X load of the
      // step: loads complete in order, so waiting for that X then leaves the
      // weight loads in flight.
      load_x(xc, 0, H0, xh);
      if constexpr (H1 == 0) {
        load_w(wc, ring[(j + D - 1) % D]);
        advance(wc);
      }
      const MmqW<R>& w = ring[j];
      uint32_t bq[R][4][4];
      float sc[R];
#pragma unroll
      for (int rt = 0; rt < R; ++rt) {
        const uint32_t wd[4] = {w.c[rt].x, w.c[rt].y, w.c[rt].z, w.c[rt].w};
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) bq[rt][t][e] = int4_pair(wd[t], e, magic);
        sc[rt] = __uint_as_float(w.s[rt] << 16);
      }
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        uint32_t a[4][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint4 v = *reinterpret_cast<const uint4*>(xb + xrow_chunk(16 * mi + r, 4 * t + q));
          a[t][0] = v.x;
          a[t][1] = v.y;
          a[t][2] = v.z;
          a[t][3] = v.w;
        }
        // The first half's rows have been read: the next step's first half
        // replaces them (in-order LDS) and its second half goes out.
        if constexpr (H1 > 0) {
          if (mi == H0 - 1) {
            if (!block_done) {
              store_x(0, H0, xh);
              load_x(xc, H0, H1, xh);
            }
            load_w(wc, ring[(j + D - 1) % D]);
            advance(wc);
          }
        }
        // The zero-code chain and the R tiles' chains: the same four MFMAs
        // from zero, so a tile's chain equals the zero-code one bit for bit
        // where its codes are zero.
        f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        f32x4_t c[R];
#pragma unroll
        for (int rt = 0; rt < R; ++rt) c[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          z = mfma16x16x32(a[t], zero_codes, z);
#pragma unroll
          for (int rt = 0; rt < R; ++rt) c[rt] = mfma16x16x32(a[t], bq[rt][t], c[rt]);
        }
#pragma unroll
        for (int rt = 0; rt < R; ++rt)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[rt][mi][e] = fmaf(sc[rt], c[rt][e] - z[e], acc[rt][mi][e]);
      }
      if (block_done) {
        // Every wave is at the same step, so this branch (and its barriers)
        // is uniform.  The partial sums of one row tile at a time meet in LDS.
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
              const float v[4] = {tot.x, tot.y, tot.z, tot.w};
#pragma unroll
              for (int ii = 0; ii < 4; ++ii)
                if (mb + ii < M && n < N) Y[(size_t)(mb + ii) * N + n] = f32_to_bf16_rne(v[ii]);
            }
            __syncthreads();
          }
        }
        blk += (int)gridDim.x;
        cc = 0;
        // The next block's first X: its first half waited in registers.
        store_x(0, H0, xh);
        if constexpr (H1 > 0) {
          load_x(xc, H0, H1, xh);
          store_x(H0, H1, xh);
        }
      } else {
        ++cc;
        if constexpr (H1 > 0) store_x(H0, H1, xh);
        else store_x(0, H0, xh);
      }
      advance(xc);
    }
    i0 += D;
  } while (i0 < T);
}

}  // namespace
