// kernels.h -- gfx950 (CDNA4) device code behind the entry points of svq.h:
// helpers, tile loaders and the kernel templates, instantiated by the
// translation units that launch them (svq_int4.hip, svq_planes_*.hip,
// svq_sa_*.hip).
//
// What is computed (see svq.h for the full statements and citations):
//   W4A16         y = sum_g s[n][g] * sum_{k in g} c[n][k] x[k]
//                 (Efficient Qwen Competition report, sec. 2.1 and 3.3)
//   binary planes y = sum_g sum_p alpha[p][n][g] * sum_{k in g} b[p][n][k] x[k]
//                 (ShiftAddQwen README, intro and "Method / Format")
//   sa* storage   the same with alpha[p][n][g] = d[n][j] * a[p][n][g]: u8 codes
//                 a, one fp16 d per 256-weight super-block j (same page,
//                 "Method / Format")
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
// dot products see 136 + c exactly.  The 136 is taken back out per group
// before the scale is applied: the same chain of instructions, in the same
// order, run once on the constant operand 136 gives the value subtracted, so
// a group whose codes are all zero (decoded 136) cancels to exactly 0 and
// otherwise only the two chains' fp32 rounding remains.  A sign bit becomes the
// bf16 value +1 or -1 (0x3F80 with the sign bit set for b = -1) with one
// shift and one AND-OR; the M <= 16 sign-plane tiles skip the shift (see
// plane_operands) and the M = 1 ones read precomputed signed sums from LDS.
// Neither s*c nor sum_p alpha_p b_p is ever rounded to bf16; the scales are
// applied per group in fp32, and the output is rounded to bf16 once, to
// nearest even.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cstdint>
#include <type_traits>

#include "svq.h"

namespace {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

constexpr uint32_t kInt4Magic = 0x43004300u;  // bf16 pair (128, 128)
constexpr uint32_t kOnePair = 0x3F803F80u;    // bf16 pair (1, 1)
constexpr uint32_t kInt4ZeroPair = 0x43084308u;  // bf16 pair (136, 136): two decoded zero codes

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

// An SGPR holding the constant V, produced by a scalar move the compiler
// cannot see through, so it is not folded back into a literal.
template <uint32_t V>
__device__ __forceinline__ uint32_t opaque_sgpr() {
  uint32_t s;
  asm volatile("s_mov_b32 %0, %1" : "=s"(s) : "i"(V));
  return s;
}

// The same for a VGPR (one move at kernel start; only VALU instructions read
// it, so no matrix-core hazard depends on this move).
template <uint32_t V>
__device__ __forceinline__ uint32_t opaque_vgpr() {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "i"(V));
  return v;
}

// The wave's index in its workgroup, as a wave-uniform (scalar) value: the
// compiler cannot tell that threadIdx.x >> 6 is the same in every lane, and
// would otherwise form every address term derived from it (the wave's
// column tiles) with vector instructions at each step.  (In the streaming
// 16 < M <= 64 sign-plane kernel this made the M = 64 calls 4-5% faster; in
// the other kernels, whose per-step addressing is lighter, it made no
// difference or cost 1-4%.)
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// A copy of v the compiler cannot see through (its known bits are lost).  Only
// VALU instructions read the result.
__device__ __forceinline__ uint32_t opaque_copy(uint32_t v) {
  uint32_t d;
  asm volatile("v_mov_b32 %0, %1" : "=v"(d) : "v"(v));
  return d;
}

// Pair decoders: one shift plus one v_and_or_b32 per bf16 pair.  The VOP3
// encoding of v_and_or_b32 takes no literal and at most one SGPR, so the
// mask lives in an SGPR and the OR value in a VGPR; with literals the
// compiler would split the operation into an AND and an OR.
struct PairDecode {
  uint32_t mask, orv;
};

// Nibble pairs: each u = c + 8 becomes the bf16 value 128 + u.
__device__ __forceinline__ PairDecode int4_decode() {
  return PairDecode{opaque_sgpr<0x000F000Fu>(), opaque_vgpr<kInt4Magic>()};
}

// Sign pairs: a clear bit becomes +1, a set bit -1 (the bit lands in the
// bf16 sign position).
__device__ __forceinline__ PairDecode sign_decode() {
  return PairDecode{opaque_sgpr<0x80008000u>(), opaque_vgpr<kOnePair>()};
}

// bf16 pair (136 + c_even, 136 + c_odd) for pair i (k = 2i, 2i+1) of a code dword.
__device__ __forceinline__ uint32_t int4_pair(uint32_t w, int i, const PairDecode& d) {
  return ((w >> (4 * i)) & d.mask) | d.orv;
}

// int4_pair of pairs i = 0..3 of the two code dwords lo and hi, with one
// 64-bit shift of hi:lo per nonzero i in place of two 32-bit ones: the bits
// a shift moves from hi into lo land at bits 20 and up, outside the mask.
__device__ __forceinline__ void int4_pairs2(uint32_t lo, uint32_t hi, const PairDecode& d, uint32_t (&bl)[4],
                                            uint32_t (&bh)[4]) {
  const uint64_t w = (uint64_t)hi << 32 | lo;
  uint64_t s[4];
  s[0] = w;
  asm("v_lshrrev_b64 %0, 4, %1" : "=v"(s[1]) : "v"(w));
  asm("v_lshrrev_b64 %0, 8, %1" : "=v"(s[2]) : "v"(w));
  asm("v_lshrrev_b64 %0, 12, %1" : "=v"(s[3]) : "v"(w));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bl[i] = ((uint32_t)s[i] & d.mask) | d.orv;
    bh[i] = ((uint32_t)(s[i] >> 32) & d.mask) | d.orv;
  }
}

// bf16 pair (b_even, b_odd) in {-1, +1} for pair ip = 4t + i of a sign dword.
__device__ __forceinline__ uint32_t sign_pair(uint32_t w, int ip, const PairDecode& d) {
  return ((w << (15 - ip)) & d.mask) | d.orv;
}

// Sign-plane MFMA operands, one AND-OR per bf16 pair.  A sign bit b is not
// moved to the bf16 sign position; it stays where a view of the dword puts
// it, at bit 4, 5, 6 or 7 of a half (or 15), over a base C chosen so that
// setting the bit adds exactly 2: C = 16, 8, 4 (mantissa bits 4-6, one ulp
// of C being 2^-3 C, 2^-2 C, 2^-1 C) and C = 2 (exponent LSB, 2 -> 4).  At
// bit 15 the pair is the plain +-1 and its activations enter negated.  Every
// product is then c x + 2 b x with c in {16, 8, 4, 2, -1} known per
// position, so a chain started at -(sum x + sum c x) over the group ends at
// -(sum of (1 - 2b) x): minus the plane's signed sum.  Four views (w, w << 4,
// w >> 4, w >> 8) cover the 16 pairs: 3 shifts and 16 AND-ORs per dword.
struct PlaneDecode {
  uint32_t m4, m5, m6, m7, m15;  // SGPR masks: bit p of both halves
  uint32_t c4, c5, c6, c7, c15;  // VGPR base pairs
};

__device__ __forceinline__ PlaneDecode plane_decode() {
  return PlaneDecode{opaque_sgpr<0x00100010u>(), opaque_sgpr<0x00200020u>(), opaque_sgpr<0x00400040u>(),
                     opaque_sgpr<0x00800080u>(), opaque_sgpr<0x80008000u>(), opaque_vgpr<0x41804180u>(),
                     opaque_vgpr<0x41004100u>(), opaque_vgpr<0x40804080u>(), opaque_vgpr<0x40004000u>(),
                     opaque_vgpr<kOnePair>()};
}

// B operands of the four 32-wide k blocks of sign dword w: b[t][i] is pair
// ip = 4t + i (bits ip and 16 + ip of w).
__device__ __forceinline__ void plane_operands(uint32_t w, const PlaneDecode& d, uint32_t (&b)[4][4]) {
  const uint32_t v1 = w << 4, v2 = w >> 4, v3 = w >> 8;
  b[0][0] = (v1 & d.m4) | d.c4;  // pairs 0-3 at bits 4-7 of w << 4
  b[0][1] = (v1 & d.m5) | d.c5;
  b[0][2] = (v1 & d.m6) | d.c6;
  b[0][3] = (v1 & d.m7) | d.c7;
  b[1][0] = (w & d.m4) | d.c4;  // pairs 4-7 at bits 4-7 of w
  b[1][1] = (w & d.m5) | d.c5;
  b[1][2] = (w & d.m6) | d.c6;
  b[1][3] = (w & d.m7) | d.c7;
  b[2][0] = (v2 & d.m4) | d.c4;  // pairs 8-10 at bits 4-6 of w >> 4
  b[2][1] = (v2 & d.m5) | d.c5;
  b[2][2] = (v2 & d.m6) | d.c6;
  b[2][3] = (v1 & d.m15) | d.c15;  // pair 11 at bit 15 of w << 4
  b[3][0] = (v3 & d.m4) | d.c4;  // pairs 12-14 at bits 4-6 of w >> 8
  b[3][1] = (v3 & d.m5) | d.c5;
  b[3][2] = (v3 & d.m6) | d.c6;
  b[3][3] = (w & d.m15) | d.c15;  // pair 15 at bit 15 of w
}

// The same operands one 32-wide k block at a time, from the four views of
// the dword (w, w << 4, w >> 4, w >> 8), so that several dwords' MFMA
// chains can be interleaved without holding every decoded operand.
struct PlaneViews {
  uint32_t w, v1, v2, v3;
};

__device__ __forceinline__ PlaneViews plane_views(uint32_t w) { return PlaneViews{w, w << 4, w >> 4, w >> 8}; }

// The views of two sign dwords at once, by 64-bit shifts of the pair: the
// bits one dword's view receives from the other lie only where no view is
// read (bits 0-3 of hi's w << 4; bits 28-31 and 24-31 of lo's w >> 4 and
// w >> 8).  A 64-bit shift issues at about 1.1 times the cost of a 32-bit
// one on gfx950 (measured), and the compiler would split these into 32-bit
// shifts, so they are written out.
__device__ __forceinline__ void plane_views2(uint32_t lo, uint32_t hi, PlaneViews& vl, PlaneViews& vh) {
  const uint64_t w = (uint64_t)hi << 32 | lo;
  uint64_t a, b, c;
  asm("v_lshlrev_b64 %0, 4, %1" : "=v"(a) : "v"(w));
  asm("v_lshrrev_b64 %0, 4, %1" : "=v"(b) : "v"(w));
  asm("v_lshrrev_b64 %0, 8, %1" : "=v"(c) : "v"(w));
  vl = PlaneViews{lo, (uint32_t)a, (uint32_t)b, (uint32_t)c};
  vh = PlaneViews{hi, (uint32_t)(a >> 32), (uint32_t)(b >> 32), (uint32_t)(c >> 32)};
}

// Views of the sign dwords w(0) .. w(N - 1), two at a time where N allows.
template <int N, class W>
__device__ __forceinline__ void plane_views_n(W&& w, PlaneViews (&v)[N]) {
  if constexpr (N % 2 == 0) {
#pragma unroll
    for (int u = 0; u < N; u += 2) plane_views2(w(u), w(u + 1), v[u], v[u + 1]);
  } else {
#pragma unroll
    for (int u = 0; u < N; ++u) v[u] = plane_views(w(u));
  }
}

__device__ __forceinline__ void plane_operands_t(const PlaneViews& v, int t, const PlaneDecode& d, uint32_t (&b)[4]) {
  const uint32_t lo = t == 0 ? v.v1 : t == 1 ? v.w : t == 2 ? v.v2 : v.v3;
  b[0] = (lo & d.m4) | d.c4;
  b[1] = (lo & d.m5) | d.c5;
  b[2] = (lo & d.m6) | d.c6;
  b[3] = t < 2 ? (lo & d.m7) | d.c7 : ((t == 2 ? v.v1 : v.w) & d.m15) | d.c15;
}

// Chain-start weights (1 + c) of the 16 pair positions of a k block, as
// bf16 pairs: 17, 9, 5, 3 for the positions decoded over bases 16, 8, 4, 2,
// and 0 at the two plain +-1 positions (pairs 11 and 15).
__device__ __forceinline__ void plane_chain_weights(uint32_t (&lo)[4], uint32_t (&hi)[4]) {
  lo[0] = opaque_vgpr<0x41884188u>();  // 17
  lo[1] = opaque_vgpr<0x41104110u>();  // 9
  lo[2] = opaque_vgpr<0x40A040A0u>();  // 5
  lo[3] = opaque_vgpr<0x40404040u>();  // 3: k blocks 0 and 1
  hi[0] = lo[0];
  hi[1] = lo[1];
  hi[2] = lo[2];
  hi[3] = opaque_vgpr<0u>();  // the +-1 positions of k blocks 2 and 3
}

// Sum over the four lanes r, r+16, r+32, r+48 of a wave (the q index), via
// the gfx950 lane-swap instructions (no LDS traffic).
__device__ __forceinline__ float sum_over_q(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float a = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  const uint32_t ua = __float_as_uint(a);
  const auto s16 = __builtin_amdgcn_permlane16_swap(ua, ua, false, false);
  return __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
}

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Running greedy choices (value, row) combined across lanes without LDS:
// DPP moves within a row of 16 lanes (rotations by 8 and 4, then the quad
// swaps of lanes 1 apart and 2 apart) and the gfx950 lane-swap instructions
// across rows.  Every lane ends with the best of the lanes combined, lowest
// row on equal values.
template <int CTRL>
__device__ __forceinline__ void best_with_dpp(float& v, int& i) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xF, 0xF, false);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// Over the 16 lanes of each row.
__device__ __forceinline__ void best_over_row(float& v, int& i) {
  best_with_dpp<0x128>(v, i);  // row_ror:8
  best_with_dpp<0x124>(v, i);  // row_ror:4
  best_with_dpp<0x4E>(v, i);   // quad_perm [2, 3, 0, 1]
  best_with_dpp<0xB1>(v, i);   // quad_perm [1, 0, 3, 2]
}

// Over all 64 lanes of the wave.
__device__ __forceinline__ void best_over_wave(float& v, int& i) {
  {
    const auto sv = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const auto si = __builtin_amdgcn_permlane32_swap((uint32_t)i, (uint32_t)i, false, false);
    v = __uint_as_float(sv[0]);
    i = (int)si[0];
    if (better(__uint_as_float(sv[1]), (int)si[1], v, i)) {
      v = __uint_as_float(sv[1]);
      i = (int)si[1];
    }
  }
  {
    const auto sv = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const auto si = __builtin_amdgcn_permlane16_swap((uint32_t)i, (uint32_t)i, false, false);
    v = __uint_as_float(sv[0]);
    i = (int)si[0];
    if (better(__uint_as_float(sv[1]), (int)si[1], v, i)) {
      v = __uint_as_float(sv[1]);
      i = (int)si[1];
    }
  }
  best_over_row(v, i);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(const uint32_t* a, const uint32_t* b, f32x4_t c) {
  u32x4_t av = {a[0], a[1], a[2], a[3]};
  u32x4_t bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                 __builtin_bit_cast(bf16x8_t, bv), c, 0, 0, 0);
}

// Chain starts of the sign-plane MFMA tiles: -Z per group of GPW (per half
// group, k blocks 0-1 and 2-3, when H = 2), Z[m] = sum_k (1 + c_k) x[m][k],
// as an MFMA chain of the activation operands against the constant operand
// (1 + c_k).  Every column of the product holds Z, so each lane receives it
// for the rows 4q + i its accumulators hold, with no cross-lane moves.
template <int GPW, int H>
__device__ __forceinline__ void plane_chain_starts(const uint32_t (&xa)[GPW][16], f32x4_t (&cs)[GPW][2]) {
  uint32_t lo[4], hi[4];
  plane_chain_weights(lo, hi);
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    f32x4_t z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
    z0 = mfma16x16x32(&xa[gi][0], lo, z0);
    z0 = mfma16x16x32(&xa[gi][4], lo, z0);
    if constexpr (H == 2) {
      z1 = mfma16x16x32(&xa[gi][8], hi, z1);
      z1 = mfma16x16x32(&xa[gi][12], hi, z1);
    } else {
      z0 = mfma16x16x32(&xa[gi][8], hi, z0);
      z0 = mfma16x16x32(&xa[gi][12], hi, z0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cs[gi][0][e] = -z0[e];
      cs[gi][1][e] = -z1[e];
    }
  }
}

// ---------------------------------------------------------------------------
// Activation staging: lane (q, r) keeps the bf16 pairs of activation row
// `row` at k = 128g + 32t + 8q + [0, 8) for the wave's GPW groups:
// xp[gi][4t + i] is the pair (k, k+1), k = 128g + 32t + 8q + 2i.  Rows >= M
// and groups >= KT read a clamped (valid) address; mask_x_pairs() zeroes
// them afterwards, so the loads stay branch-free and can be issued before
// the weight prefetch while their consumers wait until after it.
template <int GPW>
__device__ __forceinline__ void load_x_pairs(const uint32_t* __restrict__ X, int row, int M, int g0, int KT, int q,
                                             uint32_t (&xp)[GPW][16]) {
  const uint32_t* xrow = X + (size_t)min(row, M - 1) * KT * 64;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 v = *reinterpret_cast<const uint4*>(xrow + 64 * min(g0 + gi, KT - 1) + 16 * t + 4 * q);
      xp[gi][4 * t + 0] = v.x;
      xp[gi][4 * t + 1] = v.y;
      xp[gi][4 * t + 2] = v.z;
      xp[gi][4 * t + 3] = v.w;
    }
}

template <int GPW>
__device__ __forceinline__ void mask_x_pairs(int row, int M, int g0, int KT, uint32_t (&xp)[GPW][16]) {
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const bool live = row < M && g0 + gi < KT;
#pragma unroll
    for (int j = 0; j < 16; ++j) xp[gi][j] = live ? xp[gi][j] : 0u;
  }
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// The M = 1 W4A16 chain of each of the lane's groups run on decoded zero
// codes: 136 * (the lane's sum of x over the group), formed by exactly the
// dot2 sequence w4a16_tile_partial applies to a tile, so the two agree bit
// for bit wherever the tile's codes are zero.
template <int GPW>
__device__ __forceinline__ void lane_zero_code_chains(const uint32_t (&xp)[GPW][16], float (&z)[GPW]) {
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s = dot2(kInt4ZeroPair, xp[gi][j], s);
    z[gi] = s;
  }
}

// ---------------------------------------------------------------------------
// Tile loaders (global -> registers).  Weights and scales are read through
// buffer resources: an access at an offset past the section's end returns
// zero without touching memory.  Tiles past the workgroup's last tile (the
// pipeline's tail) and groups past K (a wave's unused slots) are given such
// an offset, so every load is unconditional -- the compiler then counts
// outstanding loads exactly and a D-deep ring of tiles stays in flight while
// earlier tiles are computed -- and the tail costs no HBM traffic.  Weight
// bytes are read once per call, so they are loaded non-temporally.
typedef uint32_t v2u_t __attribute__((ext_vector_type(2)));
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));


// 2^31 (past the end of every section, which are all < 2 GiB) unless `valid`;
// OR-ed into an in-range offset (always < 2^31),
// so the choice stays arithmetic instead of becoming a branch around a load.
__device__ __forceinline__ uint32_t oob_bit(bool valid) { return (uint32_t)(!valid) << 31; }
constexpr int kAuxStream = 2;                   // cache policy: non-temporal
constexpr int kBufferFlags = 0x00020000;        // raw (unswizzled, unformatted) buffer

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFlags);
}

__device__ __forceinline__ uint4 ld_stream16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4u_t t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAuxStream);
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ uint32_t ld_stream4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kAuxStream);
}

// Activation staging for the M = 1 kernels.  The 16 lanes of a row q all
// need the same 16 pairs (their k sub-range), so instead of loading them 16
// times over, lane (q, r) loads only the pair with (t, i) = (r/4, r%4) -- a
// wave reads each of a group's 64 pairs exactly once -- and DPP row_newbcast
// then copies pair j of the row to every lane of the row.  Groups past K
// read zero (buffer offset bit 31), so nothing is masked afterwards.
template <int GPW>
__device__ __forceinline__ void load_x_own(const uint32_t* __restrict__ xw, int g0, int KT, int q, int r,
                                           uint32_t (&xo)[GPW]) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(xw, (uint32_t)KT * 256u);
  const uint32_t lo = (uint32_t)(16 * (r >> 2) + 4 * q + (r & 3)) * 4u;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi)
    xo[gi] = __builtin_amdgcn_raw_buffer_load_b32(rs, (lo + 256u * (uint32_t)(g0 + gi)) | oob_bit(g0 + gi < KT), 0, 0);
}

template <int GPW>
__device__ __forceinline__ void expand_x(const uint32_t (&xo)[GPW], uint32_t (&xp)[GPW][16]) {
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    static_for<0, 16>([&](auto J) {
      constexpr int j = decltype(J)::value;
      // Every lane is written (all rows and banks enabled), so the move
      // needs no old value and the compiler no initialising move.
      xp[gi][j] = __builtin_amdgcn_mov_dpp(xo[gi], 0x150 + j, 0xF, 0xF, false);  // row_newbcast:j
    });
  }
}

// GPW consecutive 16-bit scale entries, kept as the raw dwords one load
// returns (entry gi in the low half of dword gi/2 when gi is even, in the
// high half when odd) and unpacked at the point of use.
template <int GPW>
struct U16Run {
  uint32_t d[(GPW + 1) / 2];

  __device__ __forceinline__ float bf16(int gi) const {  // entry gi as a bf16 value
    return __uint_as_float((gi & 1) ? (d[gi >> 1] & 0xFFFF0000u) : (d[gi >> 1] << 16));
  }
  __device__ __forceinline__ float f16(int gi) const {  // entry gi as an fp16 value
    return f16_to_f32((uint16_t)((gi & 1) ? (d[gi >> 1] >> 16) : d[gi >> 1]));
  }
};

template <int GPW>
struct Int4Slot {
  uint4 c[GPW];    // the lane's 16 code bytes of each group
  U16Run<GPW> s;   // bf16 scales of (row r, groups g0 .. g0 + GPW - 1)
};

template <int GPW, int P>
struct SignSlot {
  uint32_t w[GPW][P];  // the lane's sign dword of each (group, plane)
  U16Run<GPW> a[P];    // fp16 alphas of (plane, row r, groups g0 ..)
};

// One load of a run (scale rows are padded to a multiple of four entries,
// so the run is aligned to its own size).
template <int GPW>
__device__ __forceinline__ void load_u16_run(__amdgpu_buffer_rsrc_t r, uint32_t off, U16Run<GPW>& v) {
  if constexpr (GPW == 4) {
    const v2u_t t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    v.d[0] = t.x;
    v.d[1] = t.y;
  } else if constexpr (GPW == 2) {
    v.d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else {
    v.d[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  }
}

// Buffer views of one packed blob: weights (codes or sign planes) and scales.
struct BlobView {
  __amdgpu_buffer_rsrc_t w, s;
  int KT, KT4, NT;
};

__device__ __forceinline__ BlobView int4_view(const uint8_t* blob, int KT, int NT) {
  BlobView v;
  v.KT = KT;
  v.KT4 = (KT + 3) & ~3;
  v.NT = NT;
  const uint32_t wbytes = (uint32_t)NT * (uint32_t)KT * 1024u;
  v.w = make_rsrc(blob, wbytes);
  v.s = make_rsrc(blob + wbytes, (uint32_t)NT * 16u * (uint32_t)v.KT4 * 2u);
  return v;
}

__device__ __forceinline__ BlobView sign_view(const uint8_t* blob, int KT, int NT, int P) {
  BlobView v;
  v.KT = KT;
  v.KT4 = (KT + 3) & ~3;
  v.NT = NT;
  const uint32_t wbytes = (uint32_t)NT * (uint32_t)KT * 256u * (uint32_t)P;
  v.w = make_rsrc(blob, wbytes);
  v.s = make_rsrc(blob + wbytes, (uint32_t)P * (uint32_t)NT * 16u * (uint32_t)v.KT4 * 2u);
  return v;
}

// live: this tile is one of the workgroup's (else every load reads zero).
template <int GPW>
__device__ __forceinline__ void load_int4_tile(Int4Slot<GPW>& sl, const BlobView& b, int rt, bool live, int g0,
                                               int lane, int r) {
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = g0 + gi;
    const uint32_t off = (uint32_t)(rt * b.KT + g) * 1024u + 16u * lane;
    sl.c[gi] = ld_stream16(b.w, off | oob_bit(live && g < b.KT));
  }
  const uint32_t soff = ((uint32_t)(16 * rt + r) * b.KT4 + g0) * 2u;
  load_u16_run<GPW>(b.s, soff | oob_bit(live && g0 < b.KT4), sl.s);
}

template <int GPW, int P>
__device__ __forceinline__ void load_sign_tile(SignSlot<GPW, P>& sl, const BlobView& b, int rt, bool live, int g0,
                                               int lane, int r) {
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = g0 + gi;
    const uint32_t off = ((uint32_t)(rt * b.KT + g) * 256u * P + 4u * lane) | oob_bit(live && g < b.KT);
#pragma unroll
    for (int p = 0; p < P; ++p) sl.w[gi][p] = ld_stream4(b.w, off + 256u * p);
  }
  const int N16 = b.NT * 16;
  const uint32_t oob = oob_bit(live && g0 < b.KT4);
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const uint32_t aoff = ((uint32_t)(p * N16 + 16 * rt + r) * b.KT4 + g0) * 2u;
    load_u16_run<GPW>(b.s, aoff | oob, sl.a[p]);
  }
}

// sa* tiles.  The sign dwords are the plane blob's; a lane also reads, per
// plane, the run of u8 codes of its row over the wave's GPW column tiles
// (2, 1 or 1/2 codes per column tile for G = 64, 128, 256) and the fp16 d of
// the one or two super-blocks those tiles cover, each run with one load.
template <int GPW, int G>
constexpr int sa_code_bytes() { return GPW * 128 / G > 0 ? GPW * 128 / G : 1; }

template <int GPW, int P, int G>
struct SaSlot {
  uint32_t w[GPW][P];                                // sign dword of each (column tile, plane)
  uint32_t a[P][(sa_code_bytes<GPW, G>() + 3) / 4];  // raw code bytes of (plane, row r, the wave's groups)
  uint32_t d;                                        // raw fp16 d of the wave's super-blocks

  // Code of plane p for column tile gi, 32-wide k block t.  The wave's first
  // column tile g0 is a multiple of GPW, so its super-blocks and groups start
  // at the run's first byte.
  __device__ __forceinline__ uint32_t code(int p, int gi, int t) const {
    const int ci = G == 64 ? 2 * gi + (t >> 1) : G == 128 ? gi : gi >> 1;
    return (a[p][ci >> 2] >> (8 * (ci & 3))) & 0xFFu;
  }
  // d of the super-block holding column tile gi.
  __device__ __forceinline__ float dscale(int gi) const {
    return f16_to_f32((uint16_t)(d >> (16 * (gi >> 1))));
  }
};

template <int BYTES>
__device__ __forceinline__ void load_run(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t* v) {
  if constexpr (BYTES == 8) {
    const v2u_t t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    v[0] = t.x;
    v[1] = t.y;
  } else if constexpr (BYTES == 4) {
    v[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (BYTES == 2) {
    v[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  } else {
    v[0] = __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
  }
}

struct SaView {
  __amdgpu_buffer_rsrc_t w, a, d;
  int KT, KT4, NT;
};

template <int G>
__device__ __forceinline__ SaView sa_view(const uint8_t* blob, int KT, int NT, int P) {
  SaView v;
  v.KT = KT;
  v.KT4 = (KT + 3) & ~3;
  v.NT = NT;
  const uint32_t wbytes = (uint32_t)NT * (uint32_t)KT * 256u * (uint32_t)P;
  const uint32_t abytes = (uint32_t)P * (uint32_t)NT * 16u * (uint32_t)(v.KT4 * 128 / G);
  v.w = make_rsrc(blob, wbytes);
  v.a = make_rsrc(blob + wbytes, abytes);
  v.d = make_rsrc(blob + wbytes + abytes, (uint32_t)NT * 16u * (uint32_t)(v.KT4 / 2) * 2u);
  return v;
}

template <int GPW, int P, int G>
__device__ __forceinline__ void load_sa_tile(SaSlot<GPW, P, G>& sl, const SaView& b, int rt, bool live, int g0,
                                             int lane, int r) {
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = g0 + gi;
    const uint32_t off = ((uint32_t)(rt * b.KT + g) * 256u * P + 4u * lane) | oob_bit(live && g < b.KT);
#pragma unroll
    for (int p = 0; p < P; ++p) sl.w[gi][p] = ld_stream4(b.w, off + 256u * p);
  }
  const int N16 = b.NT * 16, CG = b.KT4 * 128 / G, row = 16 * rt + r;
  const uint32_t oob = oob_bit(live && g0 < b.KT4);
#pragma unroll
  for (int p = 0; p < P; ++p)
    load_run<sa_code_bytes<GPW, G>()>(b.a, ((uint32_t)((p * N16 + row) * CG + g0 * 128 / G)) | oob, sl.a[p]);
  load_run<GPW >= 4 ? 4 : 2>(b.d, ((uint32_t)(row * (b.KT4 / 2) + g0 / 2) * 2u) | oob, &sl.d);
}

// Activation staging for the full-register M <= 16 mat-muls (the lean
// shapes keep load_x_pairs above).  Loading xp directly
// gives the 16 lanes of a quarter-wave 16 different rows, i.e. 16 cache
// lines per quarter; instead a quarter-wave loads one row's 256 bytes
// of a column tile (lane: row 4 u + lane / 16, 16-byte chunk lane % 16), and
// the wave transposes through a private 4 KiB LDS region, one column tile at
// a time, with the chunks of row p XOR-swizzled by p mod 16 so that neither
// the writes nor the reads have bank conflicts.  Rows >= M and groups >= KT
// read zero (buffer range and offset bit 31).
template <int GPW>
struct XRows {
  uint4 v[GPW][4];
};

template <int GPW>
__device__ __forceinline__ void load_x_rows(const uint16_t* __restrict__ X, int M, int K, int g0, int KT, int lane,
                                            XRows<GPW>& xr) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
  const uint32_t lo = ((uint32_t)(lane >> 4) * (uint32_t)K + 8u * (lane & 15)) * 2u;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t off = (lo + (uint32_t)(4 * u) * (uint32_t)K * 2u + 256u * (g0 + gi)) | oob_bit(g0 + gi < KT);
      const v4u_t t = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
      xr.v[gi][u] = make_uint4(t.x, t.y, t.z, t.w);
    }
}

// Byte offset of 16-byte chunk c of row p in a transposition region of
// 256-byte rows (chunk index XOR-swizzled by the row).
__device__ __forceinline__ uint32_t xrow_chunk(int p, int c) { return (uint32_t)(p * 256 + ((c ^ (p & 15)) << 4)); }

template <int GPW>
__device__ __forceinline__ void transpose_x_rows(const XRows<GPW>& xr, uint4* region, int lane, int q, int r,
                                                 uint32_t (&xp)[GPW][16]) {
  char* base = reinterpret_cast<char*>(region);
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<uint4*>(base + xrow_chunk(4 * u + (lane >> 4), lane & 15)) = xr.v[gi][u];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 v = *reinterpret_cast<const uint4*>(base + xrow_chunk(r, 4 * t + q));
      xp[gi][4 * t + 0] = v.x;
      xp[gi][4 * t + 1] = v.y;
      xp[gi][4 * t + 2] = v.z;
      xp[gi][4 * t + 3] = v.w;
    }
  }
}

// Number of row tiles this workgroup owns in the grid-stride order.
__device__ __forceinline__ int tiles_of_wg(int NT) { return (NT - 1 - (int)blockIdx.x) / (int)gridDim.x + 1; }

// Row tile of the workgroup's i-th iteration.
__device__ __forceinline__ int row_tile(int i) { return blockIdx.x + i * gridDim.x; }

// Row tiles of an M <= 16 mat-mul workgroup.  With ms == 1 the grid walks
// the row tiles in grid-stride order (row_tile, tiles_of_wg).  With ms > 1
// one launch covers a block of 16 < M <= 64 rows as ms 16-row m-tiles:
// workgroup b computes m-tile (b / 8) % ms for the row tiles j, j + G / ms,
// ... (G workgroups, a multiple of 8 ms), j = b % 8 + 8 (b / (8 ms)).  The
// ms workgroups of one row-tile set then share b % 8, which round-robin
// dispatch places on one XCD, and run side by side, so the later readers of
// a weight tile find it in that XCD's L2.
struct TileWalk {
  int first, stride, mt;
  __device__ __forceinline__ int tile(int i) const { return first + i * stride; }
  __device__ __forceinline__ int count(int NT) const { return first < NT ? (NT - 1 - first) / stride + 1 : 0; }
};

__device__ __forceinline__ TileWalk tile_walk(int ms) {
  const int b = (int)blockIdx.x, c = b >> 3, g = (int)gridDim.x >> 3;  // dispatch rounds of 8 workgroups
  int cq, gq;  // c / ms and g / ms, by constant divisors (ms <= 4)
  switch (ms) {
    case 1: return TileWalk{b, (int)gridDim.x, 0};
    case 2: cq = c >> 1; gq = g >> 1; break;
    case 3: cq = c / 3; gq = g / 3; break;
    default: cq = c >> 2; gq = g >> 2; break;
  }
  return TileWalk{(b & 7) + 8 * cq, 8 * gq, c - cq * ms};
}

// ---------------------------------------------------------------------------
// M = 1 mat-vec cores.  Each returns the lane's partial sum for row r over its
// k sub-ranges of the wave's groups.  zc[g] (lane_zero_code_chains) is the
// group's chain on zero codes; subtracting it removes the +136 carried by
// every decoded code.
template <int GPW>
__device__ __forceinline__ float w4a16_tile_partial(const Int4Slot<GPW>& sl, const uint32_t (&xp)[GPW][16],
                                                    const float (&zc)[GPW], const PairDecode& magic) {
  float part = 0.f;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    uint32_t b[4][4];
    int4_pairs2(sl.c[gi].x, sl.c[gi].y, magic, b[0], b[1]);
    int4_pairs2(sl.c[gi].z, sl.c[gi].w, magic, b[2], b[3]);
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = dot2(b[t][i], xp[gi][4 * t + i], acc);
    part = fmaf(sl.s.bf16(gi), acc - zc[gi], part);
  }
  return part;
}

template <int GPW, int P>
__device__ __forceinline__ float binplane_tile_partial(const SignSlot<GPW, P>& sl, const uint32_t (&xp)[GPW][16],
                                                       const PairDecode& one) {
  float part = 0.f;
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float acc = 0.f;
#pragma unroll
      for (int ip = 0; ip < 16; ++ip) acc = dot2(sign_pair(sl.w[gi][p], ip, one), xp[gi][ip], acc);
      part = fmaf(sl.a[p].f16(gi), acc, part);
    }
  return part;
}

// bf16 pair (a, a) of a u8 scale code; exact, since a <= 255 has at most
// eight significant bits.
__device__ __forceinline__ uint32_t code_pair(uint32_t a) {
  const uint32_t h = __float_as_uint((float)a) >> 16;
  return h | (h << 16);
}

// bf16 pair (a * b_even, a * b_odd) for pair ip = 4t + i of a sign dword: the
// +-1 decode with the code pair in place of (1, 1).
__device__ __forceinline__ uint32_t scaled_sign_pair(uint32_t w, int ip, uint32_t mask, uint32_t apair) {
  return ((w << (15 - ip)) & mask) | apair;
}

// sa* lane partial with the weights decoded to a * b pairs: every plane and
// group of a super-block adds exact products a * b * x into one fp32 sum,
// which the super-block's d scales once.
template <int GPW, int P, int G>
__device__ __forceinline__ float sa_tile_partial(const SaSlot<GPW, P, G>& sl, const uint32_t (&xp)[GPW][16],
                                                 const PairDecode& one) {
  constexpr int SB = GPW >= 2 ? GPW / 2 : 1;
  float part = 0.f;
#pragma unroll
  for (int sb = 0; sb < SB; ++sb) {
    float acc = 0.f;
#pragma unroll
    for (int gi = 2 * sb; gi < 2 * sb + 2 && gi < GPW; ++gi)
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t ap = code_pair(sl.code(p, gi, t));
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc = dot2(scaled_sign_pair(sl.w[gi][p], 4 * t + i, one.mask, ap), xp[gi][4 * t + i], acc);
        }
    part = fmaf(sl.dscale(2 * sb), acc, part);
  }
  return part;
}

// ---------------------------------------------------------------------------
// Cross-wave combination.  The waves of a workgroup each own a slice of K,
// so every output of a tile needs one partial from every wave.  Partials
// wait in LDS and are combined once per chunk of C tiles, so the waves meet
// at one barrier per chunk.  The staging area is double-buffered (chunk k
// uses half k % 2): the barrier that ends chunk k + 1 also guarantees that
// every thread has finished reading half k % 2 before chunk k + 2 writes
// it.  A wave stages its partial at every loop step, also past the
// workgroup's last tile (into a discard slot), so the partial is computed
// before the next loads are issued rather than sunk into the branch that
// consumes it.
constexpr int kChunkGemv = 16;  // tiles per chunk, M = 1 kernels

// Tiles per chunk of the M <= 16 kernels (bounded by LDS: 1 KiB per wave and tile).
template <int MAXW>
constexpr int chunk_gemm() { return MAXW <= 8 ? 4 : 2; }

// The M <= 16 mat-muls' full-register forms (X loaded coalesced and
// transposed through LDS, interleaved MFMA chains, the one-instruction sign
// decode) need the activations of GPW column tiles and the ring in the
// registers of a wave: 256 a lane at eight waves.  The sixteen-wave shapes
// (K above 4096, four column tiles a wave, 128 registers a lane) use the
// lean forms.
template <int GPW, int MAXW>
constexpr bool mma_fast_shape() { return GPW * MAXW <= 32; }

template <class V, int C, int MAXW, int L>
struct ChunkStage {
  V buf[2 * C + 1][MAXW][L];  // [half * C + tile in chunk][wave][lane]; the last row discards

  __device__ __forceinline__ void put(int i, bool live, int wave, int lane, const V& v) {
    const int k = live ? ((i / C) & 1) * C + i % C : 2 * C;
    if (lane < L) buf[k][wave][lane] = v;
  }

  // Sum over the waves of tile c of the chunk that holds tile i, in wave
  // order.  With U > 1 the reads go out U at a time (nwaves is uniform), so
  // the sum waits for one LDS round trip per U waves instead of one per
  // wave.  The scalar partials of the eight-wave mat-vecs take all seven at
  // once; the mat-muls choose U by their register headroom (an unrolled
  // float4 read holds four registers until its add).
  template <int U = (sizeof(V) == sizeof(float) && MAXW <= 8) ? MAXW - 1 : 1>
  __device__ __forceinline__ V sum(int i, int c, int nwaves, int l) const {
    const int k = ((i / C) & 1) * C + c;
    V s = buf[k][0][l];
    if constexpr (U > 1) {
#pragma unroll
      for (int w0 = 1; w0 < MAXW; w0 += U) {
        V t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) t[u] = buf[k][w0 + u < nwaves ? w0 + u : 0][l];  // nwaves <= MAXW
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (w0 + u < nwaves) s += t[u];
      }
    } else {
      for (int w = 1; w < nwaves; ++w) s += buf[k][w][l];
    }
    return s;
  }
};

// ---------------------------------------------------------------------------
// lmhead_argmax completion.  A (logit, row) pair becomes one 64-bit key whose
// unsigned order is the greedy order: the high word is the logit's bits
// mapped so that unsigned comparison follows float comparison, the low word
// is 2^32 - 1 - row, so a larger logit wins and the lower row wins a tie.
// Device-scope atomics on one address are performed one after another, so
// when all 256 workgroups of a launch finish together, a single key and
// counter for all of them cost about 2.9 us over an empty launch (MI355X,
// measured); meeting in two levels, 16 groups and then the groups, costs
// about 1.2 us there but adds a dependent round trip, which costs more than
// it saves when the workgroups' completions are spread out (many tiles
// each).  HeadOut::levels, uniform over the launch, selects the form.  In
// two levels workgroup b belongs to group b mod 16; in one level all are in
// group 0.  A workgroup folds its per-query-row best into its group's keys
// with device-scope atomicMax, waits for the atomics to complete, and bumps
// its group's counter; in two levels the group's last workgroup clears that
// counter and bumps the launch counter.  The launch's last workgroup takes
// every group's keys with atomic exchanges against zero (all at once, one
// per thread), keeps the largest per row, writes the outputs and clears the
// launch counter.  Keys and counters are only ever touched by
// device-scope read-modify-write atomics, which every XCD performs at the
// same point of coherence, and each step is issued only after the step
// before it has returned, so no cache-wide fence is needed.  A max does not
// depend on the order of its operands, so neither does the result.
constexpr int kWaitVmcnt0 = 0x0F70;  // s_waitcnt vmcnt(0) expcnt(7) lgkmcnt(15)
constexpr int kWsGroups = 16;
constexpr int kWsKeys = 0;                         // [group][16] uint64 keys, one 128-byte line a group
constexpr int kWsGroupCounters = kWsGroups * 128;  // uint32 a group, one 128-byte line each
constexpr int kWsCounter = 2 * kWsGroups * 128;    // uint32 launch counter
constexpr int kWsBytes = kWsCounter + 256;

__device__ __forceinline__ unsigned long long argmax_key(float v, int n) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)n);
}

// Where a head launch leaves its results (all device pointers; see svq.h).
// draft and accept are set only by lmhead_verify_greedy.
struct HeadOut {
  const int32_t* row_ids;  // NULL or [N] row -> token id
  int32_t* idx;            // [M] greedy token per query row
  float* max;              // [M] its logit
  const int32_t* draft;    // NULL or [M - 1] drafted tokens d_1 .. d_{M-1}
  int32_t* accept;         // [1] tau, when draft is set
  int levels;              // argmax completion in one level (all workgroups) or two (16 groups)
};

// Greedy acceptance of a verified block (DFlash summary sec. 4.1): query row
// m of the block [anchor, d_1, ..., d_{M-1}] predicts the token after
// position m, so d_{j+1} is accepted while every earlier draft was accepted
// and t_j == d_{j+1}.  tau = accepted + 1: the accepted drafts plus the
// target's own next token, i.e. t_0 .. t_{tau-1}.  A row without a valid
// maximum (id -1) ends the accepted prefix.
__device__ __forceinline__ int greedy_accept_len(const int32_t* t, const int32_t* __restrict__ draft, int M) {
  int a = 0;
  while (a < M - 1 && t[a] >= 0 && t[a] == draft[a]) ++a;
  return a + 1;
}

__device__ __forceinline__ void argmax_complete(unsigned long long key, bool holds_row, int m, uint8_t* ws, int M,
                                                int N, const HeadOut& ho) {
  unsigned long long* keys = reinterpret_cast<unsigned long long*>(ws + kWsKeys);
  unsigned* group_counter = reinterpret_cast<unsigned*>(ws + kWsGroupCounters);
  unsigned* counter = reinterpret_cast<unsigned*>(ws + kWsCounter);
  const bool split = ho.levels > 1;
  const int grp = split ? (int)(blockIdx.x % kWsGroups) : 0;
  const int ngroups = !split ? 1 : gridDim.x < (unsigned)kWsGroups ? (int)gridDim.x : kWsGroups;
  if (holds_row) {
    atomicMax(&keys[16 * grp + m], key);
    // Wait until the atomic has completed before the counter increment
    // below can be issued (vmcnt(0); the other counters are left free).
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }
  __syncthreads();
  __shared__ int last;
  if (threadIdx.x == 0) {
    int l = 0;
    if (!split) {
      l = atomicAdd(counter, 1u) == gridDim.x - 1;
    } else if (atomicAdd(&group_counter[32 * grp], 1u) == (gridDim.x - 1 - grp) / kWsGroups) {
      // The group's last member (the group has (gridDim.x - 1 - grp) / 16 + 1).
      atomicExch(&group_counter[32 * grp], 0u);
      l = atomicAdd(counter, 1u) == (unsigned)ngroups - 1;
    }
    last = l;
  }
  __syncthreads();
  if (!last) return;
  __shared__ unsigned long long group_keys[kWsGroups][SVQ_MAX_M];
  for (int t = threadIdx.x; t < ngroups * M; t += blockDim.x)
    group_keys[t / M][t % M] = atomicExch(&keys[16 * (t / M) + t % M], 0ull);
  __syncthreads();
  __shared__ int32_t ids[SVQ_MAX_M];
  if ((int)threadIdx.x < M) {
    unsigned long long k = 0ull;
    for (int g = 0; g < ngroups; ++g) k = group_keys[g][threadIdx.x] > k ? group_keys[g][threadIdx.x] : k;
    const uint32_t o = (uint32_t)(k >> 32);
    const int n = (int)(0xFFFFFFFFu - (uint32_t)k);
    // key 0 means no row compared above it: every logit of the row was NaN.
    const bool found = k != 0ull && n >= 0 && n < N;
    const uint32_t u = (o & 0x80000000u) ? (o ^ 0x80000000u) : ~o;
    const int32_t id = !found ? -1 : ho.row_ids ? ho.row_ids[n] : n;
    ho.idx[threadIdx.x] = id;
    ho.max[threadIdx.x] = found ? __uint_as_float(u) : __builtin_nanf("");
    ids[threadIdx.x] = id;
  }
  if (threadIdx.x == 0) atomicExch(counter, 0u);
  if (ho.accept) {
    __syncthreads();  // the whole completing workgroup takes this branch
    if (threadIdx.x == 0) ho.accept[0] = greedy_accept_len(ids, ho.draft, M);
  }
}

// M = 1 heads: combines the threads' running bests (lowest index wins ties)
// and completes the launch's argmax.
template <int MAXW>
__device__ __forceinline__ void gemv_argmax_epilogue(float best_v, int best_i, int wave, int lane, int nwaves,
                                                     uint8_t* ws, int N, const HeadOut& ho) {
  __shared__ ArgBest part[MAXW];
  best_over_wave(best_v, best_i);
  if (lane == 0) part[wave] = ArgBest{best_v, best_i};
  __syncthreads();
  if (threadIdx.x == 0) {
    // Up to eight waves, every wave's entry is read at once (unrolled over
    // MAXW; nwaves is uniform), then folded in wave order.
    constexpr int U = MAXW <= 8 ? MAXW : 1;
    ArgBest t[U];
#pragma unroll
    for (int w = 0; w < U; ++w) t[w] = part[w < nwaves ? w : 0];
#pragma unroll
    for (int w = 1; w < U; ++w)
      if (w < nwaves && better(t[w].v, t[w].idx, best_v, best_i)) {
        best_v = t[w].v;
        best_i = t[w].idx;
      }
    for (int w = U; w < nwaves; ++w)
      if (better(part[w].v, part[w].idx, best_v, best_i)) {
        best_v = part[w].v;
        best_i = part[w].idx;
      }
  }
  argmax_complete(argmax_key(best_v, best_i), threadIdx.x == 0 && best_i < N, 0, ws, 1, N, ho);
}

// ---------------------------------------------------------------------------
// gemv_w4a16 / lmhead (M = 1).  ARGMAX selects the epilogue.
template <int GPW, int MAXW, int D, bool ARGMAX>
__global__ void __launch_bounds__(64 * MAXW)
    k_gemv_w4a16(const uint8_t* __restrict__ blob, const uint32_t* __restrict__ xw, uint16_t* __restrict__ y,
                 uint8_t* __restrict__ ws, HeadOut ho, int N, int KT, int NT) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int g0 = wave * GPW;
  const BlobView bv = int4_view(blob, KT, NT);
  const int T = tiles_of_wg(NT);

  uint32_t xo[GPW];
  load_x_own<GPW>(xw, g0, KT, q, r, xo);
  // The activation loads go out first: the first tile's work waits on them.
  __builtin_amdgcn_sched_barrier(0);
  Int4Slot<GPW> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    load_int4_tile<GPW>(ring[j], bv, row_tile(j), j < T, g0, lane, r);
    // Issue each slot's loads in the same order the loop refills them.
    __builtin_amdgcn_sched_barrier(0);
  }
  // Keep the whole prefetch issued before anything waits on the activations.
  __builtin_amdgcn_sched_barrier(0);
  __shared__ ChunkStage<float, kChunkGemv, MAXW, 16> stage;
  uint32_t xp[GPW][16];
  expand_x<GPW>(xo, xp);
  float zc[GPW];
  lane_zero_code_chains<GPW>(xp, zc);
  const PairDecode magic = int4_decode();

  float best_v = -FLT_MAX;
  int best_i = INT_MAX;
  int i0 = 0;
  auto step = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const int i = i0 + j;
    const float part = sum_over_q(w4a16_tile_partial<GPW>(ring[j], xp, zc, magic));
    stage.put(i, i < T, wave, lane, part);
    // Slot j is refilled only after its last use, so it keeps its registers.
    __builtin_amdgcn_sched_barrier(0);
    load_int4_tile<GPW>(ring[j], bv, row_tile(i + D), i + D < T, g0, lane, r);
    const int ci = i % kChunkGemv;
    if (i < T && (ci == kChunkGemv - 1 || i == T - 1)) {
      __syncthreads();
      const int first = i - ci;
      // Output o = 16c + row of the chunk; a thread meets the same c in
      // every chunk, so its rows arrive in increasing n.
      for (int o = threadIdx.x; o < (ci + 1) * 16; o += nwaves * 64) {
        const float v = stage.sum(i, o >> 4, nwaves, o & 15);
        const int n = 16 * row_tile(first + (o >> 4)) + (o & 15);
        if (n < N) {
          if constexpr (ARGMAX) {
            if (v > best_v) {
              best_v = v;
              best_i = n;
            }
          } else {
            y[n] = f32_to_bf16_rne(v);
          }
        }
      }
    }
  };
  // Whole rounds of the ring, then the tiles of a partial last round (held in
  // the ring's first slots) one by one, so no step runs on an empty tile:
  // the workgroups that own one tile more than the rest finish last, and at
  // an odd count a step on an empty tile was on that path (0.7% of the
  // 248320-row heads, measured).  A uniform early exit inside the round
  // slowed every launch instead.  Every workgroup owns at least one tile
  // (grid <= number of tiles).
  const int whole = T - T % D;
  for (; i0 < whole; i0 += D) static_for<0, D>(step);
  static_for<0, D - 1>([&](auto jc) {
    if (decltype(jc)::value < T - whole) step(jc);
  });
  if constexpr (ARGMAX) gemv_argmax_epilogue<MAXW>(best_v, best_i, wave, lane, nwaves, ws, N, ho);
}

// Sign-nibble lookup tables for the M = 1 sign-plane kernel.  In a sign
// dword, the bits of k-block t form two nibbles: bits 4t..4t+3 hold the signs
// of the lane's even k's (32t + 8q + 2i) and bits 16+4t..16+4t+3 those of its
// odd k's (+1).  For every (group, t, parity) the table holds, for each of
// the 16 nibble values v, the sum over i of (bit i of v set ? -x : +x) over
// those four activations, so a plane's sum over 128 k is eight table reads
// instead of 64 sign decodes and 64 multiply-adds.  Every wave builds and
// reads only its own tables, so no barrier is needed.  In a read, the 16
// lanes of a row q address the 16 consecutive entries of one table and the
// four rows use disjoint 16-bank ranges, so a read is free of bank
// conflicts.  Table (group, t, parity) holds entry v of row q at word
// base + 16 q + v; its base is shifted by 4 t words from the 64-word grid,
// so that the 16-byte stores of a table build, where the 16 lanes of a pass
// write four entries of the four rows of four blocks t, meet 16 distinct
// bank quads (on the plain grid they met four, four stores to each).  A
// group's eight tables then span 8 x 64 + 12 words; groups are 528 words
// apart, and the size is rounded up to a multiple of 256 bytes: a wave's
// tables start at a multiple of 256, whose low bits the read addresses fill
// by OR.
template <int GPW>
struct SignLut {
  static constexpr int kGroupWords = 8 * 64 + 16;
  float e[(GPW * kGroupWords + 63) / 64 * 64];
  static constexpr int base(int gi, int t, int par) { return kGroupWords * gi + 64 * (2 * t + par) + 4 * t; }
};

// The tables are built on the matrix cores, from the activations as loaded
// (lane (q, r) holds the pair (t = r / 4, i = r % 4) of its row q, see
// load_x_own).  For one group and parity the 256 entries of its four k
// blocks and four rows are one 16 x 16 product D = S B over 32 k slots
// (8 h + 2 i + p: lane row h, pair i, half p):
//   S[v][k] = (p == parity) ? (bit i of v set ? -1 : +1) : 0
//   B[k][n] = x of row n % 4, block n / 4, pair i, half p  if h == n % 4, else 0
// so D[v][n] is entry v of table (block n / 4, row n % 4).  The B operand of
// lane (q, r) is the four pairs of its own quad (a DPP quad broadcast each),
// kept where r % 4 == q and zero elsewhere; every product is exact and each
// entry sums four of them in fp32.  Per wave: 8 MFMAs and 32 VALU
// instructions (one dot2 chain per entry took 128 instructions, plus 64
// moves to spread the activations over the row).  Lane (q, r) receives
// entries 4q .. 4q + 3 of table (r / 4, r % 4) and writes them as one
// 16-byte store.
template <int GPW>
__device__ __forceinline__ void build_sign_lut(SignLut<GPW>& lut, const uint32_t (&xo)[GPW], int q, int r) {
  uint32_t s0[4], s1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s0[i] = ((r >> i) & 1) ? 0xBF80u : 0x3F80u;
    s1[i] = s0[i] << 16;
  }
  const bool own = (r & 3) == q;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    uint32_t b[4];
    b[0] = __builtin_amdgcn_mov_dpp(xo[gi], 0x00, 0xF, 0xF, false);  // quad_perm [0, 0, 0, 0]
    b[1] = __builtin_amdgcn_mov_dpp(xo[gi], 0x55, 0xF, 0xF, false);  // quad_perm [1, 1, 1, 1]
    b[2] = __builtin_amdgcn_mov_dpp(xo[gi], 0xAA, 0xF, 0xF, false);  // quad_perm [2, 2, 2, 2]
    b[3] = __builtin_amdgcn_mov_dpp(xo[gi], 0xFF, 0xF, 0xF, false);  // quad_perm [3, 3, 3, 3]
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = own ? b[i] : 0u;
    const f32x4_t e0 = mfma16x16x32(s0, b, zero);
    const f32x4_t e1 = mfma16x16x32(s1, b, zero);
    float* row = &lut.e[SignLut<GPW>::base(gi, r >> 2, 0) + 16 * (r & 3) + 4 * q];
    *reinterpret_cast<float4*>(row) = make_float4(e0[0], e0[1], e0[2], e0[3]);
    *reinterpret_cast<float4*>(row + 64) = make_float4(e1[0], e1[1], e1[2], e1[3]);  // parity 1: the next table
  }
}

// ((w >> shift) & 15) * 4: a nibble as the byte offset of a table entry.
__device__ __forceinline__ uint32_t nibble_offset(uint32_t w, int shift) {
  return shift >= 2 ? (w >> (shift - 2)) & 0x3Cu : (w << (2 - shift)) & 0x3Cu;
}

// Byte offsets ((w >> (4 j - 2)) & 0x3C) | lane_off of the eight nibbles j
// of two sign dwords: one 64-bit shift of the pair hi:lo places nibble j of
// both dwords at bits 2-5 (the bits shifted in from the other dword land
// outside the mask), and a 64-bit shift issues at about the cost of a 32-bit
// one.
__device__ __forceinline__ void nibble_offsets2(uint32_t lo, uint32_t hi, uint32_t lane_off, uint32_t (&ol)[8],
                                                uint32_t (&oh)[8]) {
  const uint64_t w = (uint64_t)hi << 32 | lo;
  uint64_t s[8];
  asm("v_lshlrev_b64 %0, 2, %1" : "=v"(s[0]) : "v"(w));
  asm("v_lshrrev_b64 %0, 2, %1" : "=v"(s[1]) : "v"(w));
  asm("v_lshrrev_b64 %0, 6, %1" : "=v"(s[2]) : "v"(w));
  asm("v_lshrrev_b64 %0, 10, %1" : "=v"(s[3]) : "v"(w));
  asm("v_lshrrev_b64 %0, 14, %1" : "=v"(s[4]) : "v"(w));
  asm("v_lshrrev_b64 %0, 18, %1" : "=v"(s[5]) : "v"(w));
  asm("v_lshrrev_b64 %0, 22, %1" : "=v"(s[6]) : "v"(w));
  asm("v_lshrrev_b64 %0, 26, %1" : "=v"(s[7]) : "v"(w));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ol[j] = ((uint32_t)s[j] & 0x3Cu) | lane_off;
    oh[j] = ((uint32_t)(s[j] >> 32) & 0x3Cu) | lane_off;
  }
}

// The same offsets for one dword.
__device__ __forceinline__ void nibble_offsets1(uint32_t w, uint32_t lane_off, uint32_t (&o)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = nibble_offset(w, 4 * j) | lane_off;
}

// Offsets of the sign dwords u0 and u0 + 1 of a run (o1 unused when the run
// ends at u0).
template <int U, class W>
__device__ __forceinline__ void nibble_offsets_at(W&& w, int u0, uint32_t lane_off, uint32_t (&o0)[8],
                                                  uint32_t (&o1)[8]) {
  if (u0 + 1 < U) nibble_offsets2(w(u0), w(u0 + 1), lane_off, o0, o1);
  else nibble_offsets1(w(u0), lane_off, o0);
}

// Lane's partial for row r over its k sub-ranges of the wave's groups, all
// planes: sum_p alpha_p * (eight table reads per group).  lane_off is the
// byte offset of the lane's table row (wave's tables + 64 q); the nibble's
// offset has disjoint bits, so one AND-OR forms each address and the
// (group, t, parity) part is the read's constant offset.  Nibble j = 4
// parity + t of a dword holds the signs of block t, parity.
template <int GPW, int P>
__device__ __forceinline__ float binplane_tile_partial_lut(const SignSlot<GPW, P>& sl, const SignLut<GPW>* luts,
                                                           uint32_t lane_off) {
  const char* base = reinterpret_cast<const char*>(luts);
  auto sum8 = [&](int gi, const uint32_t (&o)[8]) {
    float acc;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const float v = *reinterpret_cast<const float*>(base + o[4 * par + t] + 4 * SignLut<GPW>::base(gi, t, par));
        acc = (t == 0 && par == 0) ? v : acc + v;
      }
    return acc;
  };
  // The (group, plane) dwords in order u = gi P + p, two at a time.
  constexpr int U = GPW * P;
  float part = 0.f;
#pragma unroll
  for (int u = 0; u < U; u += 2) {
    uint32_t o0[8], o1[8];
    nibble_offsets_at<U>([&](int v) { return sl.w[v / P][v % P]; }, u, lane_off, o0, o1);
    part = fmaf(sl.a[u % P].f16(u / P), sum8(u / P, o0), part);
    if (u + 1 < U) part = fmaf(sl.a[(u + 1) % P].f16((u + 1) / P), sum8((u + 1) / P, o1), part);
  }
  return part;
}

// sa* counterpart: per plane the two halves of a column tile (k blocks 0-1
// and 2-3) are summed apart, so that at G = 64 each takes its own code; the
// codes weight the table sums and d scales each super-block once.
template <int GPW, int P, int G>
__device__ __forceinline__ float sa_tile_partial_lut(const SaSlot<GPW, P, G>& sl, const SignLut<GPW>* luts,
                                                     uint32_t lane_off) {
  const char* base = reinterpret_cast<const char*>(luts);
  constexpr int SB = GPW >= 2 ? GPW / 2 : 1;
  constexpr int GB = GPW >= 2 ? 2 : 1;  // column tiles of a super-block held by the wave
  constexpr int U = GB * P;
  // Table sums of column tile gi, plane p, folded into the super-block sum.
  auto fold = [&](int gi, int p, const uint32_t (&o)[8], float& acc) {
    float h[2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const float v = *reinterpret_cast<const float*>(base + o[4 * par + t] + 4 * SignLut<GPW>::base(gi, t, par));
        h[t >> 1] = ((t & 1) == 0 && par == 0) ? v : h[t >> 1] + v;
      }
    if constexpr (G == 64) {
      acc = fmaf((float)sl.code(p, gi, 0), h[0], acc);
      acc = fmaf((float)sl.code(p, gi, 2), h[1], acc);
    } else {
      acc = fmaf((float)sl.code(p, gi, 0), h[0] + h[1], acc);
    }
  };
  float part = 0.f;
#pragma unroll
  for (int sb = 0; sb < SB; ++sb) {
    float acc = 0.f;
    // The super-block's (column tile, plane) dwords in order, two at a time.
#pragma unroll
    for (int u = 0; u < U; u += 2) {
      uint32_t o0[8], o1[8];
      nibble_offsets_at<U>([&](int v) { return sl.w[GB * sb + v / P][v % P]; }, u, lane_off, o0, o1);
      fold(GB * sb + u / P, u % P, o0, acc);
      if (u + 1 < U) fold(GB * sb + (u + 1) / P, (u + 1) % P, o1, acc);
    }
    part = fmaf(sl.dscale(2 * sb), acc, part);
  }
  return part;
}

// ---------------------------------------------------------------------------
// Sign-plane storages.  Both share the sign section and the two kernels
// below; a format names its tile registers (Slot), its buffer views, the
// loads of one tile and the tile's arithmetic: the M = 1 lane partial (from
// the nibble tables or from decoded pairs) and the M <= 16 MFMA tile.

// fp16 alpha per (plane, row, group of 128).
template <int P_>
struct PlaneFmt {
  static constexpr int P = P_;
  template <int GPW>
  using Slot = SignSlot<GPW, P>;
  using View = BlobView;

  static __device__ __forceinline__ View view(const uint8_t* blob, int KT, int NT) {
    return sign_view(blob, KT, NT, P);
  }
  template <int GPW>
  static __device__ __forceinline__ void load(Slot<GPW>& sl, const View& b, int rt, bool live, int g0, int lane,
                                              int r) {
    load_sign_tile<GPW, P>(sl, b, rt, live, g0, lane, r);
  }
  template <int GPW>
  static __device__ __forceinline__ float partial_lut(const Slot<GPW>& sl, const SignLut<GPW>* luts,
                                                      uint32_t lane_off) {
    return binplane_tile_partial_lut<GPW, P>(sl, luts, lane_off);
  }
  template <int GPW>
  static __device__ __forceinline__ float partial(const Slot<GPW>& sl, const uint32_t (&xp)[GPW][16],
                                                  const PairDecode& one) {
    return binplane_tile_partial<GPW, P>(sl, xp, one);
  }
  // MFMA tiles.  Full-register shapes (mma_fast_shape): the activations
  // with the pairs at the +-1 positions negated, and per group the chain
  // start -(sum x + sum c x) of the rows 4q + i this lane's results hold
  // (see plane_operands).  The lean shapes keep the two instructions per
  // pair of sign_pair and chains started at zero.
  template <int GPW>
  struct MmaFast {
    f32x4_t cinit[GPW];
    PlaneDecode d;
  };
  struct MmaLean {
    PairDecode one;
  };
  template <int GPW, int MAXW>
  using MmaX = std::conditional_t<mma_fast_shape<GPW, MAXW>(), MmaFast<GPW>, MmaLean>;

  template <int GPW, int MAXW>
  static __device__ __forceinline__ void prepare_mma(uint32_t (&xa)[GPW][16], int q, MmaX<GPW, MAXW>& mx) {
    if constexpr (mma_fast_shape<GPW, MAXW>()) {
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        xa[gi][11] ^= 0x80008000u;
        xa[gi][15] ^= 0x80008000u;
      }
      f32x4_t cs[GPW][2];
      plane_chain_starts<GPW, 1>(xa, cs);
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) mx.cinit[gi] = cs[gi][0];
      mx.d = plane_decode();
    } else {
      mx.one = sign_decode();
    }
  }
  // One accumulator chain per (column tile, plane), scaled by its alpha.  In
  // the fast form each chain ends at minus the plane's signed sum, so the
  // weighted total is negated once, and a plane's chains over the wave's
  // column tiles are interleaved k block by k block (consecutive MFMAs are
  // independent).
  template <int GPW, int MAXW>
  static __device__ __forceinline__ float4 mma(const Slot<GPW>& sl, const uint32_t (&xa)[GPW][16],
                                               const MmaX<GPW, MAXW>& mx) {
    float4 yv = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (mma_fast_shape<GPW, MAXW>()) {
      if constexpr (P <= 4) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          PlaneViews v[GPW];
          f32x4_t c[GPW];
          plane_views_n<GPW>([&](int gi) { return sl.w[gi][p]; }, v);
#pragma unroll
          for (int gi = 0; gi < GPW; ++gi) c[gi] = mx.cinit[gi];
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int gi = 0; gi < GPW; ++gi) {
              uint32_t b[4];
              plane_operands_t(v[gi], t, mx.d, b);
              c[gi] = mfma16x16x32(&xa[gi][4 * t], b, c[gi]);
            }
#pragma unroll
          for (int gi = 0; gi < GPW; ++gi) {
            const float a = sl.a[p].f16(gi);
            yv.x = fmaf(a, c[gi][0], yv.x);
            yv.y = fmaf(a, c[gi][1], yv.y);
            yv.z = fmaf(a, c[gi][2], yv.z);
            yv.w = fmaf(a, c[gi][3], yv.w);
          }
        }
      } else {
        // Five or six planes: the tile's registers leave no room for
        // interleaved chains, so each (column tile, plane) runs its own.
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
          for (int p = 0; p < P; ++p) {
            uint32_t b[4][4];
            plane_operands(sl.w[gi][p], mx.d, b);
            f32x4_t c = mx.cinit[gi];
#pragma unroll
            for (int t = 0; t < 4; ++t) c = mfma16x16x32(&xa[gi][4 * t], b[t], c);
            const float a = sl.a[p].f16(gi);
            yv.x = fmaf(a, c[0], yv.x);
            yv.y = fmaf(a, c[1], yv.y);
            yv.z = fmaf(a, c[2], yv.z);
            yv.w = fmaf(a, c[3], yv.w);
          }
      }
      return make_float4(-yv.x, -yv.y, -yv.z, -yv.w);
    } else {
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const uint32_t wp = sl.w[gi][p];
          f32x4_t c = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t bq[4] = {sign_pair(wp, 4 * t + 0, mx.one), sign_pair(wp, 4 * t + 1, mx.one),
                                    sign_pair(wp, 4 * t + 2, mx.one), sign_pair(wp, 4 * t + 3, mx.one)};
            c = mfma16x16x32(&xa[gi][4 * t], bq, c);
          }
          const float a = sl.a[p].f16(gi);
          yv.x = fmaf(a, c[0], yv.x);
          yv.y = fmaf(a, c[1], yv.y);
          yv.z = fmaf(a, c[2], yv.z);
          yv.w = fmaf(a, c[3], yv.w);
        }
      return yv;
    }
  }

  // Two 16-row m-tiles at once (the 17..32-row form, full-register shapes,
  // P <= 4): every decoded operand feeds both m-tiles' chains, so the
  // weights are read and decoded once for the 32 rows.  Chains are
  // interleaved over IL column tiles (two, so that both m-tiles' chains fit
  // beside the two blocks of activations).
  template <int GPW>
  struct Mma2 {
    f32x4_t cinit[2][GPW];
    PlaneDecode d;
  };
  template <int GPW>
  static __device__ __forceinline__ void prepare_mma2(uint32_t (&xa)[2][GPW][16], Mma2<GPW>& mx) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        xa[mt][gi][11] ^= 0x80008000u;
        xa[mt][gi][15] ^= 0x80008000u;
      }
      f32x4_t cs[GPW][2];
      plane_chain_starts<GPW, 1>(xa[mt], cs);
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) mx.cinit[mt][gi] = cs[gi][0];
    }
    mx.d = plane_decode();
  }
  template <int GPW>
  static __device__ __forceinline__ void mma2(const Slot<GPW>& sl, const uint32_t (&xa)[2][GPW][16],
                                              const Mma2<GPW>& mx, float4 (&yv)[2]) {
    static_assert(P <= 4, "two m-tiles hold the operands of up to four planes");
    constexpr int IL = GPW < 2 ? GPW : 2;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) yv[mt] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int g0c = 0; g0c < GPW; g0c += IL) {
        PlaneViews v[IL];
        f32x4_t c[2][IL];
        plane_views_n<IL>([&](int u) { return sl.w[g0c + u][p]; }, v);
#pragma unroll
        for (int u = 0; u < IL; ++u) {
          c[0][u] = mx.cinit[0][g0c + u];
          c[1][u] = mx.cinit[1][g0c + u];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int u = 0; u < IL; ++u) {
            uint32_t b[4];
            plane_operands_t(v[u], t, mx.d, b);
            c[0][u] = mfma16x16x32(&xa[0][g0c + u][4 * t], b, c[0][u]);
            c[1][u] = mfma16x16x32(&xa[1][g0c + u][4 * t], b, c[1][u]);
          }
#pragma unroll
        for (int u = 0; u < IL; ++u) {
          const float a = sl.a[p].f16(g0c + u);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            yv[mt].x = fmaf(a, c[mt][u][0], yv[mt].x);
            yv[mt].y = fmaf(a, c[mt][u][1], yv[mt].y);
            yv[mt].z = fmaf(a, c[mt][u][2], yv[mt].z);
            yv[mt].w = fmaf(a, c[mt][u][3], yv[mt].w);
          }
        }
      }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) yv[mt] = make_float4(-yv[mt].x, -yv[mt].y, -yv[mt].z, -yv[mt].w);
  }
};

// sa*: u8 codes per (plane, row, group of G) and one fp16 d per (row,
// super-block).  In the MFMA tile, B holds a * b exactly, so all planes and
// groups of a super-block accumulate in one chain that d scales once.
template <int P_, int G>
struct SaFmt {
  static constexpr int P = P_;
  template <int GPW>
  using Slot = SaSlot<GPW, P, G>;
  using View = SaView;

  static __device__ __forceinline__ View view(const uint8_t* blob, int KT, int NT) {
    return sa_view<G>(blob, KT, NT, P);
  }
  template <int GPW>
  static __device__ __forceinline__ void load(Slot<GPW>& sl, const View& b, int rt, bool live, int g0, int lane,
                                              int r) {
    load_sa_tile<GPW, P, G>(sl, b, rt, live, g0, lane, r);
  }
  template <int GPW>
  static __device__ __forceinline__ float partial_lut(const Slot<GPW>& sl, const SignLut<GPW>* luts,
                                                      uint32_t lane_off) {
    return sa_tile_partial_lut<GPW, P, G>(sl, luts, lane_off);
  }
  template <int GPW>
  static __device__ __forceinline__ float partial(const Slot<GPW>& sl, const uint32_t (&xp)[GPW][16],
                                                  const PairDecode& one) {
    return sa_tile_partial<GPW, P, G>(sl, xp, one);
  }
  // MFMA tiles.  Full-register shapes: the sign decode of PlaneFmt (one AND-OR
  // per pair, chains ending at minus each plane's signed sum over a group,
  // or over each half of a group at G = 64, where the two halves take their
  // own codes), each chain weighted by its code and the super-block's sum by
  // d.  The lean shapes keep the B = a * b pairs: there every plane and
  // group of a super-block accumulates in one chain that d scales once (a
  // code a <= 255 is exact in bf16, so a * b * x is an exact product).
  template <int GPW>
  struct MmaFast {
    f32x4_t cinit[GPW][G == 64 ? 2 : 1];
    PlaneDecode d;
  };
  struct MmaLean {
    PairDecode one;
  };
  template <int GPW, int MAXW>
  using MmaX = std::conditional_t<mma_fast_shape<GPW, MAXW>(), MmaFast<GPW>, MmaLean>;

  template <int GPW, int MAXW>
  static __device__ __forceinline__ void prepare_mma(uint32_t (&xa)[GPW][16], int q, MmaX<GPW, MAXW>& mx) {
    if constexpr (mma_fast_shape<GPW, MAXW>()) {
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        xa[gi][11] ^= 0x80008000u;
        xa[gi][15] ^= 0x80008000u;
      }
      f32x4_t cs[GPW][2];
      plane_chain_starts<GPW, G == 64 ? 2 : 1>(xa, cs);
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi)
#pragma unroll
        for (int h = 0; h < (G == 64 ? 2 : 1); ++h) mx.cinit[gi][h] = cs[gi][h];
      mx.d = plane_decode();
    } else {
      mx.one = sign_decode();
    }
  }
  template <int GPW, int MAXW>
  static __device__ __forceinline__ float4 mma(const Slot<GPW>& sl, const uint32_t (&xa)[GPW][16],
                                               const MmaX<GPW, MAXW>& mx) {
    constexpr int SB = GPW >= 2 ? GPW / 2 : 1;
    float4 yv = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (mma_fast_shape<GPW, MAXW>() && P <= 4 && G != 64) {
      // Up to four planes at G >= 128: a plane's chains over the wave's
      // column tiles are interleaved k block by k block, so consecutive
      // MFMAs are independent.  (At G = 64 the halves double the chains and
      // the codes the slot, and the interleaved form spills registers.)
      constexpr int H = 1;
      constexpr int IL = GPW;
      float4 ys[SB];
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) ys[sb] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int g0c = 0; g0c < GPW; g0c += IL)
#pragma unroll
        for (int p = 0; p < P; ++p) {
          PlaneViews v[IL];
          f32x4_t c[IL][H];
          plane_views_n<IL>([&](int u) { return sl.w[g0c + u][p]; }, v);
#pragma unroll
          for (int u = 0; u < IL; ++u) {
#pragma unroll
            for (int h = 0; h < H; ++h) c[u][h] = mx.cinit[g0c + u][h];
          }
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int u = 0; u < IL; ++u) {
              uint32_t b[4];
              plane_operands_t(v[u], t, mx.d, b);
              c[u][H == 2 ? t >> 1 : 0] = mfma16x16x32(&xa[g0c + u][4 * t], b, c[u][H == 2 ? t >> 1 : 0]);
            }
#pragma unroll
          for (int u = 0; u < IL; ++u)
#pragma unroll
            for (int h = 0; h < H; ++h) {
              const int gi = g0c + u;
              const float a = (float)sl.code(p, gi, 2 * h);
              float4& y = ys[gi >> 1 < SB ? gi >> 1 : SB - 1];
              y.x = fmaf(a, c[u][h][0], y.x);
              y.y = fmaf(a, c[u][h][1], y.y);
              y.z = fmaf(a, c[u][h][2], y.z);
              y.w = fmaf(a, c[u][h][3], y.w);
            }
        }
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        const float d = sl.dscale(2 * sb);
        yv.x = fmaf(d, ys[sb].x, yv.x);
        yv.y = fmaf(d, ys[sb].y, yv.y);
        yv.z = fmaf(d, ys[sb].z, yv.z);
        yv.w = fmaf(d, ys[sb].w, yv.w);
      }
      return make_float4(-yv.x, -yv.y, -yv.z, -yv.w);
    } else if constexpr (mma_fast_shape<GPW, MAXW>()) {
      // Five or six planes, or G = 64: each (column tile, plane) runs its
      // own chains.
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        float4 ys = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int gi = 2 * sb; gi < 2 * sb + 2 && gi < GPW; ++gi)
#pragma unroll
          for (int p = 0; p < P; ++p) {
            uint32_t b[4][4];
            plane_operands(sl.w[gi][p], mx.d, b);
#pragma unroll
            for (int h = 0; h < (G == 64 ? 2 : 1); ++h) {
              f32x4_t c = mx.cinit[gi][h];
#pragma unroll
              for (int t = (G == 64 ? 2 * h : 0); t < (G == 64 ? 2 * h + 2 : 4); ++t)
                c = mfma16x16x32(&xa[gi][4 * t], b[t], c);
              const float a = (float)sl.code(p, gi, 2 * h);
              ys.x = fmaf(a, c[0], ys.x);
              ys.y = fmaf(a, c[1], ys.y);
              ys.z = fmaf(a, c[2], ys.z);
              ys.w = fmaf(a, c[3], ys.w);
            }
          }
        const float d = sl.dscale(2 * sb);
        yv.x = fmaf(d, ys.x, yv.x);
        yv.y = fmaf(d, ys.y, yv.y);
        yv.z = fmaf(d, ys.z, yv.z);
        yv.w = fmaf(d, ys.w, yv.w);
      }
      return make_float4(-yv.x, -yv.y, -yv.z, -yv.w);
    } else {
      const PairDecode& one = mx.one;
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gi = 2 * sb; gi < 2 * sb + 2 && gi < GPW; ++gi)
#pragma unroll
          for (int p = 0; p < P; ++p) {
            const uint32_t wp = sl.w[gi][p];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const uint32_t ap = code_pair(sl.code(p, gi, t));
              const uint32_t bq[4] = {scaled_sign_pair(wp, 4 * t + 0, one.mask, ap),
                                      scaled_sign_pair(wp, 4 * t + 1, one.mask, ap),
                                      scaled_sign_pair(wp, 4 * t + 2, one.mask, ap),
                                      scaled_sign_pair(wp, 4 * t + 3, one.mask, ap)};
              c = mfma16x16x32(&xa[gi][4 * t], bq, c);
            }
          }
        const float d = sl.dscale(2 * sb);
        yv.x = fmaf(d, c[0], yv.x);
        yv.y = fmaf(d, c[1], yv.y);
        yv.z = fmaf(d, c[2], yv.z);
        yv.w = fmaf(d, c[3], yv.w);
      }
      return yv;
    }
  }

  // Two 16-row m-tiles at once (the 17..32-row form, G >= 128, P <= 4), as
  // PlaneFmt::mma2: every decoded operand feeds both m-tiles' chains.
  template <int GPW>
  struct Mma2 {
    f32x4_t cinit[2][GPW];
    PlaneDecode d;
  };
  template <int GPW>
  static __device__ __forceinline__ void prepare_mma2(uint32_t (&xa)[2][GPW][16], Mma2<GPW>& mx) {
    static_assert(G != 64, "the two-m-tile form takes whole-tile codes");
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        xa[mt][gi][11] ^= 0x80008000u;
        xa[mt][gi][15] ^= 0x80008000u;
      }
      f32x4_t cs[GPW][2];
      plane_chain_starts<GPW, 1>(xa[mt], cs);
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) mx.cinit[mt][gi] = cs[gi][0];
    }
    mx.d = plane_decode();
  }
  template <int GPW>
  static __device__ __forceinline__ void mma2(const Slot<GPW>& sl, const uint32_t (&xa)[2][GPW][16],
                                              const Mma2<GPW>& mx, float4 (&yv)[2]) {
    static_assert(P <= 4 && G != 64, "two m-tiles hold up to four planes of whole-tile codes");
    // Each chain is weighted by its alpha = d x a, exact in fp32 (an fp16
    // significand times an 8-bit code), so no per-super-block sums are held.
    constexpr int IL = GPW < 2 ? GPW : 2;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) yv[mt] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int g0c = 0; g0c < GPW; g0c += IL) {
        PlaneViews v[IL];
        f32x4_t c[2][IL];
        plane_views_n<IL>([&](int u) { return sl.w[g0c + u][p]; }, v);
#pragma unroll
        for (int u = 0; u < IL; ++u) {
          c[0][u] = mx.cinit[0][g0c + u];
          c[1][u] = mx.cinit[1][g0c + u];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int u = 0; u < IL; ++u) {
            uint32_t b[4];
            plane_operands_t(v[u], t, mx.d, b);
            c[0][u] = mfma16x16x32(&xa[0][g0c + u][4 * t], b, c[0][u]);
            c[1][u] = mfma16x16x32(&xa[1][g0c + u][4 * t], b, c[1][u]);
          }
#pragma unroll
        for (int u = 0; u < IL; ++u) {
          const int gi = g0c + u;
          const float a = sl.dscale(gi) * (float)sl.code(p, gi, 0);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            yv[mt].x = fmaf(a, c[mt][u][0], yv[mt].x);
            yv[mt].y = fmaf(a, c[mt][u][1], yv[mt].y);
            yv[mt].z = fmaf(a, c[mt][u][2], yv[mt].z);
            yv[mt].w = fmaf(a, c[mt][u][3], yv[mt].w);
          }
        }
      }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) yv[mt] = make_float4(-yv[mt].x, -yv[mt].y, -yv[mt].z, -yv[mt].w);
  }
};

// Chunk length of the table kernel: the tables (8 KiB per wave at four groups)
// plus the chunk staging must leave room for two workgroups per CU.
constexpr int kChunkGemvLut = 13;

// Sign-plane mat-vec and head (M = 1) for storage format F.  ARGMAX selects
// the epilogue.
template <class F, int GPW, int MAXW, int D, bool ARGMAX>
__global__ void __launch_bounds__(64 * MAXW)
    k_gemv_planes(const uint8_t* __restrict__ blob, const uint32_t* __restrict__ xw, uint16_t* __restrict__ y,
                    uint8_t* __restrict__ ws, HeadOut ho, int N, int KT, int NT) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int g0 = wave * GPW;
  const typename F::View bv = F::view(blob, KT, NT);
  const int T = tiles_of_wg(NT);

  uint32_t xo[GPW];
  load_x_own<GPW>(xw, g0, KT, q, r, xo);
  // The activation loads go out first: the first tile's work waits on them.
  __builtin_amdgcn_sched_barrier(0);
  typename F::template Slot<GPW> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    F::template load<GPW>(ring[j], bv, row_tile(j), j < T, g0, lane, r);
    // Issue each slot's loads in the same order the loop refills them.
    __builtin_amdgcn_sched_barrier(0);
  }
  // Keep the whole prefetch issued before anything waits on the activations.
  __builtin_amdgcn_sched_barrier(0);
  // Up to eight waves the nibble tables fit beside the staging area; wider
  // workgroups (K > 4096) decode every sign pair instead.
  constexpr bool kLut = MAXW <= 8;
  constexpr int C = kLut ? kChunkGemvLut : kChunkGemv;
  __shared__ ChunkStage<float, C, MAXW, 16> stage;
  __shared__ SignLut<kLut ? GPW : 1> luts[kLut ? MAXW : 1];
  uint32_t xp[GPW][16];
  if constexpr (kLut)
    build_sign_lut<GPW>(luts[wave], xo, q, r);
  else
    expand_x<GPW>(xo, xp);
  const PairDecode one = sign_decode();
  // Opaque copy: the compiler would otherwise turn the OR of disjoint bits in
  // every address into an ADD and lose the one-instruction AND-OR form.
  const uint32_t lut_off =
      opaque_copy((uint32_t)wave * (uint32_t)sizeof(SignLut<kLut ? GPW : 1>) | (uint32_t)(64 * q));
  float best_v = -FLT_MAX;
  int best_i = INT_MAX;

  int i0 = 0;
  auto step = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const int i = i0 + j;
    float part;
    if constexpr (kLut)
      part = sum_over_q(F::template partial_lut<GPW>(ring[j], luts, lut_off));
    else
      part = sum_over_q(F::template partial<GPW>(ring[j], xp, one));
    stage.put(i, i < T, wave, lane, part);
    // Slot j is refilled only after its last use, so it keeps its registers.
    __builtin_amdgcn_sched_barrier(0);
    F::template load<GPW>(ring[j], bv, row_tile(i + D), i + D < T, g0, lane, r);
    const int ci = i % C;
    if (i < T && (ci == C - 1 || i == T - 1)) {
      __syncthreads();
      const int first = i - ci;
      for (int o = threadIdx.x; o < (ci + 1) * 16; o += nwaves * 64) {
        const int n = 16 * row_tile(first + (o >> 4)) + (o & 15);
        if (n < N) {
          const float v = stage.sum(i, o >> 4, nwaves, o & 15);
          if constexpr (ARGMAX) {
            if (v > best_v) {  // a thread's rows arrive in increasing n
              best_v = v;
              best_i = n;
            }
          } else {
            y[n] = f32_to_bf16_rne(v);
          }
        }
      }
    }
  };
  // Whole rounds of the ring, then the tiles of a partial last round (held in
  // the ring's first slots) one by one, so no step runs on an empty tile.
  const int whole = T - T % D;
  for (; i0 < whole; i0 += D) static_for<0, D>(step);
  static_for<0, D - 1>([&](auto jc) {
    if (decltype(jc)::value < T - whole) step(jc);
  });
  if constexpr (ARGMAX) gemv_argmax_epilogue<MAXW>(best_v, best_i, wave, lane, nwaves, ws, N, ho);
}

// ---------------------------------------------------------------------------
// M <= 16 verify kernels on v_mfma_f32_16x16x32_bf16.  Per 32-wide k block t,
// A = X[m = r][k = 32t + 8q + 0..7] (lane q, r) and B = W^T[k][n = r] from the
// tile's dword t; D lands as D[m = 4q + i][n = r], i = 0..3.

// The W4A16 MFMA chain of each group run on decoded zero codes (B = 136
// everywhere): 136 * sum_k X[m][k] over the group for the rows m = 4q + i
// whose outputs this lane's result holds, formed by the same four MFMAs, in
// the same order and from the same zero start, as a tile's chain, so the two
// agree bit for bit wherever the tile's codes are zero.  The value does not
// depend on the row tile, so it is formed once per kernel.
template <int GPW>
__device__ __forceinline__ void zero_code_chains(const uint32_t (&xa)[GPW][16], f32x4_t (&z)[GPW]) {
  const uint32_t b[4] = {kInt4ZeroPair, kInt4ZeroPair, kInt4ZeroPair, kInt4ZeroPair};
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) c = mfma16x16x32(&xa[gi][4 * t], b, c);
    z[gi] = c;
  }
}

// Running greedy choice per query row m = 4q + ii of a lane (M <= 16 heads).
struct RowBest4 {
  float v[4];
  int idx[4];
};

// Combines the lanes' and waves' running bests (lowest index wins ties) and
// completes the launch's argmax.
template <int MAXW>
__device__ __forceinline__ void gemm_argmax_epilogue(RowBest4& b, int wave, int lane, int nwaves, uint8_t* ws,
                                                     int M, int N, const HeadOut& ho) {
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) best_over_row(b.v[ii], b.idx[ii]);  // over the 16 lanes of one q
  __shared__ ArgBest fin[MAXW][16];  // [wave][query row]
  if ((lane & 15) == 0)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) fin[wave][4 * (lane >> 4) + ii] = ArgBest{b.v[ii], b.idx[ii]};
  __syncthreads();
  float bvv = -FLT_MAX;
  int bii = INT_MAX;
  if ((int)threadIdx.x < M) {
    // Every wave's entry read at once (unrolled over MAXW; nwaves is
    // uniform), then folded in wave order.
    ArgBest t[MAXW];
#pragma unroll
    for (int w = 0; w < MAXW; ++w) t[w] = fin[w < nwaves ? w : 0][threadIdx.x];
#pragma unroll
    for (int w = 0; w < MAXW; ++w)
      if (w < nwaves && better(t[w].v, t[w].idx, bvv, bii)) {
        bvv = t[w].v;
        bii = t[w].idx;
      }
  }
  argmax_complete(argmax_key(bvv, bii), (int)threadIdx.x < M && bii < N, threadIdx.x, ws, M, N, ho);
}

// Emits a completed 16 x 16 output tile held as lane (q, r) -> rows 4q + ii,
// column r of row tile rt.
template <bool ARGMAX>
__device__ __forceinline__ void gemm_emit(const float4& tot, int q, int r, int rt, int M, int N,
                                          uint16_t* __restrict__ Y, RowBest4& best) {
  const int n = 16 * rt + r;
  const float v[4] = {tot.x, tot.y, tot.z, tot.w};
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int m = 4 * q + ii;
    if (m < M && n < N) {
      if constexpr (ARGMAX) {
        if (v[ii] > best.v[ii]) {  // a lane's columns arrive in increasing n
          best.v[ii] = v[ii];
          best.idx[ii] = n;
        }
      } else {
        Y[(size_t)m * N + n] = f32_to_bf16_rne(v[ii]);
      }
    }
  }
}

template <int GPW, int MAXW, int D, bool ARGMAX>
__global__ void __launch_bounds__(64 * MAXW)
    k_gemm_w4a16(const uint8_t* __restrict__ blob, const uint32_t* __restrict__ Xw, uint16_t* __restrict__ Y,
                 uint8_t* __restrict__ ws, HeadOut ho, int M, int N, int KT, int NT, int ms) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int g0 = wave * GPW;
  const BlobView bv = int4_view(blob, KT, NT);
  // The heads never split their rows (M <= 16).
  const TileWalk tw = ARGMAX ? TileWalk{(int)blockIdx.x, (int)gridDim.x, 0} : tile_walk(ms);
  const int T = tw.count(NT);
  if constexpr (!ARGMAX) {
    // This workgroup's m-tile: 16 rows of X (K / 2 dwords each) and of Y.
    Xw += (size_t)tw.mt * 16 * KT * 64;
    Y += (size_t)tw.mt * 16 * N;
    M = M - 16 * tw.mt < 16 ? M - 16 * tw.mt : 16;
  }

  // In the full-register shapes X comes in coalesced and is transposed
  // through LDS; the lean ones (16 waves of four column tiles, 128
  // registers a lane) load it in operand order directly.
  constexpr bool kRowsX = mma_fast_shape<GPW, MAXW>();
  XRows<kRowsX ? GPW : 1> xrows;
  uint32_t xa[GPW][16];
  if constexpr (kRowsX)
    load_x_rows<GPW>(reinterpret_cast<const uint16_t*>(Xw), M, KT * 128, g0, KT, lane, xrows);
  else
    load_x_pairs<GPW>(Xw, r, M, g0, KT, q, xa);
  // The activation loads go out first: the first tile's work waits on them.
  __builtin_amdgcn_sched_barrier(0);
  Int4Slot<GPW> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    load_int4_tile<GPW>(ring[j], bv, tw.tile(j), j < T, g0, lane, r);
    // Issue each slot's loads in the same order the loop refills them.
    __builtin_amdgcn_sched_barrier(0);
  }
  // Keep the whole prefetch issued before anything waits on the activations.
  __builtin_amdgcn_sched_barrier(0);
  constexpr int C = chunk_gemm<MAXW>();
  // Reads in flight in the cross-wave sum of a tile (ChunkStage::sum): as
  // many as the registers left beside the ring allow.
  constexpr int kSumW4 = MAXW <= 8 && D <= 2 ? MAXW - 1 : 1;
  __shared__ ChunkStage<float4, C, MAXW, 64> stage;
  if constexpr (kRowsX) {
    __shared__ uint4 xt[MAXW][256];  // a wave's transposition region (4 KiB)
    transpose_x_rows<GPW>(xrows, xt[wave], lane, q, r, xa);
  } else {
    mask_x_pairs<GPW>(r, M, g0, KT, xa);
  }
  f32x4_t zc[GPW];
  zero_code_chains<GPW>(xa, zc);
  const PairDecode magic = int4_decode();

  RowBest4 best;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    best.v[ii] = -FLT_MAX;
    best.idx[ii] = INT_MAX;
  }
  int i0 = 0;
  auto step = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const int i = i0 + j;
    float4 yv = make_float4(0.f, 0.f, 0.f, 0.f);
    // One MFMA chain per group.  In the full-register shapes the groups'
    // chains are interleaved k block by k block, so consecutive MFMAs are
    // independent and the matrix core need not wait for each result before
    // the next issue; the lean shapes run them one after another.
    constexpr int IL = mma_fast_shape<GPW, MAXW>() ? GPW : 1;  // chains in flight
#pragma unroll
    for (int g0c = 0; g0c < GPW; g0c += IL) {
      f32x4_t c[IL];
#pragma unroll
      for (int u = 0; u < IL; ++u) c[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t0 = 0; t0 < 4; t0 += 2) {
        // k blocks t0 and t0 + 1 of every chain decoded together
        // (int4_pairs2 on adjacent code dwords), then the MFMAs in k-block
        // order.
        uint32_t b[IL][2][4];
#pragma unroll
        for (int u = 0; u < IL; ++u)
          int4_pairs2((&ring[j].c[g0c + u].x)[t0], (&ring[j].c[g0c + u].x)[t0 + 1], magic, b[u][0], b[u][1]);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int u = 0; u < IL; ++u) c[u] = mfma16x16x32(&xa[g0c + u][4 * (t0 + tt)], b[u][tt], c[u]);
      }
#pragma unroll
      for (int u = 0; u < IL; ++u) {
        const float sc = ring[j].s.bf16(g0c + u);
        const f32x4_t& z = zc[g0c + u];
        yv.x = fmaf(sc, c[u][0] - z[0], yv.x);
        yv.y = fmaf(sc, c[u][1] - z[1], yv.y);
        yv.z = fmaf(sc, c[u][2] - z[2], yv.z);
        yv.w = fmaf(sc, c[u][3] - z[3], yv.w);
      }
    }
    stage.put(i, i < T, wave, lane, yv);
    // Slot j is refilled only after its last use, so it keeps its registers.
    __builtin_amdgcn_sched_barrier(0);
    load_int4_tile<GPW>(ring[j], bv, tw.tile(i + D), i + D < T, g0, lane, r);
    const int ci = i % C;
    if (i < T && (ci == C - 1 || i == T - 1)) {
      __syncthreads();
      const int first = i - ci;
      // Wave c finishes tile c of the chunk (C <= waves); a lane meets the
      // same outputs of every tile, so its columns arrive in increasing n.
      if (wave <= ci) gemm_emit<ARGMAX>(stage.template sum<kSumW4>(i, wave, nwaves, lane), q, r, tw.tile(first + wave), M, N, Y, best);
    }
  };
  // Whole rounds of the ring, then the tiles of a partial last round (held in
  // the ring's first slots) one by one, so no step runs on an empty tile.
  const int whole = T - T % D;
  for (; i0 < whole; i0 += D) static_for<0, D>(step);
  static_for<0, D - 1>([&](auto jc) {
    if (decltype(jc)::value < T - whole) step(jc);
  });
  if constexpr (ARGMAX)
    gemm_argmax_epilogue<MAXW>(best, wave, lane, nwaves, ws, M, N, ho);
}

// W4A16 mat-mul for blocks of 17..32 rows at K <= 4096 (eight waves or
// fewer): the M <= 16 kernel with both 16-row m-tiles of X held in registers,
// so every decoded weight pair feeds the MFMAs of both m-tiles and the
// weights are read once for the block.  X arrives as for the M <= 16 kernel
// (coalesced, transposed through a wave-private LDS region per m-tile); the
// partial tiles of the two m-tiles meet in two staging areas, two tiles per
// chunk, waves 0-1 finishing m-tile 0 and waves 2-3 m-tile 1.
template <int GPW, int D>
__global__ void __launch_bounds__(64 * 8)
    k_gemm_w4a16_x2(const uint8_t* __restrict__ blob, const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                    int M, int N, int KT, int NT) {
  constexpr int MAXW = 8, C = 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int g0 = wave * GPW;
  const int K = KT * 128;
  const BlobView bv = int4_view(blob, KT, NT);
  const int T = tiles_of_wg(NT);

  // Rows 16..M-1 of the second m-tile read zero past M (buffer range).
  XRows<GPW> xr0, xr1;
  load_x_rows<GPW>(X, M, K, g0, KT, lane, xr0);
  load_x_rows<GPW>(X + (size_t)16 * K, M - 16, K, g0, KT, lane, xr1);
  __builtin_amdgcn_sched_barrier(0);
  Int4Slot<GPW> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    load_int4_tile<GPW>(ring[j], bv, row_tile(j), j < T, g0, lane, r);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_sched_barrier(0);
  __shared__ ChunkStage<float4, C, MAXW, 64> stage[2];
  __shared__ uint4 xt[MAXW][2][256];  // a wave's two transposition regions (2 x 4 KiB)
  uint32_t xa[2][GPW][16];
  transpose_x_rows<GPW>(xr0, xt[wave][0], lane, q, r, xa[0]);
  transpose_x_rows<GPW>(xr1, xt[wave][1], lane, q, r, xa[1]);
  f32x4_t zc[2][GPW];
  zero_code_chains<GPW>(xa[0], zc[0]);
  zero_code_chains<GPW>(xa[1], zc[1]);
  const PairDecode magic = int4_decode();
  RowBest4 unused;

  int i0 = 0;
  do {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int i = i0 + j;
      f32x4_t c[2][GPW];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) c[mt][gi] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int gi = 0; gi < GPW; ++gi) {
          const uint32_t w = (&ring[j].c[gi].x)[t];
          const uint32_t bq[4] = {int4_pair(w, 0, magic), int4_pair(w, 1, magic), int4_pair(w, 2, magic),
                                  int4_pair(w, 3, magic)};
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) c[mt][gi] = mfma16x16x32(&xa[mt][gi][4 * t], bq, c[mt][gi]);
        }
      float4 yv[2] = {make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
#pragma unroll
      for (int gi = 0; gi < GPW; ++gi) {
        const float sc = ring[j].s.bf16(gi);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const f32x4_t& z = zc[mt][gi];
          yv[mt].x = fmaf(sc, c[mt][gi][0] - z[0], yv[mt].x);
          yv[mt].y = fmaf(sc, c[mt][gi][1] - z[1], yv[mt].y);
          yv[mt].z = fmaf(sc, c[mt][gi][2] - z[2], yv[mt].z);
          yv[mt].w = fmaf(sc, c[mt][gi][3] - z[3], yv[mt].w);
        }
      }
      stage[0].put(i, i < T, wave, lane, yv[0]);
      stage[1].put(i, i < T, wave, lane, yv[1]);
      // Slot j is refilled only after its last use, so it keeps its registers.
      __builtin_amdgcn_sched_barrier(0);
      load_int4_tile<GPW>(ring[j], bv, row_tile(i + D), i + D < T, g0, lane, r);
      const int ci = i % C;
      if (i < T && (ci == C - 1 || i == T - 1)) {
        __syncthreads();
        const int first = i - ci;
        const int mt = wave / C, cc = wave % C;  // (m-tile, tile of the chunk) of waves 0-3
        if (mt < 2 && cc <= ci)
          gemm_emit<false>(stage[mt].sum(i, cc, nwaves, lane), q, r, row_tile(first + cc), M - 16 * mt, N,
                           Y + (size_t)16 * mt * N, unused);
      }
    }
    i0 += D;
  } while (i0 < T);
}

// Sign-plane verify mat-mul and head (M <= 16) for storage format F.
template <class F, int GPW, int MAXW, int D, bool ARGMAX>
__global__ void __launch_bounds__(64 * MAXW)
    k_gemm_planes(const uint8_t* __restrict__ blob, const uint32_t* __restrict__ Xw, uint16_t* __restrict__ Y,
                    uint8_t* __restrict__ ws, HeadOut ho, int M, int N, int KT, int NT, int ms) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int g0 = wave * GPW;
  const typename F::View bv = F::view(blob, KT, NT);
  // The heads never split their rows (M <= 16).
  const TileWalk tw = ARGMAX ? TileWalk{(int)blockIdx.x, (int)gridDim.x, 0} : tile_walk(ms);
  const int T = tw.count(NT);
  if constexpr (!ARGMAX) {
    // This workgroup's m-tile: 16 rows of X (K / 2 dwords each) and of Y.
    Xw += (size_t)tw.mt * 16 * KT * 64;
    Y += (size_t)tw.mt * 16 * N;
    M = M - 16 * tw.mt < 16 ? M - 16 * tw.mt : 16;
  }

  // In the full-register shapes X comes in coalesced and is transposed
  // through LDS; the lean ones (16 waves of four column tiles, 128
  // registers a lane) load it in operand order directly.
  constexpr bool kRowsX = mma_fast_shape<GPW, MAXW>();
  XRows<kRowsX ? GPW : 1> xrows;
  uint32_t xa[GPW][16];
  if constexpr (kRowsX)
    load_x_rows<GPW>(reinterpret_cast<const uint16_t*>(Xw), M, KT * 128, g0, KT, lane, xrows);
  else
    load_x_pairs<GPW>(Xw, r, M, g0, KT, q, xa);
  // The activation loads go out first: the first tile's work waits on them.
  __builtin_amdgcn_sched_barrier(0);
  typename F::template Slot<GPW> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    F::template load<GPW>(ring[j], bv, tw.tile(j), j < T, g0, lane, r);
    // Issue each slot's loads in the same order the loop refills them.
    __builtin_amdgcn_sched_barrier(0);
  }
  // Keep the whole prefetch issued before anything waits on the activations.
  __builtin_amdgcn_sched_barrier(0);
  constexpr int C = chunk_gemm<MAXW>();
  // Reads in flight in the cross-wave sum of a tile (ChunkStage::sum): as
  // many as the registers left beside the ring allow.
  constexpr int kSumPl = MAXW <= 8 && D <= 2 && F::P <= 3 ? MAXW - 1 : 1;
  __shared__ ChunkStage<float4, C, MAXW, 64> stage;
  if constexpr (kRowsX) {
    __shared__ uint4 xt[MAXW][256];  // a wave's transposition region (4 KiB)
    transpose_x_rows<GPW>(xrows, xt[wave], lane, q, r, xa);
  } else {
    mask_x_pairs<GPW>(r, M, g0, KT, xa);
  }
  typename F::template MmaX<GPW, MAXW> mx;
  F::template prepare_mma<GPW, MAXW>(xa, q, mx);

  RowBest4 best;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    best.v[ii] = -FLT_MAX;
    best.idx[ii] = INT_MAX;
  }
  int i0 = 0;
  auto step = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const int i = i0 + j;
    const float4 yv = F::template mma<GPW, MAXW>(ring[j], xa, mx);
    stage.put(i, i < T, wave, lane, yv);
    // Slot j is refilled only after its last use, so it keeps its registers.
    __builtin_amdgcn_sched_barrier(0);
    F::template load<GPW>(ring[j], bv, tw.tile(i + D), i + D < T, g0, lane, r);
    const int ci = i % C;
    if (i < T && (ci == C - 1 || i == T - 1)) {
      __syncthreads();
      const int first = i - ci;
      // Wave c finishes tile c of the chunk (C <= waves); a lane meets the
      // same outputs of every tile, so its columns arrive in increasing n.
      if (wave <= ci) gemm_emit<ARGMAX>(stage.template sum<kSumPl>(i, wave, nwaves, lane), q, r, tw.tile(first + wave), M, N, Y, best);
    }
  };
  // Whole rounds of the ring, then the tiles of a partial last round (held in
  // the ring's first slots) one by one, so no step runs on an empty tile.
  const int whole = T - T % D;
  for (; i0 < whole; i0 += D) static_for<0, D>(step);
  static_for<0, D - 1>([&](auto jc) {
    if (decltype(jc)::value < T - whole) step(jc);
  });
  if constexpr (ARGMAX)
    gemm_argmax_epilogue<MAXW>(best, wave, lane, nwaves, ws, M, N, ho);
}

// Sign-plane mat-mul for blocks of 17..32 rows at K <= 4096 (eight waves or
// fewer), format F with a two-m-tile tile (PlaneFmt, or SaFmt at G >= 128):
// the M <= 16 kernel with both m-tiles of X in registers, as
// k_gemm_w4a16_x2 does for W4A16, so the weights are read and decoded once
// for the block.
template <class F, int GPW, int D>
__global__ void __launch_bounds__(64 * 8)
    k_gemm_planes_x2(const uint8_t* __restrict__ blob, const uint16_t* __restrict__ X, uint16_t* __restrict__ Y,
                     int M, int N, int KT, int NT) {
  constexpr int MAXW = 8, C = 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const int q = lane >> 4, r = lane & 15;
  const int g0 = wave * GPW;
  const int K = KT * 128;
  const typename F::View bv = F::view(blob, KT, NT);
  const int T = tiles_of_wg(NT);

  // Rows 16..M-1 of the second m-tile read zero past M (buffer range).
  XRows<GPW> xr0, xr1;
  load_x_rows<GPW>(X, M, K, g0, KT, lane, xr0);
  load_x_rows<GPW>(X + (size_t)16 * K, M - 16, K, g0, KT, lane, xr1);
  __builtin_amdgcn_sched_barrier(0);
  typename F::template Slot<GPW> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    F::template load<GPW>(ring[j], bv, row_tile(j), j < T, g0, lane, r);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_sched_barrier(0);
  __shared__ ChunkStage<float4, C, MAXW, 64> stage[2];
  __shared__ uint4 xt[MAXW][2][256];  // a wave's two transposition regions (2 x 4 KiB)
  uint32_t xa[2][GPW][16];
  transpose_x_rows<GPW>(xr0, xt[wave][0], lane, q, r, xa[0]);
  transpose_x_rows<GPW>(xr1, xt[wave][1], lane, q, r, xa[1]);
  typename F::template Mma2<GPW> mx;
  F::template prepare_mma2<GPW>(xa, mx);
  RowBest4 unused;

  int i0 = 0;
  auto step = [&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const int i = i0 + j;
    float4 yv[2];
    F::template mma2<GPW>(ring[j], xa, mx, yv);
    stage[0].put(i, i < T, wave, lane, yv[0]);
    stage[1].put(i, i < T, wave, lane, yv[1]);
    // Slot j is refilled only after its last use, so it keeps its registers.
    __builtin_amdgcn_sched_barrier(0);
    F::template load<GPW>(ring[j], bv, row_tile(i + D), i + D < T, g0, lane, r);
    const int ci = i % C;
    if (i < T && (ci == C - 1 || i == T - 1)) {
      __syncthreads();
      const int first = i - ci;
      const int mt = wave / C, cc = wave % C;  // (m-tile, tile of the chunk) of waves 0-3
      if (mt < 2 && cc <= ci)
        gemm_emit<false>(stage[mt].sum(i, cc, nwaves, lane), q, r, row_tile(first + cc), M - 16 * mt, N,
                         Y + (size_t)16 * mt * N, unused);
    }
  };
  // Whole rounds of the ring, then the tiles of a partial last round one by
  // one, so no step runs on an empty tile.
  const int whole = T - T % D;
  for (; i0 < whole; i0 += D) static_for<0, D>(step);
  static_for<0, D - 1>([&](auto jc) {
    if (decltype(jc)::value < T - whole) step(jc);
  });
}

}  // namespace
