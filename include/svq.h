/*
 * svq.h -- C ABI of the MI355X (gfx950) low-bit linear-layer library.
 *
 * Operations (what each call computes is stated with its declaration):
 *   W4A16:  y[m][n] = sum_g s[n][g] * sum_{k in g} c[n][k] * x[m][k]
 *           c in [-8, 7] INT4 codes, s bf16 symmetric per-group scales, no
 *           zero point, groups of 128 along the input dimension k.
 *           (Efficient Qwen Competition report, sec. 2.1 "Target Model
 *           Optimization with QAD" and sec. 3.3 "Drafter Optimization".)
 *   Binary planes: y[m][n] = sum_g sum_p alpha[p][n][g] * sum_{k in g} b[p][n][k] * x[m][k]
 *           b in {-1, +1}, alpha fp16, one scale per (plane, row, group).
 *           (ShiftAddQwen README, intro and "Method / Format".)
 *   sa* storage of the same sum: alpha[p][n][g] = d[n][j] * a[p][n][g],
 *           a a u8 code per (plane, row, group of G in {64, 128, 256}) and
 *           d an fp16 value per (row, j = the 256-wide k range holding g).
 *           (ShiftAddQwen README, "Method / Format", the sa{2..6} types.)
 *   Greedy verify head: argmax over the W4A16 logits of a (possibly
 *           vocabulary-trimmed) head, lowest index on ties, optionally mapped
 *           through a row -> token-id table.  (DFlash summary sec. 4.1 and the
 *           report's sec. 2.2 for parallel verification; small-vocabulary
 *           MTP study sec. 3.3 for the trimmed 32,768-row head.)
 *
 * Conventions for every call:
 *   - bf16 and fp16 values travel as uint16_t bit patterns.
 *   - Shapes: W is [N][K] (row n = output feature), x/X is [M][K] row-major,
 *     y/Y is [M][N] row-major.  K % 128 == 0, G == 128 (sa calls: K % 256
 *     == 0, G in {64, 128, 256}).
 *   - Return 0 (SVQ_OK) on success or a negative SVQ_ERR_* code.  On error
 *     nothing is written and svq_last_error() returns a message for the
 *     calling thread.  No C++ exception crosses this boundary.
 *   - The caller owns every buffer.  The library allocates no device memory
 *     and keeps no state beyond cached device attributes and the per-thread
 *     error string.
 *   - Device calls are asynchronous on `stream` (a hipStream_t passed as
 *     void*, NULL = the null stream); they do not synchronise.  A launch
 *     error is reported as SVQ_ERR_HIP; faults during execution surface at
 *     the caller's next synchronisation.  Calls on one stream are ordered;
 *     calls are reentrant.
 *
 * Packed blob layouts (the pages name the formats; the byte layout is this
 * library's own, chosen so one 64-lane wave reads whole 1 KiB tiles and the
 * same tile feeds both the mat-vec and the 16x16x32 bf16 MFMA):
 *   INT4 blob, N16 = N rounded up to 16, KT = K / 128:
 *     codes: tile (rt, kt) at byte (rt*KT + kt) * 1024.  Inside a tile,
 *       lane = 16*q + r owns bytes [16*lane, 16*lane + 16) = four
 *       little-endian dwords t = 0..3.  Dword t holds row n = 16*rt + r at
 *       k = 128*kt + 32*t + 8*q + j (j = 0..7): even j = 2i in bits
 *       [4i, 4i+4), odd j = 2i+1 in bits [16+4i, 20+4i), each nibble
 *       u = c + 8.  Padding rows (n >= N) hold c = 0.
 *     scales: right after the codes, i.e. at byte N16 * K / 2: row n < N16
 *       holds bf16 s[n][g] at entry n*KT4 + g, KT4 = KT rounded up to 4, so
 *       a lane fetches four groups' scales with one 8-byte load.  Entries
 *       g >= KT and padding rows are 0.
 *   Binary-plane blob with P planes:
 *     signs: tile (rt, kt) at byte (rt*KT + kt) * 256 * P; plane p of the
 *       tile is the 256 bytes at offset 256*p, in which lane 16*q + r owns
 *       the dword at 4*lane: plane p, row 16*rt + r, k = 128*kt + 32*t +
 *       8*q + j: even j = 2i at bit 4t + i, odd j = 2i+1 at bit 16 + 4t + i.
 *       A set bit means b = -1.  Padding rows hold +1.
 *     alphas: right after the signs, i.e. at byte N16 * K / 8 * P: fp16
 *       alpha[p][n][g] at entry (p*N16 + n)*KT4 + g.  Entries g >= KT and
 *       padding rows are 0.
 *   sa blob with P planes and group G (K % 256 == 0):
 *     signs: exactly the binary-plane blob's sign section.
 *     codes: right after the signs (byte N16 * K / 8 * P): u8 a[p][n][g] at
 *       byte (p*N16 + n)*CG + g, CG = KT4 * 128 / G (a row of codes spans
 *       KT4 column tiles, so a wave's run of codes is one aligned load).
 *       Entries g >= K/G and padding rows are 0.
 *     d: right after the codes: fp16 d[n][j] (super-block j covers
 *       k in [256j, 256j + 256)) at entry n*KS2 + j, KS2 = KT4 / 2.  Entries
 *       j >= K/256 and padding rows are 0.
 */
#ifndef SVQ_H
#define SVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SVQ_OK = 0,
  SVQ_ERR_NULL = -1,      /* a required pointer is NULL */
  SVQ_ERR_SHAPE = -2,     /* a size is out of the supported range */
  SVQ_ERR_ALIGN = -3,     /* a pointer is not aligned as required */
  SVQ_ERR_RANGE = -4,     /* a code or sign is outside its alphabet */
  SVQ_ERR_WORKSPACE = -5, /* workspace missing or too small */
  SVQ_ERR_HIP = -6        /* the HIP runtime reported an error */
};

#define SVQ_GROUP 128     /* the only supported group size */
#define SVQ_MAX_M 16      /* rows of a verify block (heads, acceptance) */
#define SVQ_MAX_M_GEMM 65536 /* rows of X a gemm_smallm_* call takes */
#define SVQ_BLOCK_M 64       /* rows of X one launch of gemm_smallm_* covers */
#define SVQ_MAX_P 6       /* sign planes per weight */
#define SVQ_MAX_K 8192    /* largest input dimension the kernels accept */

/* Message describing the last error on the calling thread ("" if none). */
const char* svq_last_error(void);

/* Bytes of a packed INT4 blob: N16*K/2 + N16*KT4*2.  0 for bad sizes. */
size_t svq_int4_packed_bytes(int64_t N, int64_t K, int32_t G);

/* Bytes of a packed binary-plane blob: N16*K/8*P + P*N16*KT4*2.  0 for bad sizes. */
size_t svq_binplane_packed_bytes(int64_t N, int64_t K, int32_t G, int32_t P);

/* Bytes of a packed sa blob: N16*K/8*P + P*N16*CG + N16*KS2*2.  0 for bad
 * sizes (K % 256, G not in {64, 128, 256}, P outside 2..6). */
size_t svq_sa_packed_bytes(int64_t N, int64_t K, int32_t G, int32_t P);

/* Workspace bytes that lmhead_argmax needs for M query rows. */
size_t svq_lmhead_workspace_bytes(int32_t M);

/*
 * pack_int4_grouped -- HOST pointers, synchronous, CPU only.
 * Stores INT4 codes with their frozen per-group scales in the INT4 blob
 * layout above (report sec. 2.1: the updated weights are rounded back onto
 * the original grid and served as W4A16; sec. 3.3: group size 128).
 *   codes        [N][K] int8, each in [-8, 7]
 *   scales_bf16  [N][K/G] bf16 bits
 *   packed       svq_int4_packed_bytes(N, K, G) bytes, written in full
 * Errors: NULL, SHAPE (N < 1, K % 128, G != 128), RANGE (first offending
 * (n, k) is named in the message).
 */
int pack_int4_grouped(const int8_t* codes, const uint16_t* scales_bf16,
                      int64_t N, int64_t K, int32_t G, uint8_t* packed);

/* Inverse of pack_int4_grouped (HOST, for tests and inspection). */
int unpack_int4_grouped(const uint8_t* packed, int64_t N, int64_t K, int32_t G,
                        int8_t* codes, uint16_t* scales_bf16);

/*
 * pack_binary_planes -- HOST pointers, synchronous, CPU only.
 * Stores P sign planes and their per-(plane, row, group) fp16 scales in the
 * binary-plane blob layout above (ShiftAddQwen README, "Format": sign planes
 * plus one scale per plane and group along the input dimension).
 *   signs      [P][N][K] int8, each -1 or +1
 *   alpha_f16  [P][N][K/G] fp16 bits
 *   packed     svq_binplane_packed_bytes(N, K, G, P) bytes, written in full
 * Errors: NULL, SHAPE (P outside 1..6, N < 1, K % 128, G != 128), RANGE.
 */
int pack_binary_planes(const int8_t* signs, const uint16_t* alpha_f16,
                       int64_t N, int64_t K, int32_t G, int32_t P,
                       uint8_t* packed);

/* Inverse of pack_binary_planes (HOST, for tests and inspection). */
int unpack_binary_planes(const uint8_t* packed, int64_t N, int64_t K, int32_t G,
                         int32_t P, int8_t* signs, uint16_t* alpha_f16);

/*
 * pack_sa -- HOST pointers, synchronous, CPU only.
 * Writes the sa* storage of P sign planes (ShiftAddQwen README, "Method /
 * Format") as the sa blob above: the signs into its sign section, code
 * a[p][n][g] into its code section and d[n][j] into its d section; the scale
 * of plane p, row n, group g is then d[n][g * G / 256] * a[p][n][g].
 *   signs   [P][N][K] int8, each -1 or +1
 *   codes   [P][N][K/G] uint8 scale codes a
 *   d_f16   [N][K/256] fp16 bits
 *   packed  svq_sa_packed_bytes(N, K, G, P) bytes, written in full
 * Errors: NULL, SHAPE (P outside 2..6, N < 1, K % 256, G not in
 * {64, 128, 256}), RANGE (a sign other than +-1).
 */
int pack_sa(const int8_t* signs, const uint8_t* codes, const uint16_t* d_f16,
            int64_t N, int64_t K, int32_t G, int32_t P, uint8_t* packed);

/* Inverse of pack_sa (HOST, for tests and inspection). */
int unpack_sa(const uint8_t* packed, int64_t N, int64_t K, int32_t G, int32_t P,
              int8_t* signs, uint8_t* codes, uint16_t* d_f16);

/*
 * Offline quantizers -- HOST pointers, synchronous, CPU only (threads over
 * rows).  All arithmetic is fp64; results do not depend on the thread count.
 *
 * quantize_int4_frozen: the packing step of the report's sec. 2.1 -- weights
 * trained under frozen symmetric group scales go back onto the same INT4
 * grid, each to its nearest grid point:
 *   codes[n][k] = clamp(round_half_even(w[n][k] / s[n][k/G]), -8, 7)
 * (0 where s == 0).
 *   w_bf16       [N][K] bf16 bits;  scales_bf16 [N][K/G] bf16 bits
 *   codes        [N][K] int8 (pack with pack_int4_grouped)
 * Errors: NULL, SHAPE (N < 1, G not in {64, 128, 256}, K % G).
 */
int quantize_int4_frozen(const uint16_t* w_bf16, const uint16_t* scales_bf16,
                         int64_t N, int64_t K, int32_t G, int8_t* codes);

/*
 * fit_binary_planes: the binary-coding fit of the ShiftAddQwen README
 * ("Output-aware fit": greedy initialisation, then alternating least squares
 * with exhaustive code choice), per (row, group of G), on the plain weight
 * error sum_k (w_k - sum_p alpha_p b_pk)^2:
 *   greedy  r = w; for p = 1..P: b_p = sign(r) (+1 at 0), alpha_p = mean|r|,
 *           r -= alpha_p b_p
 *   round   each weight takes the sign vector whose sum_p alpha_p b_p is
 *           nearest (lowest index on ties, index bit p set means b_p = -1),
 *           then alpha is re-solved by least squares for those signs (kept
 *           when the system is singular); `iters` rounds, fewer once the
 *           signs stop changing (a fixed point)
 *   finally every plane with alpha_p < 0 is negated (same weights), and
 *   alpha is rounded to fp16 (nearest even).
 *   w_bf16     [N][K] bf16 bits
 *   signs      [P][N][K] int8 in {-1, +1};  alpha_f16 [P][N][K/G] fp16 bits
 * Errors: NULL, SHAPE (N < 1, G not in {64, 128, 256}, K % G, P outside
 * 1..6, iters < 0).
 */
int fit_binary_planes(const uint16_t* w_bf16, int64_t N, int64_t K, int32_t G,
                      int32_t P, int32_t iters, int8_t* signs,
                      uint16_t* alpha_f16);

/*
 * snap_sa_scales: plane scales onto the sa* grid (README "Format": alpha =
 * d * a, u8 a per (plane, group), one fp16 d per 256-weight super-block;
 * "Scale distillation": scales end snapped to the u8 grid).  Per (row,
 * super-block j): d = fp16(max alpha / 255) over its planes and groups, and
 * a = min(round_half_even(alpha / d), 255) (0 when d == 0).
 *   alpha_f16  [P][N][K/G] fp16 bits, each >= 0
 *   codes      [P][N][K/G] uint8;  d_f16 [N][K/256] fp16 bits (for pack_sa)
 * Errors: NULL, SHAPE (N < 1, G not in {64, 128, 256}, K % 256, P outside
 * 1..6), RANGE (a negative or NaN alpha).
 */
int snap_sa_scales(const uint16_t* alpha_f16, int64_t N, int64_t K, int32_t G,
                   int32_t P, uint8_t* codes, uint16_t* d_f16);

/*
 * gemv_w4a16 -- DEVICE pointers, asynchronous on `stream`.
 * One decode step of a W4A16 linear layer (report sec. 2.1, 3.3):
 *   y[n] = bf16_rne( sum_g s[n][g] * sum_{k in g} c[n][k] * x[k] ),
 * accumulated in fp32 per group, scaled per group in fp32.
 *   packed  INT4 blob, 16-byte aligned
 *   x       [K] bf16 bits, 16-byte aligned
 *   y       [N] bf16 bits, 2-byte aligned
 * Errors: NULL, SHAPE (N < 1, K % 128, K > SVQ_MAX_K, G != 128), ALIGN, HIP.
 */
int gemv_w4a16(const uint8_t* packed, const uint16_t* x, uint16_t* y,
               int64_t N, int64_t K, int32_t G, void* stream);

/*
 * gemv_binplane -- DEVICE pointers, asynchronous on `stream`.
 * One decode step of a binary-plane linear layer (ShiftAddQwen README):
 *   y[n] = bf16_rne( sum_g sum_p alpha[p][n][g] * sum_{k in g} b[p][n][k] * x[k] ).
 * Pointers and errors as gemv_w4a16, plus P in 1..6.
 */
int gemv_binplane(const uint8_t* packed, const uint16_t* x, uint16_t* y,
                  int64_t N, int64_t K, int32_t G, int32_t P, void* stream);

/*
 * gemm_smallm_w4a16 -- DEVICE pointers, asynchronous on `stream`.
 * The target's pass over a drafted block of M <= 16 positions (DFlash
 * summary sec. 4.1: the drafted tokens are verified in parallel; report
 * sec. 3.2: block size 16):  Y[m][n] = the W4A16 result for row m of X.
 * Blocks of 16 < M <= 64 rows (a prefill chunk; the ShiftAddQwen README
 * places batches below 64 in the quantized mat-mul regime) take the same
 * kernel: with two 16-row tiles of X (M <= 32, K <= 4096, more row tiles
 * than CUs), or with each 16-row tile of the block on workgroups of its own
 * (other blocks at K <= 4096); above K = 4096, a kernel that streams X with
 * the weights.  The result is defined the same way.  Larger
 * blocks (up to SVQ_MAX_M_GEMM rows) run as consecutive launches of
 * SVQ_BLOCK_M rows each, each reading the weights once.
 *   X  [M][K] bf16 bits, 16-byte aligned;  Y [M][N] bf16 bits, 2-byte aligned.
 * Errors: as gemv_w4a16, plus SHAPE for M outside 1..SVQ_MAX_M_GEMM.
 */
int gemm_smallm_w4a16(const uint8_t* packed, const uint16_t* X, uint16_t* Y,
                      int32_t M, int64_t N, int64_t K, int32_t G, void* stream);

/*
 * gemm_smallm_binplane -- DEVICE pointers, asynchronous on `stream`.
 * Y[m][n] = the binary-plane result for row m of X, M in 1..SVQ_MAX_M_GEMM
 * (17..64 rows: as gemm_smallm_w4a16, the two-m-tile form taking up to four
 * planes; above 64, consecutive launches of SVQ_BLOCK_M rows).
 */
int gemm_smallm_binplane(const uint8_t* packed, const uint16_t* X, uint16_t* Y,
                         int32_t M, int64_t N, int64_t K, int32_t G, int32_t P,
                         void* stream);

/*
 * gemv_sa -- DEVICE pointers, asynchronous on `stream`.
 * One decode step of an sa* layer (ShiftAddQwen README, "Method / Format"):
 *   y[n] = bf16_rne( sum_j d[n][j] * sum_{g in j} sum_p a[p][n][g] * sum_{k in g} b[p][n][k] * x[k] ),
 * j over the 256-weight super-blocks, accumulated in fp32 and scaled by d
 * once per super-block.
 *   packed  sa blob, 16-byte aligned; x [K] bf16, 16-byte aligned; y [N] bf16
 * Errors: NULL, SHAPE (N < 1, K % 256, K > SVQ_MAX_K, G not in {64, 128, 256},
 * P outside 2..6), ALIGN, HIP.
 */
int gemv_sa(const uint8_t* packed, const uint16_t* x, uint16_t* y, int64_t N,
            int64_t K, int32_t G, int32_t P, void* stream);

/*
 * gemm_smallm_sa -- DEVICE pointers, asynchronous on `stream`.
 * Y[m][n] = the sa* result for row m of X, M in 1..SVQ_MAX_M_GEMM (the
 * verify pass over a drafted block, as gemm_smallm_w4a16; the README's
 * batches below 64 run its quantized mat-mul: 17..64 rows as
 * gemm_smallm_w4a16, the two-m-tile form taking up to four planes at
 * G >= 128; larger blocks consecutive launches of SVQ_BLOCK_M rows).
 * Errors: as gemv_sa, plus SHAPE for M outside 1..SVQ_MAX_M_GEMM.
 */
int gemm_smallm_sa(const uint8_t* packed, const uint16_t* X, uint16_t* Y,
                   int32_t M, int64_t N, int64_t K, int32_t G, int32_t P,
                   void* stream);

/*
 * lmhead_argmax -- DEVICE pointers, asynchronous on `stream`.
 * Greedy decision of a W4A16 LM head for M <= 16 query rows (DFlash summary
 * sec. 4.1; MTP study sec. 3.3):
 *   z[m][n]     = W4A16 logits (fp32, never written to memory)
 *   idx         = smallest n with z[m][n] == max_n z[m][n]
 *   argmax[m]   = row_ids ? row_ids[idx] : idx          (int32)
 *   maxlogit[m] = z[m][idx]                              (fp32)
 *   X          [M][K] bf16 bits, 16-byte aligned
 *   row_ids    NULL or [N] int32 (trimmed row -> token id), 4-byte aligned
 *   argmax, maxlogit  [M], 4-byte aligned
 *   workspace  >= svq_lmhead_workspace_bytes(M) bytes of device memory,
 *              16-byte aligned, all zero before the first call (allocate
 *              it zeroed).  Every call leaves it zero again, so one
 *              workspace serves any number of calls of any M.
 * One launch: each workgroup folds its per-row best (logit, row) into the
 * workspace with device-scope 64-bit atomic max operations (into the keys
 * of one of 16 groups when every workgroup owns at most 8 row tiles, whose
 * last workgroup then signals a launch counter); the last workgroup to
 * finish reads every group's keys, writes the result and clears the
 * workspace.
 * Errors: as gemm_smallm_w4a16, plus WORKSPACE.  Calls that overlap in time
 * must not share a workspace.
 */
int lmhead_argmax(const uint8_t* packed, const uint16_t* X, int32_t M,
                  int64_t N, int64_t K, int32_t G, const int32_t* row_ids,
                  int32_t* argmax, float* maxlogit, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * lmhead_argmax_noalloc -- DEVICE pointers, asynchronous on `stream`.
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * call and results as lmhead_argmax, without the workspace argument.  The
 * argmax completion state lives in a static device array of the library
 * (4352 bytes per GPU, held until the process ends); the call itself
 * allocates nothing.  On the first call on a device the array's address is
 * looked up and the array is cleared by a kernel on `stream`, ordered before
 * the head; every completed call leaves it zero again.
 *   X, row_ids, argmax, maxlogit  as lmhead_argmax
 * All calls on one GPU share that GPU's array: calls that overlap in time on
 * one GPU (on different streams, or from different threads) race and must
 * not be issued.
 * Errors: as lmhead_argmax without WORKSPACE; SHAPE for M outside 1..16 (the
 * largest block the array's state covers); HIP if the array's address cannot
 * be obtained.
 */
int lmhead_argmax_noalloc(const uint8_t* packed, const uint16_t* X, int32_t M,
                          int64_t N, int64_t K, int32_t G, const int32_t* row_ids,
                          int32_t* argmax, float* maxlogit, void* stream);

/*
 * lmhead_argmax_binplane -- DEVICE pointers, asynchronous on `stream`.
 * lmhead_argmax for a head stored as P sign planes (ShiftAddQwen README,
 * Method/Format; the MTP study sec. 3.3 for the trimmed head):
 *   z[m][n] = sum_g sum_p alpha[p][n][g] * sum_{k in g} b[p][n][k] * X[m][k]
 * with the same outputs, workspace contract and tie rule as lmhead_argmax.
 *   packed  binary-plane blob (layout above), 1 <= P <= 6
 * Errors: as gemm_smallm_binplane, plus WORKSPACE.
 */
int lmhead_argmax_binplane(const uint8_t* packed, const uint16_t* X, int32_t M,
                           int64_t N, int64_t K, int32_t G, int32_t P,
                           const int32_t* row_ids, int32_t* argmax,
                           float* maxlogit, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Greedy acceptance of a verified block (DFlash summary sec. 4.1: a cycle
 * drafts gamma tokens, the target checks them in one parallel pass and
 * accepts tau in [1, gamma + 1] tokens; the report's sec. 2.2 for parallel
 * verification).  The block holds M = gamma + 1 query rows
 * [anchor, d_1, ..., d_{M-1}]; row j's greedy token t_j is the target's
 * prediction for the position after row j, so d_{j+1} is accepted while every
 * earlier draft was accepted and t_j == d_{j+1}.  With a the number of
 * accepted drafts, tau = a + 1 and the tokens to emit are t_0 .. t_a (the
 * accepted drafts followed by the target's own next token).  A row without a
 * valid maximum (id -1) ends the accepted prefix.
 */

/*
 * lmhead_verify_greedy -- DEVICE pointers, asynchronous on `stream`.
 * lmhead_argmax over the block, then, in the same launch (the workgroup that
 * completes the argmax), greedy acceptance:
 *   draft_ids   [M-1] int32 token ids d_1 .. d_{M-1}, 4-byte aligned; may be
 *               NULL when M == 1
 *   accept_len  [1] int32: tau; argmax[0 .. tau-1] are the tokens to emit
 * Other arguments, the workspace contract and errors as lmhead_argmax.
 */
int lmhead_verify_greedy(const uint8_t* packed, const uint16_t* X, int32_t M,
                         int64_t N, int64_t K, int32_t G,
                         const int32_t* row_ids, const int32_t* draft_ids,
                         int32_t* argmax, float* maxlogit, int32_t* accept_len,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * verify_greedy -- DEVICE pointers, asynchronous on `stream`.
 * Greedy acceptance alone, for target tokens produced elsewhere:
 *   target_ids  [M] int32 t_0 .. t_{M-1}
 *   draft_ids   [M-1] int32 d_1 .. d_{M-1} (may be NULL when M == 1)
 *   accept_len  [1] int32: tau
 * 1 <= M <= 16; pointers 4-byte aligned.
 * Errors: NULL, SHAPE (M), ALIGN, HIP.
 */
int verify_greedy(const int32_t* target_ids, const int32_t* draft_ids,
                  int32_t M, int32_t* accept_len, void* stream);

/*
 * svq_stream_read -- DEVICE pointers, asynchronous on `stream`.
 * Measurement aid, not part of the method: reads `bytes` (a positive
 * multiple of 16 below 2 GiB) from `src` with non-temporal 16-byte loads,
 * eight per thread in flight, on wgs_per_cu workgroups of 256 threads per
 * CU (0 means 1; at most 8), and writes one uint32 checksum per workgroup
 * into `sink` (>= 8 * CUs * 4 bytes).  Gives the achievable streaming-read
 * ceiling for a buffer of that size and the counter calibration.
 * Errors: NULL, SHAPE (size, wgs_per_cu), ALIGN (src 16-byte, sink 4-byte),
 * HIP.
 */
int svq_stream_read(const void* src, size_t bytes, uint32_t* sink,
                    int32_t wgs_per_cu, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SVQ_H */
