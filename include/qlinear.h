/*
 * qlinear.h -- C ABI of the ThinkBit low-bit GEMV/GEMM library for MI355X (gfx950).
 *
 * Weight format (ThinkBit summary page, onedev.kr/papers/1416, section "How it
 * works"): every weight is an integer codeword c times a bf16 scale s shared by
 * 128 consecutive input-dimension weights; the codeword grid is ternary
 * {-1,0,1}, 2-bit {-2,-1,0,1} or 3-bit {-4,...,3}; dequantization is one
 * multiply, with no codebook, rotation or zero point.  The same page (section
 * "Premises & limits") notes that published checkpoints keep the codewords in
 * 4-bit containers because kernels that read 2- and 3-bit codes directly do
 * not exist; this library reads them at 1.6, 2 and 3 bits.
 *
 * Notation: W is [N][K] (N output rows, K input columns, K % 128 == 0),
 * x is [M][K] bf16, y = x * W^T is [M][N] fp32.
 *
 * Packed layout, version 2 (this project's definition; the pages fix no bit
 * order).  u = c - c_min is stored (ternary c+1, 2-bit c+2, 3-bit c+4).
 *   row bytes: ternary 16*ceil(K/80); 2-bit K/4; 3-bit 3K/8.
 *   ternary: byte j of a row holds inputs 5j..5j+4 as a base-3 number,
 *            byte = sum_{i<5} u[k(j,i)] * 3^i, with k(j,i) = 5j+i for even j
 *            and, for odd j, k(j,i) = 5j+1+i (i < 4), k(j,4) = 5j.  Read as a
 *            pair, bytes 2q, 2q+1 then hold every even-aligned input pair of
 *            10q..10q+9 as adjacent digits except (10q+4, 10q+5), so a kernel
 *            can multiply decoded code pairs against aligned activation pairs.
 *            Trits past K are padding with c = 0; bytes <= 242.
 *   2-bit:   little-endian 32-bit word j holds k = 16j+i at bits [2i, 2i+1].
 *   3-bit:   96-bit triple t (words w0,w1,w2 read as w0 | w1<<32 | w2<<64)
 *            holds k = 32t+i at bits [3i, 3i+2].
 *   slabs:   rows are grouped in slabs of 64; within a slab the bytes run
 *            chunk-major: bytes 16c..16c+15 of row r of the slab sit at
 *            c*1024 + r*16.  Rows past N are padding (all c = 0).
 *   grids:   one grid per block of 128 rows.  A packed matrix is its blocks
 *            concatenated in row order, each in its own grid's layout; block b
 *            holds min(2, slabs left) slabs and starts at byte blk_off[b].
 *            A uniform matrix is the special case with one grid everywhere.
 *   scales:  bf16 bits; the packed scale array stores scale (n, g) at element
 *            ((n/64 * G8 + g/8) * 64 + n%64) * 8 + g%8, G = K/128,
 *            G8 = ceil(G/8); unused entries are 0.  Scales sit apart from the
 *            codes, so recalibrated scales can be written without repacking.
 *
 * Conventions for every entry point:
 *   - Pointers marked (dev) are device memory owned by the caller; (host) are
 *     host memory.  The library allocates nothing and never synchronizes;
 *     device calls are enqueued on `stream` (0 = the null stream).
 *   - Arguments are checked before anything is enqueued; a bad argument
 *     returns QL_EINVAL (or QL_EUNSUPPORTED) and enqueues nothing.  A failed
 *     launch returns QL_EHIP.  qlinear_last_error() describes the last failure
 *     of the calling thread.
 *   - Device pointers must be 16-byte aligned; y and every output must not
 *     alias an input.
 *   - Codes outside the grid, ternary bytes above 242 and non-finite inputs
 *     are outside the contract (undefined results, never out-of-bounds
 *     accesses).
 *   - GEMV results are bitwise deterministic for a given launch shape.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QL_GROUP 128 /* weights per scale, along K */
#define QL_SLAB 64   /* rows per interleaved slab */
#define QL_BLOCK 128 /* rows per grid block */
#define QL_LAYOUT_VERSION 2

typedef enum { QL_GRID_T = 0, QL_GRID_I2 = 1, QL_GRID_I3 = 2, QL_GRID_MIXED = 3 } ql_grid;
typedef enum { QL_OK = 0, QL_EINVAL = 1, QL_EUNSUPPORTED = 2, QL_EHIP = 3 } ql_status;

/* Library and layout version (QL_LAYOUT_VERSION). */
int qlinear_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *qlinear_last_error(void);

/* ---------------------------------------------------------------- sizes (host only, no GPU) */

/* Bytes of one packed row of grid T/I2/I3 (multiple of 16); 0 if the grid or K is invalid. */
int64_t qlinear_row_bytes(int grid, int64_t K);

/* Byte offset of every grid block of a packed N x K matrix.  blk_grid (host, ceil(N/128)
 * entries) holds the grid of each block; off (host, ceil(N/128)+1 entries) receives the
 * offsets, off[nblk] being the total packed size. */
ql_status qlinear_block_offsets(int64_t N, int64_t K, const int8_t *blk_grid, int64_t *off);

/* Packed size of an N x K matrix of one uniform grid (bytes); 0 if invalid. */
int64_t qlinear_packed_bytes(int64_t N, int64_t K, int grid);

/* Elements (bf16) of the packed scale array of an N x K matrix; 0 if invalid. */
int64_t qlinear_packed_scales_len(int64_t N, int64_t K);

/* ---------------------------------------------------------------- quantize / pack (device) */

/* Round-to-nearest quantization of fp32 weights, the rule of the synthetic workloads:
 * per row n and group g, s = bf16_rne(max|W[n,g*128..g*128+127]| / |c_min|), and
 * c = clamp(rint(W / s), c_min, c_max) with the quotient in fp64 and ties to even
 * (c = 0 where s = 0).  Re-rounding with a stored scale reproduces stored codes (k-quant
 * calibration page, sotaaz.com/post/quantized-model-less-sure, section "Open question").
 *   grid: QL_GRID_T/I2/I3, or QL_GRID_MIXED with blk_grid (dev, ceil(N/128) int8) giving
 *         the grid of each 128-row block (ignored otherwise, may be NULL).
 *   W (dev) fp32 [N][K]; codes (dev) int8 [N][K]; scales (dev) bf16 bits [N][K/128]. */
ql_status qlinear_quantize(int64_t N, int64_t K, int grid, const int8_t *blk_grid, const float *W,
                           int8_t *codes, uint16_t *scales, hipStream_t stream);

/* Pack a quantized weight (summary page, section "How it works": codes c and one bf16 scale
 * per 128 inputs) into the layout above: codes int8 [N][K] (dev) -> packed (dev, the packed
 * size), and scales bf16 bits [N][K/128] (dev) -> pscales (dev, qlinear_packed_scales_len
 * elements), the packed scale array that the products read.  grid/blk_grid as for quantize;
 * blk_off (dev, ceil(N/128)+1 int64, from qlinear_block_offsets) is required for
 * QL_GRID_MIXED and ignored otherwise.  scales and pscales may both be NULL (codes only). */
ql_status qlinear_pack(int64_t N, int64_t K, int grid, const int8_t *blk_grid, const int64_t *blk_off,
                       const int8_t *codes, const uint16_t *scales, void *packed, uint16_t *pscales,
                       hipStream_t stream);

/* Scales bf16 [N][K/128] (dev) -> packed scale array (dev, qlinear_packed_scales_len elements);
 * the scale half of qlinear_pack, for scales recalibrated without repacking the codes. */
ql_status qlinear_pack_scales(int64_t N, int64_t K, const uint16_t *scales, uint16_t *pscales,
                              hipStream_t stream);

/* Inverse of qlinear_pack for the N real rows: codes int8 [N][K] (dev). */
ql_status qlinear_unpack(int64_t N, int64_t K, int grid, const int8_t *blk_grid, const int64_t *blk_off,
                         const void *packed, int8_t *codes, hipStream_t stream);

/* Inverse of qlinear_pack_scales: scales bf16 [N][K/128] (dev). */
ql_status qlinear_unpack_scales(int64_t N, int64_t K, const uint16_t *pscales, uint16_t *scales,
                                hipStream_t stream);

/* Dequantize (summary page, "How it works": one multiply): out[n][k] = c * s as fp32
 * (exact) when out_bf16 == 0, or bf16_rne(c * s) bits when out_bf16 != 0.  out (dev) [N][K]. */
ql_status qlinear_dequant(int64_t N, int64_t K, int grid, const int8_t *blk_grid, const int64_t *blk_off,
                          const void *packed, const uint16_t *pscales, int out_bf16, void *out,
                          hipStream_t stream);

/* ---------------------------------------------------------------- data validation (device)
 *
 * The products leave codes outside the grid, ternary bytes above 242 and bad padding outside
 * their contract (undefined results, never an out-of-bounds access).  These checks find such
 * data (summary page, section "How it works": the three grids' value sets; a base-3 byte of
 * five trits is at most 242) and ADD their counts to counts (dev, 4 uint32, 16-byte aligned,
 * zeroed by the caller): counts[0] codes outside their row's grid (ternary bytes above 242 in
 * packed data), counts[1] padding that does not code c = 0 (rows past N, trits past K),
 * counts[2] 128-row blocks whose blk_grid entry is not a grid (such blocks are skipped),
 * counts[3] unused (0).  Read counts back after the stream reaches the call. */
ql_status qlinear_validate_codes(int64_t N, int64_t K, int grid, const int8_t *blk_grid, const int8_t *codes,
                                 uint32_t *counts, hipStream_t stream);
ql_status qlinear_validate_packed(int64_t N, int64_t K, int grid, const int8_t *blk_grid, const int64_t *blk_off,
                                  const void *packed, uint32_t *counts, hipStream_t stream);

/* ---------------------------------------------------------------- products (device) */

/* Decode-time GEMV of one matrix, 1 <= M <= 16 (the per-token weight stream that the
 * summary page, section "What it is", names as the bandwidth-bound step of decoding):
 * y[m][n] = sum_k c[n][k] * s[n][k/128] * x[m][k].  Codes are read at 1.6/2/3 bits with
 * 128-bit loads, one lane per weight row, and decoded once for all M tokens through LDS
 * tables into bf16; the products c*x are exact and run on MFMA with fp32 sums, each
 * scale applied once per 128-input group.  K must be at most 2^26.  The kernel is the
 * grouped launch's (qlinear_gemv_grouped) without its task queues or split-K.
 *   x (dev) bf16 bits [M][K]; y (dev) fp32 [M][N]. */
ql_status qlinear_gemv(int64_t M, int64_t N, int64_t K, int grid, const int8_t *blk_grid,
                       const int64_t *blk_off, const void *packed, const uint16_t *pscales,
                       const uint16_t *x, float *y, hipStream_t stream);

/* One entry of a grouped GEMV launch: an independent y = x * W^T on its own matrix. */
typedef struct {
  const void *packed;       /* (dev) packed codes */
  const uint16_t *pscales;  /* (dev) packed scales */
  const int8_t *blk_grid;   /* (dev) per-block grids, QL_GRID_MIXED only (else NULL) */
  const int64_t *blk_off;   /* (dev) block offsets, QL_GRID_MIXED only (else NULL) */
  const uint16_t *x;        /* (dev) bf16 bits [M][K] */
  float *y;                 /* (dev) fp32 [M][N] */
  int32_t N, K, grid;       /* shape and grid (QL_GRID_*) */
  int32_t slab_begin;       /* filled by prepare: the entry's first task */
  int32_t kparts;           /* split-K parts per slab: in (prepare_split), 0 = choose, else forced;
                               out, the parts used (1 = no split) */
  int32_t reserved;         /* 0 */
  int64_t ws_begin;         /* filled by prepare: first word of the entry's split-K state in the
                               launch's state buffer (0 when kparts == 1) */
} ql_gemv_desc;

/* Prepare a descriptor list (host array) for qlinear_gemv_grouped (or, for a list of 4-bit
 * containers, qlinear_c4_gemv_grouped; a list must not mix the two): check every entry, sort
 * the entries by task length (K / kparts; here kparts = 1, so by K), largest first (stable;
 * the products are independent, so their order is free), fill slab_begin and return the
 * total number of 64-row slabs (the task count), or -1 on a bad descriptor (K above 2^26
 * included: the GEMV kernel addresses 16 tokens' activations in one 32-bit range).  Longest-first task order plus dynamic task fetching keeps
 * the persistent launch balanced when row lengths differ (a K = 12288 row costs three
 * K = 4096 rows).  Entries of equal K keep the caller's order: listing them by stored
 * bytes per row, largest first (3-bit before 2-bit before ternary), ends the launch on
 * its cheapest tasks. */
int64_t qlinear_grouped_prepare(ql_gemv_desc *descs, int32_t count);

/* Largest number of split-K parts per slab (the last part's wave sums every part). */
#define QL_MAX_KPARTS 16

/* Split-K for launches with few slabs (one matrix, or the few of one layer: a 4096-row
 * matrix has 64 slabs, one per wave, on a device with thousands of wave slots).  As
 * qlinear_grouped_prepare, but the input of every slab may be cut into kparts parts of
 * whole 640-input periods, each part a task of its own; the wave that finishes a slab's
 * last part sums the parts' fp32 partial sums in part order, so results stay bitwise
 * deterministic.  An entry with kparts > 0 keeps that many parts (at most its period
 * count and QL_MAX_KPARTS); for kparts == 0 the parts are chosen so that the launch has
 * at least min_tasks tasks where rows allow (e.g. half of qlinear_grouped_wave_slots(M);
 * min_tasks <= 0 splits nothing).  Entries are sorted by task length K / kparts, longest
 * first (stable).  A list of 4-bit containers
 * is never split.  *state_words (host) receives the size of the launch's state buffer in
 * 32-bit words: QL_SCHED_WORDS, plus, per split entry, one 128-byte counter line per slab
 * and 1024 words of partial sums per part of each slab.  Returns the task count, or -1. */
int64_t qlinear_grouped_prepare_split(ql_gemv_desc *descs, int32_t count, int64_t min_tasks,
                                      int64_t *state_words);

/* Waves a grouped launch at batch size M (1..16) runs on the current device at most (the
 * persistent grid), or -1 if M is out of range or the device cannot be queried. */
int64_t qlinear_grouped_wave_slots(int32_t M);

/* Words of the task-scheduler state of a grouped launch: 64 task-queue counters and 64
 * check-out counters, each in its own 128-byte line, and a check-out word.  Draws and
 * check-outs spread over many counters because atomics on one shared address serialize
 * across the whole device. */
#define QL_SCHED_WORDS 4128

/* Run every GEMV of a prepared descriptor list (copied to device memory by the caller,
 * descs (dev), count entries) in one persistent launch, at one batch size M for all entries
 * (1 <= M <= 16; each x is M x K, each y M x N).  Every M runs one kernel: lane =
 * weight row (as in qlinear_gemv), products on 4x4x4 MFMA with the
 * activations of four tokens at a time broadcast to every row block.  It decodes each
 * packed byte once for all M tokens (products exact, fp32 sums; summary page, section
 * "What it is": a decode step at a small batch still streams every weight once).  M outside 1..16 returns QL_EINVAL.  Waves take tasks (64-row slabs, or parts of them after prepare_split) from
 * atomic queue counters in the state buffer `sched` (dev, 16-byte aligned, owned by the
 * caller; QL_SCHED_WORDS uint32 after qlinear_grouped_prepare, the state_words reported by
 * qlinear_grouped_prepare_split otherwise): its counters must be all zero when a launch
 * starts, and every launch that runs to completion leaves them zero again, so one zeroing
 * at allocation serves any number of launches.  Launches that share one state buffer must
 * not overlap (enqueue them on one stream).  total_tasks and the state buffer's size must be
 * the ones prepare reported for this list: tasks past an entry's own range are dropped on the
 * device, but a state buffer smaller than state_words is not detected.  The products are independent: no y may alias
 * another entry's x or y. */
ql_status qlinear_gemv_grouped(const ql_gemv_desc *descs, int32_t count, int64_t total_tasks, int32_t M,
                               uint32_t *sched, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): qlinear_gemv_grouped without the caller's state
 * buffer.  The task counters and split-K partial sums live in a static device array of the
 * library, QL_NOALLOC_STATE_WORDS uint32 (16 MiB) per GPU, held until the process ends.
 * state_words is what qlinear_grouped_prepare (QL_SCHED_WORDS) or qlinear_grouped_prepare_split
 * reported for the descriptor list; a launch that needs more than the array holds is rejected
 * with QL_EINVAL before anything is enqueued.  The first call on a GPU clears the array with a
 * fill kernel on `stream`; every completed launch leaves its counters zero again.  Every call on
 * one GPU shares that GPU's array, so calls that overlap on one GPU (different streams, or
 * other threads) race and give wrong results: serialize them on one stream.  Same kernels and
 * results as qlinear_gemv_grouped for the same list.  Allocates nothing. */
#define QL_NOALLOC_STATE_WORDS 4194304
ql_status qlinear_gemv_grouped_noalloc(const ql_gemv_desc *descs, int32_t count, int64_t total_tasks, int32_t M,
                                       int64_t state_words, hipStream_t stream);

/* Batched GEMM for 1 <= M (tuned for 16..512): tiles of codes are decoded into LDS as bf16
 * and contracted on MFMA (bf16 x bf16 -> fp32).  Below 16 tokens the tile holds the exact
 * codes and the group scale multiplies each 128-deep partial product in fp32; from 16 tokens
 * on it holds RNE(c * s) in bf16 (exact except 3-bit codes of magnitude 3).  Dequantizing to
 * bf16 and computing in bf16 reproduces the native low-bit result (k-quant calibration page,
 * section "Not just any noise").  workspace (dev) of qlinear_gemm_workspace_bytes(M, N, K)
 * bytes (may be 0): the K-split partial sums, added by a second kernel in split order. */
size_t qlinear_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
ql_status qlinear_gemm(int64_t M, int64_t N, int64_t K, int grid, const int8_t *blk_grid,
                       const int64_t *blk_off, const void *packed, const uint16_t *pscales,
                       const uint16_t *x, float *y, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* Grouped GEMM: many independent y = x * W^T products at one M (16 <= M < 2^24; each x M x K
 * bf16 bits, each y M x N fp32), e.g. the seven linears of a decoder layer at a prefill or
 * batched-decode size, in one persistent launch of qlinear_gemm's large-tile kernel (same
 * operands, same bar) plus, when any entry is split, one reduction launch.  Workgroups take
 * 256-row x (64, 128 or 256)-token tiles of all entries round-robin, longest first, so small
 * matrices no longer leave most of the device idle and K is split only where that shortens
 * the launch (the launch also needs no per-matrix reduction pass).
 *
 * qlinear_gemm_grouped_prepare (host) checks every descriptor (ql_gemv_desc: packed, pscales,
 * blk_grid/blk_off for mixed grids, x, y, N, K, grid; kparts and reserved are ignored), chooses
 * each entry's K splits for this M and this device, reorders the array (longest tasks first),
 * fills slab_begin (the entry's first task), kparts (its splits) and ws_begin (the first float
 * of its partial sums in the workspace), stores the workspace size in *workspace_bytes (0 when
 * nothing is split) and returns the task count, or -1 (qlinear_last_error()) on a bad
 * descriptor or M.  The plan depends on M: prepare again for another M.
 *
 * qlinear_gemm_grouped runs a prepared list (copied to device memory by the caller: descs
 * (dev), count entries) with that M and task count; workspace (dev, 16-byte aligned, owned by
 * the caller, contents need not be zeroed) of the prepared size.  An entry whose partial sums
 * would not fit workspace_bytes computes nothing (its y is left as it was); tasks past an
 * entry's own range are dropped.  No y may alias another entry's x or y.  Results are
 * bitwise reproducible for a given prepared list. */
int64_t qlinear_gemm_grouped_prepare(ql_gemv_desc *descs, int32_t count, int64_t M,
                                     int64_t *workspace_bytes);
ql_status qlinear_gemm_grouped(const ql_gemv_desc *descs, int32_t count, int64_t total_tasks, int64_t M,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- grid allocation (offline)
 *
 * Summary page, section "How it differs", stage 1 (Allocate): the sensitivity S of a layer
 * (product of the squared norms of its input activations and of its output gradients) times
 * the rounding noise of a grid approximates the loss increase of storing the layer on that
 * grid; one grid per layer is chosen under a bit budget for the whole decoder, a
 * multiple-choice knapsack solved by Lagrangian relaxation.  A unit here is any set of rows
 * the caller groups (a linear, or a 128-row grid block of one). */
typedef struct {
  int64_t weights;      /* weights in the unit, > 0 */
  double sensitivity;   /* S >= 0 */
  double noise[3];      /* rounding noise of grids T, I2, I3 (each >= 0), e.g. from qlinear_rtn_noise */
  uint32_t allowed;     /* bit g set: grid g may be chosen (nonzero; e.g. 6 keeps a unit at >= 2 bits) */
  uint32_t reserved;    /* 0 */
} ql_alloc_unit;

/* Rounding noise of round-to-nearest (the rule of qlinear_quantize) onto each grid, per
 * 128-row block: noise[b*3 + g] = sum over block b's weights of (w - c*s)^2 in fp64.
 * W (dev) fp32 [N][K]; noise (dev) double [ceil(N/128)][3].  Deterministic. */
ql_status qlinear_rtn_noise(int64_t N, int64_t K, const float *W, double *noise, hipStream_t stream);

/* Sensitivity of every 128-row block of a linear (summary page, section "How it differs",
 * stage 1: the product of the squared norms of the input activations and of the output
 * gradients), restricted to the block's output rows: S[b] = (sum_k x[k]^2) *
 * (sum_{n in block b} grad[n]^2), each sum in fp64 in ascending index order (deterministic).
 *   x (dev) bf16 bits [K]; grad (dev) fp32 [N]; S (dev) double [ceil(N/128)]. */
ql_status qlinear_block_sensitivity(int64_t N, int64_t K, const uint16_t *x, const float *grad, double *S,
                                    hipStream_t stream);

/* Lagrangian multiple-choice knapsack (host only, no GPU).  For a multiplier lam >= 0 every
 * unit takes the allowed grid minimising S*noise[g] + lam*weights*grid_bits[g] (ties to fewer
 * bits); the result is the assignment at the smallest lam whose total bits fit
 * budget_bits * (sum of weights).  That assignment is optimal among all assignments using no
 * more bits than it does (it may leave part of the budget unused: the relaxation's gap).
 *   units (host, count); grid_bits (host, 3 values, bits per weight of T, I2, I3 including
 *   the scale; NULL = log2(3) + 1/8, 2 + 1/8, 3 + 1/8); grid_out (host, count) receives the
 *   grid of each unit; lambda_out (host, may be NULL) the multiplier.
 * Returns QL_EINVAL on bad input or when even the cheapest allowed grids exceed the budget. */
ql_status qlinear_allocate(const ql_alloc_unit *units, int64_t count, double budget_bits, const double *grid_bits,
                           int8_t *grid_out, double *lambda_out);

/* ---------------------------------------------------------------- LittleBit (binary factorized linear)
 *
 * LittleBit digest page (seosoyoung.eiaserinnys.me/digest/littlebit-ultra-low-bit-quantization),
 * sections "LittleBit's structure" and "Rank sets the BPW": a linear W (d_out x d_in) is the sum
 * of a primary and a residual path, each diag(h) U_sign diag(l) V_sign^T diag(g) with +-1
 * matrices U_sign (d_out x r), V_sign (d_in x r) and 16-bit scales h (d_out), g (d_in), l (r);
 * y = sum over paths of ((((x . g) V_sign) . l) U_sign^T) . h.  Bits per original weight:
 * b = ((2r + 32)(d_out + d_in) + 32r) / (d_out d_in).
 * Layout (this project's): a sign is one bit, 1 for -1; bit t of byte B of a row is element
 * 8B + t; rows are interleaved in 64-row slabs as the packed layout (bytes 16c..16c+15 of slab
 * row q at c*1024 + q*16).
 *   v_bits: V_sign^T as latent rows of d_in bits: path 0's r rows, then path 1's, each path
 *           padded to a multiple of 64 rows (qlinear_lb_v_bytes).
 *   u_bits: d_out rows, each path 0's r bits then path 1's, each part padded to a multiple of
 *           128 bits (qlinear_lb_u_bytes).  Padding bits and rows are 0.
 *   scales: bf16 bits g [2][d_in], l [2][r], h [2][d_out] (path 0 first).
 * Requirements: d_in % 128 == 0, d_out >= 1, rank >= 1. */
typedef struct {
  int32_t d_out, d_in, rank;  /* rank r of each path */
  int32_t reserved;           /* 0 */
  const void *u_bits;         /* (dev) */
  const void *v_bits;         /* (dev) */
  const uint16_t *g;          /* (dev) bf16 [2][d_in] */
  const uint16_t *l;          /* (dev) bf16 [2][rank] */
  const uint16_t *h;          /* (dev) bf16 [2][d_out] */
} ql_littlebit;

/* Bits per original weight of a two-path LittleBit linear of rank r (host, no GPU). */
double qlinear_lb_bpw(int64_t d_out, int64_t d_in, int64_t rank);
/* Largest rank whose bits per weight do not exceed bpw (0 if none). */
int64_t qlinear_lb_rank(int64_t d_out, int64_t d_in, double bpw);
/* Sizes of the two sign buffers (bytes); 0 if the shape is invalid. */
int64_t qlinear_lb_u_bytes(int64_t d_out, int64_t rank);
int64_t qlinear_lb_v_bytes(int64_t d_in, int64_t rank);

/* Pack signs into the layout above.  u_signs (dev) int8 [2][d_out][rank], v_signs (dev) int8
 * [2][d_in][rank], entries +-1 (anything negative counts as -1); u_bits, v_bits (dev). */
ql_status qlinear_lb_pack(int64_t d_out, int64_t d_in, int64_t rank, const int8_t *u_signs,
                          const int8_t *v_signs, void *u_bits, void *v_bits, hipStream_t stream);

/* Batch-1 product y [d_out] fp32 = the two-path LittleBit linear applied to x [d_in] bf16.
 * Products are exact (sign flips of bf16 values), sums fp32 in a fixed order: deterministic.
 * w (host struct holding device pointers); workspace (dev, 16-byte aligned) of
 * qlinear_lb_workspace_bytes: it holds per-slab counters that must be zero when the first
 * call starts; every completed call leaves them zero again (zero the workspace once at
 * allocation).  Calls that share a workspace must not overlap (enqueue them on one stream). */
size_t qlinear_lb_workspace_bytes(int64_t d_out, int64_t d_in, int64_t rank);
ql_status qlinear_lb_gemv(const ql_littlebit *w, const uint16_t *x, float *y, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- 4-bit container baseline
 *
 * The summary page (onedev.kr/papers/1416, section "Premises & limits") says the
 * published checkpoints hold the 1.6/2/3-bit codewords in 4-bit containers, and that this
 * forfeits the memory and speed advantage.  These entry points store and multiply that
 * format on the same GPU, so the two can be compared on equal terms:
 *   container: code c (-8..7; every ThinkBit grid fits) as a two's complement nibble,
 *              row bytes K/2, byte i of a row holding input 2i in its low nibble and
 *              input 2i+1 in its high nibble; rows interleaved in 64-row slabs exactly as
 *              the packed layout (bytes 16c..16c+15 of slab row r at c*1024 + r*16), so the
 *              only difference to the packed layout is the number of bits per code.
 *              Size ceil(N/64)*64*K/2 bytes; rows past N are zero.
 *   scales:    the same packed scale array as the native layout.
 * QL_GRID_C4 marks a container in a ql_gemv_desc; it is not a ThinkBit grid and the native
 * entry points reject it. */
#define QL_GRID_C4 4

/* Container size of an N x K matrix (bytes); 0 if the shape is invalid. */
int64_t qlinear_c4_bytes(int64_t N, int64_t K);

/* Codes int8 [N][K] (dev, each in -8..7) -> container (dev, qlinear_c4_bytes). */
ql_status qlinear_c4_pack(int64_t N, int64_t K, const int8_t *codes, void *c4, hipStream_t stream);

/* Container (dev) -> codes int8 [N][K] (dev). */
ql_status qlinear_c4_unpack(int64_t N, int64_t K, const void *c4, int8_t *codes, hipStream_t stream);

/* Converter from a container checkpoint to the native packed layout: reads every code from
 * the container and writes it as qlinear_pack would (grid, blk_grid, blk_off as there; the
 * codes must lie in their block's grid).  packed (dev) has the packed size. */
ql_status qlinear_c4_to_packed(int64_t N, int64_t K, int grid, const int8_t *blk_grid,
                               const int64_t *blk_off, const void *c4, void *packed,
                               hipStream_t stream);

/* Batch-1 GEMV on a container: y[n] = sum_k c[n][k] * s[n][k/128] * x[k], M must be 1.
 * Same numerics as qlinear_gemv (exact c*x products, fp32 sums per group, one scale
 * multiply per group).  c4, pscales, x, y (dev). */
ql_status qlinear_c4_gemv(int64_t M, int64_t N, int64_t K, const void *c4, const uint16_t *pscales,
                          const uint16_t *x, float *y, hipStream_t stream);

/* Grouped batch-1 GEMV over containers: as qlinear_gemv_grouped, for a descriptor list
 * whose every entry has grid QL_GRID_C4 and packed pointing at a container (prepared by
 * qlinear_grouped_prepare, which rejects lists mixing containers and native grids).
 * Entries of another grid are skipped on the device (their y is not written). */
ql_status qlinear_c4_gemv_grouped(const ql_gemv_desc *descs, int32_t count, int64_t total_slabs, int32_t M,
                                  uint32_t *sched, hipStream_t stream);

/* ---------------------------------------------------------------- measurement */

/* Pure HBM read probe, the measured bandwidth ceiling beside the nominal 8 TB/s: streams
 * `bytes` (a positive multiple of 1024, below 2^32) of device memory at buf (dev, 16-byte
 * aligned) with 128-bit non-temporal loads, 1 KB blocks interleaved across all waves, and
 * folds it into out (dev, 256 uint32, 16-byte aligned): word 4 l + j is XORed with dword j of
 * bytes 16 l .. 16 l + 15 of every block (so a zeroed out afterwards holds the XOR over the
 * blocks).  The atomic fold makes out order-independent; calls that share out must not
 * overlap unless their XORs may combine. */
ql_status qlinear_read_probe(const void *buf, int64_t bytes, uint32_t *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
