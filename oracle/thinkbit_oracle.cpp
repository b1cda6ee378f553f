// ThinkBit CPU oracle — TEST INFRASTRUCTURE ONLY.
//
// This file is the plain, slow reference that the HIP library is checked
// against.  Only the test suite, the smoke entry point and the CPU-baseline
// leg of the benchmark may load it.  It shares no source with the GPU path
// (no headers, tables or helpers in common); the two meet only through the
// seeded synthetic inputs.
//
// What it computes (each function cites the passage it follows):
//   * ThinkBit summary page (onedev.kr/papers/1416), section "How it works":
//     every weight is an integer codeword c times a bf16 scale s shared by
//     128 weights; the codeword grid is ternary {-1,0,1}, 2-bit {-2..1} or
//     3-bit {-4..3}; dequantization is one multiply; no codebooks, rotations
//     or zero points.
//   * The synthetic workload's quantizer: s = max|w| / |c_min| over a group
//     of 128 consecutive input-dim weights, rounded to bf16, and
//     c = clamp(round(w / s), c_min, c_max).  Re-rounding with a stored
//     scale is the operation the k-quant calibration page
//     (sotaaz.com/post/quantized-model-less-sure, section "Open question")
//     shows to reproduce stored codes exactly.
//   * The packed layout, version 2 (five trits per byte in base 3 with the
//     digit order of tern_input below, sixteen 2-bit codes per 32-bit word,
//     thirty-two 3-bit codes per 96-bit triple, 64-row slabs, 128-row grid
//     blocks) is this project's own definition; the pages fix no bit order.
//     It is written out once more, independently, in the HIP packer.
//   * LittleBit (digest page seosoyoung.eiaserinnys.me/digest/littlebit-
//     ultra-low-bit-quantization): the two-path binary factorized linear,
//     its bits-per-weight formula and its forward pass.
//   * The grid allocation of the same page, section "How it differs"
//     (stage 1): rounding noise per grid, and a multiple-choice knapsack
//     over grids under a bit budget solved by Lagrangian relaxation.
//   * The 4-bit container the summary page (section "Premises & limits")
//     says published checkpoints use, as the baseline format: codes as
//     two's complement nibbles in the same slab interleave.
//
// Precision: codes are decided from an fp64 quotient; w = c*s is formed in
// fp32 (exact: at most 11 significant bits); products and sums are fp64,
// summed in ascending k.
//
// Readings where the pages are silent (listed with reasons in the design
// notes): tie-break of round() is half-to-even; an all-zero group has s = 0
// and all codes 0; NaN/Inf weights are rejected; trits past K are padding
// with c = 0; padding rows of a slab have c = 0 and s = 0.

#include <cstdint>
#include <cstring>
#include <cmath>
#include <thread>
#include <vector>
#include <algorithm>
#include <functional>

namespace {

constexpr int kGroup = 128;   // weights per scale (input dimension)
constexpr int kSlab = 64;     // rows interleaved per slab
constexpr int kBlock = 128;   // rows sharing one grid in a mixed matrix
constexpr int kChunk = 16;    // bytes per row per slab step

enum { GRID_T = 0, GRID_I2 = 1, GRID_I3 = 2 };

int cmin_of(int grid) { return grid == GRID_T ? -1 : grid == GRID_I2 ? -2 : -4; }
int cmax_of(int grid) { return grid == GRID_T ? 1 : grid == GRID_I2 ? 1 : 3; }
bool grid_ok(int grid) { return grid == GRID_T || grid == GRID_I2 || grid == GRID_I3; }

// IEEE-754 binary32 -> bfloat16, round to nearest, ties to even.
uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // NaN
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

int64_t row_bytes_of(int grid, int64_t K) {
  if (!grid_ok(grid) || K <= 0 || K % kGroup) return 0;
  if (grid == GRID_T) return 16 * ((K + 79) / 80);  // 80 trits per 16 bytes, padded
  if (grid == GRID_I2) return K / 4;                // 2 bits per code
  return 3 * K / 8;                                 // 3 bits per code
}

// Code of row n at input index k, or 0 past K (padding).
inline int code_at(const int8_t* codes, int64_t K, int64_t n, int64_t k) {
  return k < K ? codes[n * K + k] : 0;
}

// Ternary digit order (layout version 2).  Byte j holds the five inputs
// 5j..5j+4.  In an even byte, digit i (weight 3^i) is input 5j+i.  In an odd
// byte, digits 0..3 are inputs 5j+1..5j+4 and digit 4 is input 5j.  Read as a
// pair, bytes 2q and 2q+1 cover inputs 10q..10q+9, and every even-aligned input
// pair (2t, 2t+1) except (10q+4, 10q+5) lies inside one byte in digit order;
// the pages fix no order within a byte, so this one is chosen to line pairs up.
inline int64_t tern_input(int64_t j, int i) {
  if ((j & 1) == 0) return 5 * j + i;
  return i < 4 ? 5 * j + 1 + i : 5 * j;
}

// Bytes of one row in the grid's own order (before slab interleave).
void pack_row(int grid, int64_t K, const int8_t* codes, int64_t n, uint8_t* out) {
  const int64_t rb = row_bytes_of(grid, K);
  const int cmin = cmin_of(grid);
  std::memset(out, 0, rb);
  if (grid == GRID_T) {
    // byte j = sum_{i=0..4} u(tern_input(j, i)) * 3^i, u = c + 1
    for (int64_t j = 0; j < rb; ++j) {
      int v = 0, p = 1;
      for (int i = 0; i < 5; ++i) {
        v += (code_at(codes, K, n, tern_input(j, i)) - cmin) * p;
        p *= 3;
      }
      out[j] = (uint8_t)v;
    }
  } else if (grid == GRID_I2) {
    // little-endian 32-bit word j holds k = 16j+i at bits [2i, 2i+1], u = c + 2
    for (int64_t j = 0; j < rb / 4; ++j) {
      uint32_t w = 0;
      for (int i = 0; i < 16; ++i) w |= (uint32_t)(code_at(codes, K, n, 16 * j + i) - cmin) << (2 * i);
      std::memcpy(out + 4 * j, &w, 4);
    }
  } else {
    // 96-bit triple t: three little-endian words w0,w1,w2 read as the integer
    // w0 | w1<<32 | w2<<64 holds k = 32t+i at bits [3i, 3i+2], u = c + 4.
    for (int64_t t = 0; t < K / 32; ++t) {
      uint32_t w[3] = {0, 0, 0};
      for (int i = 0; i < 32; ++i) {
        const uint32_t u = (uint32_t)(code_at(codes, K, n, 32 * t + i) - cmin);
        for (int b = 0; b < 3; ++b) {
          const int bit = 3 * i + b;
          w[bit / 32] |= ((u >> b) & 1u) << (bit % 32);
        }
      }
      std::memcpy(out + 12 * t, w, 12);
    }
  }
}

// Inverse of pack_row.  Returns false on a ternary byte above 242.
bool unpack_row(int grid, int64_t K, const uint8_t* in, int8_t* row) {
  const int64_t rb = row_bytes_of(grid, K);
  const int cmin = cmin_of(grid);
  if (grid == GRID_T) {
    for (int64_t j = 0; j < rb; ++j) {
      int v = in[j];
      if (v > 242) return false;
      for (int i = 0; i < 5; ++i) {
        const int64_t k = tern_input(j, i);
        if (k < K) row[k] = (int8_t)(v % 3 + cmin);
        v /= 3;
      }
    }
  } else if (grid == GRID_I2) {
    for (int64_t j = 0; j < rb / 4; ++j) {
      uint32_t w;
      std::memcpy(&w, in + 4 * j, 4);
      for (int i = 0; i < 16; ++i) row[16 * j + i] = (int8_t)((int)((w >> (2 * i)) & 3u) + cmin);
    }
  } else {
    for (int64_t t = 0; t < K / 32; ++t) {
      uint32_t w[3];
      std::memcpy(w, in + 12 * t, 12);
      for (int i = 0; i < 32; ++i) {
        uint32_t u = 0;
        for (int b = 0; b < 3; ++b) {
          const int bit = 3 * i + b;
          u |= ((w[bit / 32] >> (bit % 32)) & 1u) << b;
        }
        row[32 * t + i] = (int8_t)((int)u + cmin);
      }
    }
  }
  return true;
}

int64_t nblocks_of(int64_t N) { return (N + kBlock - 1) / kBlock; }
int64_t nslabs_of(int64_t N) { return (N + kSlab - 1) / kSlab; }

// Slabs held by grid block b (the last block may hold one).
int64_t block_slabs(int64_t N, int64_t b) {
  int64_t first = b * (kBlock / kSlab);
  return std::min<int64_t>(kBlock / kSlab, nslabs_of(N) - first);
}

void parallel_rows(int64_t N, int nthreads, const std::function<void(int64_t, int64_t)>& fn) {
  if (nthreads <= 1 || N < 2) {
    fn(0, N);
    return;
  }
  nthreads = (int)std::min<int64_t>(nthreads, N);
  std::vector<std::thread> th;
  for (int t = 0; t < nthreads; ++t) {
    int64_t lo = N * t / nthreads, hi = N * (t + 1) / nthreads;
    th.emplace_back([&fn, lo, hi] { fn(lo, hi); });
  }
  for (auto& x : th) x.join();
}
}  // namespace

extern "C" {

int ora_cmin(int grid) { return grid_ok(grid) ? cmin_of(grid) : 0; }
int ora_cmax(int grid) { return grid_ok(grid) ? cmax_of(grid) : 0; }

void ora_f32_to_bf16(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_rne(in[i]);
}

void ora_bf16_to_f32(const uint16_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_to_f32(in[i]);
}

int64_t ora_row_bytes(int grid, int64_t K) { return row_bytes_of(grid, K); }

// Round-to-nearest quantization (summary page, "How it works"; scale rule of
// the synthetic workload).  row_grid[n] is the grid of row n.  W is fp32
// [N][K]; codes int8 [N][K]; scales bf16 bits [N][K/128].
// Returns 0, or -1 for bad arguments / a non-finite weight.
int ora_quantize(int64_t N, int64_t K, const int8_t* row_grid, const float* W, int8_t* codes,
                 uint16_t* scales) {
  if (N < 0 || K <= 0 || K % kGroup) return -1;
  const int64_t G = K / kGroup;
  for (int64_t n = 0; n < N; ++n) {
    const int grid = row_grid[n];
    if (!grid_ok(grid)) return -1;
    const int cmin = cmin_of(grid), cmax = cmax_of(grid);
    for (int64_t g = 0; g < G; ++g) {
      const float* w = W + n * K + g * kGroup;
      float a = 0.0f;
      for (int i = 0; i < kGroup; ++i) {
        if (!std::isfinite(w[i])) return -1;
        a = std::max(a, std::fabs(w[i]));
      }
      const uint16_t sb = bf16_rne(a / (float)(-cmin));
      scales[n * G + g] = sb;
      const double s = (double)bf16_to_f32(sb);
      for (int i = 0; i < kGroup; ++i) {
        int c = 0;
        if (s != 0.0) {
          double q = std::nearbyint((double)w[i] / s);  // ties to even (default rounding mode)
          c = (int)std::min<double>(std::max<double>(q, cmin), cmax);
        }
        codes[n * K + g * kGroup + i] = (int8_t)c;
      }
    }
  }
  return 0;
}

// Re-round W onto the grid with given scales (no new scale is computed).
int ora_requantize(int64_t N, int64_t K, const int8_t* row_grid, const float* W, const uint16_t* scales,
                   int8_t* codes) {
  if (N < 0 || K <= 0 || K % kGroup) return -1;
  const int64_t G = K / kGroup;
  for (int64_t n = 0; n < N; ++n) {
    const int grid = row_grid[n];
    if (!grid_ok(grid)) return -1;
    for (int64_t k = 0; k < K; ++k) {
      const double s = (double)bf16_to_f32(scales[n * G + k / kGroup]);
      int c = 0;
      if (s != 0.0) {
        double q = std::nearbyint((double)W[n * K + k] / s);
        c = (int)std::min<double>(std::max<double>(q, cmin_of(grid)), cmax_of(grid));
      }
      codes[n * K + k] = (int8_t)c;
    }
  }
  return 0;
}

// Byte offset of every grid block (nblk+1 entries) of a packed matrix.
int ora_block_offsets(int64_t N, int64_t K, const int8_t* blk_grid, int64_t* off) {
  if (N <= 0 || K <= 0 || K % kGroup) return -1;
  const int64_t nb = nblocks_of(N);
  off[0] = 0;
  for (int64_t b = 0; b < nb; ++b) {
    if (!grid_ok(blk_grid[b])) return -1;
    off[b + 1] = off[b] + block_slabs(N, b) * kSlab * row_bytes_of(blk_grid[b], K);
  }
  return 0;
}

// Pack codes [N][K] into the slab-interleaved buffer: within a slab of 64
// rows the bytes run chunk-major, 16 bytes of row r at offset
// chunk*1024 + r*16.  Rows past N are padding (c = 0).
int ora_pack(int64_t N, int64_t K, const int8_t* blk_grid, const int8_t* codes, uint8_t* packed) {
  if (N <= 0 || K <= 0 || K % kGroup) return -1;
  std::vector<int64_t> off(nblocks_of(N) + 1);
  if (ora_block_offsets(N, K, blk_grid, off.data())) return -1;
  std::vector<int8_t> zero(K, 0);
  for (int64_t b = 0; b < nblocks_of(N); ++b) {
    const int grid = blk_grid[b];
    const int64_t rb = row_bytes_of(grid, K);
    std::vector<uint8_t> row(rb);
    for (int64_t sl = 0; sl < block_slabs(N, b); ++sl)
      for (int r = 0; r < kSlab; ++r) {
        const int64_t n = b * kBlock + sl * kSlab + r;
        if (n < N)
          pack_row(grid, K, codes, n, row.data());
        else
          pack_row(grid, K, zero.data(), 0, row.data());
        uint8_t* dst = packed + off[b] + sl * kSlab * rb;
        for (int64_t c = 0; c < rb / kChunk; ++c) std::memcpy(dst + c * kSlab * kChunk + r * kChunk, row.data() + c * kChunk, kChunk);
      }
  }
  return 0;
}

// Inverse of ora_pack for the N real rows.  Returns -2 on an invalid ternary byte.
int ora_unpack(int64_t N, int64_t K, const int8_t* blk_grid, const uint8_t* packed, int8_t* codes) {
  if (N <= 0 || K <= 0 || K % kGroup) return -1;
  std::vector<int64_t> off(nblocks_of(N) + 1);
  if (ora_block_offsets(N, K, blk_grid, off.data())) return -1;
  for (int64_t b = 0; b < nblocks_of(N); ++b) {
    const int grid = blk_grid[b];
    const int64_t rb = row_bytes_of(grid, K);
    std::vector<uint8_t> row(rb);
    for (int64_t sl = 0; sl < block_slabs(N, b); ++sl)
      for (int r = 0; r < kSlab; ++r) {
        const int64_t n = b * kBlock + sl * kSlab + r;
        if (n >= N) continue;
        const uint8_t* src = packed + off[b] + sl * kSlab * rb;
        for (int64_t c = 0; c < rb / kChunk; ++c) std::memcpy(row.data() + c * kChunk, src + c * kSlab * kChunk + r * kChunk, kChunk);
        if (!unpack_row(grid, K, row.data(), codes + n * K)) return -2;
      }
  }
  return 0;
}

// Scales [N][G] -> slab layout: for slab s, group octet q = g/8, row r in the
// slab, element (((s*G8 + q)*64 + r)*8 + g%8), G8 = ceil(G/8); unused
// entries are 0.
int64_t ora_packed_scales_len(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % kGroup) return 0;
  return nslabs_of(N) * ((K / kGroup + 7) / 8) * kSlab * 8;
}

int ora_pack_scales(int64_t N, int64_t K, const uint16_t* scales, uint16_t* ps) {
  const int64_t len = ora_packed_scales_len(N, K);
  if (!len) return -1;
  const int64_t G = K / kGroup, G8 = (G + 7) / 8;
  std::fill(ps, ps + len, (uint16_t)0);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t g = 0; g < G; ++g)
      ps[(((n / kSlab) * G8 + g / 8) * kSlab + n % kSlab) * 8 + g % 8] = scales[n * G + g];
  return 0;
}

int ora_unpack_scales(int64_t N, int64_t K, const uint16_t* ps, uint16_t* scales) {
  if (!ora_packed_scales_len(N, K)) return -1;
  const int64_t G = K / kGroup, G8 = (G + 7) / 8;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t g = 0; g < G; ++g)
      scales[n * G + g] = ps[(((n / kSlab) * G8 + g / 8) * kSlab + n % kSlab) * 8 + g % 8];
  return 0;
}

// Dequantization, one multiply (summary page, "How it works"): w32 = c*s in
// fp32 (exact), w16 = bf16_rne(w32).  Either output may be null.
void ora_dequant(int64_t N, int64_t K, const int8_t* codes, const uint16_t* scales, float* w32, uint16_t* w16) {
  const int64_t G = K / kGroup;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      const float w = (float)codes[n * K + k] * bf16_to_f32(scales[n * G + k / kGroup]);
      if (w32) w32[n * K + k] = w;
      if (w16) w16[n * K + k] = bf16_rne(w);
    }
}

// y[m][n] = sum_k w32[n][k] * x[m][k], fp64 products and an fp64 sum in
// ascending k; x is bf16 bits [M][K].  Rows are split over threads, which
// changes no bit of the result.
void ora_gemv(int64_t M, int64_t N, int64_t K, const int8_t* codes, const uint16_t* scales, const uint16_t* x,
              double* y, int nthreads) {
  const int64_t G = K / kGroup;
  std::vector<double> xd(M * K);
  for (int64_t i = 0; i < M * K; ++i) xd[i] = (double)bf16_to_f32(x[i]);
  parallel_rows(N, nthreads, [&](int64_t lo, int64_t hi) {
    std::vector<double> w(K);
    for (int64_t n = lo; n < hi; ++n) {
      for (int64_t k = 0; k < K; ++k)
        w[k] = (double)((float)codes[n * K + k] * bf16_to_f32(scales[n * G + k / kGroup]));
      for (int64_t m = 0; m < M; ++m) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += w[k] * xd[m * K + k];
        y[m * N + n] = acc;
      }
    }
  });
}

// The product with bf16-rounded weights: y[m][n] = sum_k w16[n][k] * x[m][k]
// with w16 = bf16_rne(c*s), fp64 products and sum in ascending k.  This is
// what a matrix-core path computes when it dequantizes to bf16 before the
// contraction (k-quant calibration page, section "Not just any noise": that
// reproduces the native low-bit result); it differs from ora_gemv only where
// c*s is not a bf16 value (3-bit codes of magnitude 3).
void ora_gemv_w16(int64_t M, int64_t N, int64_t K, const int8_t* codes, const uint16_t* scales, const uint16_t* x,
                  double* y, int nthreads) {
  const int64_t G = K / kGroup;
  std::vector<double> xd(M * K);
  for (int64_t i = 0; i < M * K; ++i) xd[i] = (double)bf16_to_f32(x[i]);
  parallel_rows(N, nthreads, [&](int64_t lo, int64_t hi) {
    std::vector<double> w(K);
    for (int64_t n = lo; n < hi; ++n) {
      for (int64_t k = 0; k < K; ++k)
        w[k] = (double)bf16_to_f32(bf16_rne((float)codes[n * K + k] * bf16_to_f32(scales[n * G + k / kGroup])));
      for (int64_t m = 0; m < M; ++m) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += w[k] * xd[m * K + k];
        y[m * N + n] = acc;
      }
    }
  });
}

// The same product read from packed buffers (decode each row with this
// file's own unpacker, then as ora_gemv).  Returns -2 on a corrupt byte.
int ora_gemv_packed(int64_t M, int64_t N, int64_t K, const int8_t* blk_grid, const uint8_t* packed,
                    const uint16_t* pscales, const uint16_t* x, double* y, int nthreads) {
  if (N <= 0 || K <= 0 || K % kGroup || M <= 0) return -1;
  std::vector<int64_t> off(nblocks_of(N) + 1);
  if (ora_block_offsets(N, K, blk_grid, off.data())) return -1;
  const int64_t G = K / kGroup, G8 = (G + 7) / 8;
  std::vector<double> xd(M * K);
  for (int64_t i = 0; i < M * K; ++i) xd[i] = (double)bf16_to_f32(x[i]);
  int bad = 0;
  parallel_rows(N, nthreads, [&](int64_t lo, int64_t hi) {
    std::vector<int8_t> c(K);
    std::vector<double> w(K);
    for (int64_t n = lo; n < hi; ++n) {
      const int64_t b = n / kBlock, sl = (n % kBlock) / kSlab, r = n % kSlab;
      const int grid = blk_grid[b];
      const int64_t rb = row_bytes_of(grid, K);
      std::vector<uint8_t> row(rb);
      const uint8_t* src = packed + off[b] + sl * kSlab * rb;
      for (int64_t ch = 0; ch < rb / kChunk; ++ch) std::memcpy(row.data() + ch * kChunk, src + ch * kSlab * kChunk + r * kChunk, kChunk);
      if (!unpack_row(grid, K, row.data(), c.data())) {
        bad = 1;
        continue;
      }
      for (int64_t k = 0; k < K; ++k) {
        const uint16_t sb = pscales[(((n / kSlab) * G8 + (k / kGroup) / 8) * kSlab + r) * 8 + (k / kGroup) % 8];
        w[k] = (double)((float)c[k] * bf16_to_f32(sb));
      }
      for (int64_t m = 0; m < M; ++m) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += w[k] * xd[m * K + k];
        y[m * N + n] = acc;
      }
    }
  });
  return bad ? -2 : 0;
}

// ---------------------------------------------------------------- 4-bit containers
// The summary page (section "Premises & limits") says the published
// checkpoints store the 1.6/2/3-bit codewords in 4-bit containers.  The
// container here: the code itself as a 4-bit two's complement nibble (any
// code in -8..7), two per byte, the lower input index in the low nibble; row
// bytes K/2; rows interleaved in 64-row slabs chunk-major exactly as the
// packed layout.  The pages give no nibble order; this one is the project's.
int64_t ora_c4_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || K % kGroup) return 0;
  return nslabs_of(N) * kSlab * (K / 2);
}

// Returns 0, -1 for a bad shape, -3 for a code outside -8..7.
int ora_c4_pack(int64_t N, int64_t K, const int8_t* codes, uint8_t* out) {
  if (!ora_c4_bytes(N, K)) return -1;
  const int64_t rb = K / 2;
  std::vector<uint8_t> row(rb);
  for (int64_t n = 0; n < nslabs_of(N) * kSlab; ++n) {
    for (int64_t i = 0; i < rb; ++i) {
      int lo = 0, hi = 0;
      if (n < N) {
        lo = codes[n * K + 2 * i];
        hi = codes[n * K + 2 * i + 1];
      }
      if (lo < -8 || lo > 7 || hi < -8 || hi > 7) return -3;
      // two's complement nibbles: -1 -> 15, -8 -> 8
      const unsigned nl = (unsigned)(lo < 0 ? lo + 16 : lo), nh = (unsigned)(hi < 0 ? hi + 16 : hi);
      row[i] = (uint8_t)(nl + 16 * nh);
    }
    uint8_t* dst = out + (n / kSlab) * kSlab * rb;
    for (int64_t c = 0; c < rb / kChunk; ++c)
      std::memcpy(dst + c * kSlab * kChunk + (n % kSlab) * kChunk, row.data() + c * kChunk, kChunk);
  }
  return 0;
}

int ora_c4_unpack(int64_t N, int64_t K, const uint8_t* in, int8_t* codes) {
  if (!ora_c4_bytes(N, K)) return -1;
  const int64_t rb = K / 2;
  std::vector<uint8_t> row(rb);
  for (int64_t n = 0; n < N; ++n) {
    const uint8_t* src = in + (n / kSlab) * kSlab * rb;
    for (int64_t c = 0; c < rb / kChunk; ++c)
      std::memcpy(row.data() + c * kChunk, src + c * kSlab * kChunk + (n % kSlab) * kChunk, kChunk);
    for (int64_t i = 0; i < rb; ++i) {
      const int nl = row[i] % 16, nh = row[i] / 16;
      codes[n * K + 2 * i] = (int8_t)(nl >= 8 ? nl - 16 : nl);
      codes[n * K + 2 * i + 1] = (int8_t)(nh >= 8 ? nh - 16 : nh);
    }
  }
  return 0;
}

// ---------------------------------------------------------------- LittleBit
// LittleBit digest page (seosoyoung.eiaserinnys.me/digest/littlebit-ultra-
// low-bit-quantization), sections "LittleBit's structure" and "Rank sets the
// BPW".  A linear W (d_out x d_in) is the sum of two paths (primary and
// residual) of the same form diag(h) U_sign diag(l) V_sign^T diag(g):
// U_sign (d_out x r) and V_sign (d_in x r) hold +-1, h (d_out), g (d_in) and
// l (r) are 16-bit scales (bf16 here).  The forward pass never forms W:
// Z = ((X . g) V_sign) . l, Y = (Z U_sign^T) . h, summed over the paths.
// Storage per path is two r-column binary matrices and three scale vectors,
// so the bits per original weight are
//   b = ((2r + 32)(d_out + d_in) + 32 r) / (d_out d_in)
// and a target b fixes r (the largest r whose b does not exceed it).
double ora_lb_bpw(int64_t d_out, int64_t d_in, int64_t r) {
  return ((2.0 * r + 32.0) * (double)(d_out + d_in) + 32.0 * r) / ((double)d_out * (double)d_in);
}

int64_t ora_lb_rank(int64_t d_out, int64_t d_in, double bpw) {
  int64_t r = 0;
  while (ora_lb_bpw(d_out, d_in, r + 1) <= bpw) ++r;
  return r;
}

// Bit layout (this project's; the page only says the signs are packed into
// 32-bit words): a sign is one bit, 1 for -1.  Each binary matrix is stored
// as rows of bits along the dimension the product sums over: V_sign^T as r
// rows of d_in bits per path (the latent rows, path 0 then path 1, each path
// padded to a multiple of 64 rows), U_sign as d_out rows holding path 0's r
// bits then path 1's, each path's part padded to a multiple of 128 bits.  Bit
// t of byte B of a row is element 8B + t.  Rows are interleaved in 64-row
// slabs exactly as the packed layout (bytes 16c..16c+15 of slab row q at
// c*1024 + q*16); padding bits and rows are 0.
int64_t ora_lb_latent_rows(int64_t r) { return (r + 63) / 64 * 64; }          // rows per path in V^T
int64_t ora_lb_u_row_bytes(int64_t r) { return 2 * ((r + 127) / 128) * 16; }  // both paths

namespace {
void put_bit(uint8_t* buf, int64_t row_bytes, int64_t row, int64_t bit) {
  const int64_t B = bit / 8;
  uint8_t* slab = buf + (row / kSlab) * kSlab * row_bytes;
  slab[(B / kChunk) * kSlab * kChunk + (row % kSlab) * kChunk + B % kChunk] |= (uint8_t)(1u << (bit % 8));
}
int get_bit(const uint8_t* buf, int64_t row_bytes, int64_t row, int64_t bit) {
  const int64_t B = bit / 8;
  const uint8_t* slab = buf + (row / kSlab) * kSlab * row_bytes;
  return slab[(B / kChunk) * kSlab * kChunk + (row % kSlab) * kChunk + B % kChunk] >> (bit % 8) & 1;
}
}  // namespace

int64_t ora_lb_v_bytes(int64_t d_in, int64_t r) { return 2 * ora_lb_latent_rows(r) * (d_in / 8); }
int64_t ora_lb_u_bytes(int64_t d_out, int64_t r) { return nslabs_of(d_out) * kSlab * ora_lb_u_row_bytes(r); }

// u_signs int8 [2][d_out][r], v_signs int8 [2][d_in][r], entries +-1.
// Returns 0, -1 for a bad shape, -3 for an entry other than +-1.
int ora_lb_pack(int64_t d_out, int64_t d_in, int64_t r, const int8_t* u_signs, const int8_t* v_signs,
                uint8_t* u_bits, uint8_t* v_bits) {
  if (d_out <= 0 || d_in <= 0 || d_in % kGroup || r <= 0) return -1;
  std::memset(u_bits, 0, ora_lb_u_bytes(d_out, r));
  std::memset(v_bits, 0, ora_lb_v_bytes(d_in, r));
  const int64_t RP = ora_lb_latent_rows(r), urb = ora_lb_u_row_bytes(r), half = urb / 2;
  for (int p = 0; p < 2; ++p) {
    for (int64_t n = 0; n < d_out; ++n)
      for (int64_t j = 0; j < r; ++j) {
        const int8_t s = u_signs[(p * d_out + n) * r + j];
        if (s != 1 && s != -1) return -3;
        if (s < 0) put_bit(u_bits, urb, n, 8 * half * p + j);
      }
    for (int64_t i = 0; i < d_in; ++i)
      for (int64_t j = 0; j < r; ++j) {
        const int8_t s = v_signs[(p * d_in + i) * r + j];
        if (s != 1 && s != -1) return -3;
        if (s < 0) put_bit(v_bits, d_in / 8, p * RP + j, i);
      }
  }
  return 0;
}

// Inverse of ora_lb_pack (signs +-1).
int ora_lb_unpack(int64_t d_out, int64_t d_in, int64_t r, const uint8_t* u_bits, const uint8_t* v_bits,
                  int8_t* u_signs, int8_t* v_signs) {
  if (d_out <= 0 || d_in <= 0 || d_in % kGroup || r <= 0) return -1;
  const int64_t RP = ora_lb_latent_rows(r), urb = ora_lb_u_row_bytes(r), half = urb / 2;
  for (int p = 0; p < 2; ++p) {
    for (int64_t n = 0; n < d_out; ++n)
      for (int64_t j = 0; j < r; ++j)
        u_signs[(p * d_out + n) * r + j] = get_bit(u_bits, urb, n, 8 * half * p + j) ? -1 : 1;
    for (int64_t i = 0; i < d_in; ++i)
      for (int64_t j = 0; j < r; ++j) v_signs[(p * d_in + i) * r + j] = get_bit(v_bits, d_in / 8, p * RP + j, i) ? -1 : 1;
  }
  return 0;
}

// The forward pass of both paths in fp64, in the page's order: t = x . g,
// z = (V_sign^T t) . l, y = sum over paths of (U_sign z) . h.  Scales and x
// are bf16 bits (g, h [2][d]; l [2][r]); y [d_out].
int ora_lb_gemv(int64_t d_out, int64_t d_in, int64_t r, const int8_t* u_signs, const int8_t* v_signs,
                const uint16_t* g, const uint16_t* l, const uint16_t* h, const uint16_t* x, double* y) {
  if (d_out <= 0 || d_in <= 0 || r <= 0) return -1;
  for (int64_t n = 0; n < d_out; ++n) y[n] = 0.0;
  std::vector<double> t(d_in), z(r);
  for (int p = 0; p < 2; ++p) {
    for (int64_t i = 0; i < d_in; ++i) t[i] = (double)bf16_to_f32(x[i]) * (double)bf16_to_f32(g[p * d_in + i]);
    for (int64_t j = 0; j < r; ++j) {
      double acc = 0.0;
      for (int64_t i = 0; i < d_in; ++i) acc += (double)v_signs[(p * d_in + i) * r + j] * t[i];
      z[j] = acc * (double)bf16_to_f32(l[p * r + j]);
    }
    for (int64_t n = 0; n < d_out; ++n) {
      double acc = 0.0;
      for (int64_t j = 0; j < r; ++j) acc += (double)u_signs[(p * d_out + n) * r + j] * z[j];
      y[n] += acc * (double)bf16_to_f32(h[p * d_out + n]);
    }
  }
  return 0;
}

// ---------------------------------------------------------------- grid allocation
// Summary page, section "How it differs", stage 1 (Allocate): a layer's
// sensitivity S (product of the squared norms of its input activations and
// of its output gradients, a Kronecker-factored curvature estimate) times the
// rounding noise of each grid approximates the loss increase of giving the
// layer that grid; ternary / 2-bit / 3-bit are chosen per layer under a bit
// budget for the whole decoder as a multiple-choice knapsack, solved by
// Lagrangian relaxation.

// Rounding noise of round-to-nearest onto each grid, per 128-row block:
// noise[b*3 + g] = sum over the block's weights of (w - c*s)^2, with c and s
// from the quantizer above, summed in fp64 in ascending (row, input) order.
int ora_rtn_noise(int64_t N, int64_t K, const float* W, double* noise) {
  if (N <= 0 || K <= 0 || K % kGroup) return -1;
  const int64_t G = K / kGroup;
  std::vector<int8_t> codes(K);
  std::vector<uint16_t> scales(G);
  for (int64_t b = 0; b < nblocks_of(N); ++b)
    for (int grid = 0; grid < 3; ++grid) {
      const int8_t rg = (int8_t)grid;
      double sum = 0.0;
      for (int64_t n = b * kBlock; n < std::min<int64_t>(N, (b + 1) * kBlock); ++n) {
        if (ora_quantize(1, K, &rg, W + n * K, codes.data(), scales.data())) return -1;
        for (int64_t k = 0; k < K; ++k) {
          const double e = (double)W[n * K + k] - (double)codes[k] * (double)bf16_to_f32(scales[k / kGroup]);
          sum += e * e;
        }
      }
      noise[b * 3 + grid] = sum;
    }
  return 0;
}

// Sensitivity of every 128-row block of a linear: the squared norm of its
// input activation times the squared norm of the block's output gradient,
// each summed in fp64 in ascending index order.
int ora_block_sensitivity(int64_t K, const uint16_t* x_bf16, int64_t N, const float* grad, double* S) {
  if (K <= 0 || N <= 0) return -1;
  double xs = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    const double v = (double)bf16_to_f32(x_bf16[k]);
    xs += v * v;
  }
  for (int64_t b = 0; b < nblocks_of(N); ++b) {
    double gs = 0.0;
    for (int64_t n = b * kBlock; n < std::min<int64_t>(N, (b + 1) * kBlock); ++n) gs += (double)grad[n] * (double)grad[n];
    S[b] = xs * gs;
  }
  return 0;
}

// Multiple-choice knapsack by Lagrangian relaxation (summary page, section
// "How it differs", stage 1), written as the greedy walk along each unit's
// lower convex hull -- the textbook equivalent of sweeping the multiplier,
// and a different computation from a sweep over multiplier values.
//
// Unit i has n[i] weights, sensitivity S[i], noise E[i*3 + g] and a mask of
// allowed grids.  Its options are points (bits b_g = n*bits[g], cost
// f_g = S*E[g]).  For a multiplier lam every unit takes the option minimising
// f + lam*b (ties to fewer bits); as lam falls from +inf to 0 that choice
// walks the lower convex hull of the points from the fewest-bits option,
// one hull edge at a time, taking an edge when lam drops below its slope
// (cost saved per extra bit).  So:
//   1. start every unit at its fewest-bits option (lowest cost among equal
//      bits); if that already exceeds budget * sum(n), the budget is infeasible;
//   2. list every unit's hull edges with positive slope (points on one line
//      collapse into the edge to the farthest point, which is what a
//      multiplier strictly inside an interval picks);
//   3. take the edges in decreasing slope, all edges of one slope together
//      (no multiplier separates them), and stop at the first group that would
//      exceed the budget: a smaller multiplier would take that group too.
// The result is the Lagrangian assignment at the smallest multiplier whose
// bits fit.  lam_out receives the slope of the first group left out (0 when
// every edge fits): the assignment is the minimiser for every multiplier
// strictly between that slope and the slope of the last group taken.
// Returns 0, -1 for bad input, -2 if even the cheapest allowed options exceed
// the budget.
int ora_allocate(int64_t count, const int64_t* n, const double* S, const double* E, const uint32_t* allowed,
                 const double* bits, double budget, int8_t* out, double* lam_out) {
  if (count <= 0) return -1;
  double total_n = 0.0;
  for (int64_t i = 0; i < count; ++i) {
    if (n[i] <= 0 || !(S[i] >= 0.0) || !(allowed[i] & 7u)) return -1;
    for (int g = 0; g < 3; ++g)
      if (!(E[i * 3 + g] >= 0.0)) return -1;
    total_n += (double)n[i];
  }
  const double cap = budget * total_n;
  struct Edge {
    double slope;
    int64_t unit;
    int to;  // grid at the edge's far end
  };
  std::vector<Edge> edges;
  for (int64_t i = 0; i < count; ++i) {
    // the unit's options, by bits, then cost, then grid index; equal bits keep the first
    std::vector<int> opt;
    for (int g = 0; g < 3; ++g)
      if (allowed[i] >> g & 1u) opt.push_back(g);
    std::sort(opt.begin(), opt.end(), [&](int a, int b) {
      if (bits[a] != bits[b]) return bits[a] < bits[b];
      const double fa = S[i] * E[i * 3 + a], fb = S[i] * E[i * 3 + b];
      if (fa != fb) return fa < fb;
      return a < b;
    });
    std::vector<int> pts;
    for (int g : opt)
      if (pts.empty() || bits[g] != bits[pts.back()]) pts.push_back(g);
    out[i] = (int8_t)pts[0];
    int v = pts[0];
    for (;;) {
      int best = -1;
      double bs = 0.0;
      for (int w : pts) {
        if (!(bits[w] > bits[v])) continue;
        const double s = (S[i] * E[i * 3 + v] - S[i] * E[i * 3 + w]) / ((double)n[i] * bits[w] - (double)n[i] * bits[v]);
        if (best < 0 || s > bs || (s == bs && bits[w] > bits[best])) {
          best = w;
          bs = s;
        }
      }
      if (best < 0 || !(bs > 0.0)) break;
      edges.push_back({bs, i, best});
      v = best;
    }
  }
  auto used_bits = [&]() {
    double u = 0.0;
    for (int64_t i = 0; i < count; ++i) u += (double)n[i] * bits[out[i]];
    return u;
  };
  if (used_bits() > cap) return -2;
  // decreasing slope; within a unit the hull's slopes already decrease, and the
  // stable order keeps a unit's edges in walk order when slopes tie
  std::stable_sort(edges.begin(), edges.end(), [](const Edge& a, const Edge& b) { return a.slope > b.slope; });
  double lam = 0.0;
  for (size_t j = 0; j < edges.size();) {
    size_t e = j;
    while (e < edges.size() && edges[e].slope == edges[j].slope) ++e;
    std::vector<int8_t> keep(out, out + count);
    for (size_t q = j; q < e; ++q) out[edges[q].unit] = (int8_t)edges[q].to;
    if (used_bits() > cap) {
      std::copy(keep.begin(), keep.end(), out);
      lam = edges[j].slope;
      break;
    }
    j = e;
  }
  if (lam_out) *lam_out = lam;
  return 0;
}

}  // extern "C"
