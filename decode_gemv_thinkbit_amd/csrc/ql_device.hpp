// Device-side helpers shared by the qlinear kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlinear.h"

namespace ql {

constexpr int kGroup = QL_GROUP;  // 128 weights per scale
constexpr int kSlab = QL_SLAB;    // 64 rows per slab
constexpr int kBlock = QL_BLOCK;  // 128 rows per grid block
constexpr int kChunkBytes = 16;   // bytes per row per slab step
constexpr int kSlabChunkBytes = kChunkBytes * kSlab;  // 1024
constexpr int kTritsPerChunk = 80;  // 16 bytes x 5 trits
constexpr int kPeriodK = 640;       // lcm(80, 128): 8 ternary chunks = 5 groups
constexpr int kCounterWords = 32;   // split-K state: words per slab counter (one 128-byte line)
constexpr int kPartWords = 1024;    // split-K state: partial sums per (slab, part), 16 per lane

// Ternary digit order, layout version 2.  A stored byte j holds inputs
// 5j..5j+4 as base-3 digits.  Even bytes keep input order (digit i = input
// 5j+i).  Odd bytes rotate it: digits 0..3 are inputs 5j+1..5j+4 and digit 4
// is input 5j, so that within a byte pair every even-aligned input pair but
// one is a digit pair.  These two maps convert between the stored byte and
// the input-order value (digit i = input 5j+i).
__host__ __device__ inline uint32_t tern_to_input_order(uint32_t b, int64_t j) {
  return (j & 1) ? (b % 81u) * 3u + b / 81u : b;
}
__host__ __device__ inline uint32_t tern_from_input_order(uint32_t v, int64_t j) {
  return (j & 1) ? (v % 3u) * 81u + v / 3u : v;
}

__host__ __device__ inline int grid_cmin(int g) { return g == QL_GRID_T ? -1 : (g == QL_GRID_I2 ? -2 : -4); }
__host__ __device__ inline int grid_cmax(int g) { return g == QL_GRID_I3 ? 3 : 1; }

__host__ __device__ inline int64_t row_bytes(int grid, int64_t K) {
  if (grid == QL_GRID_T) return 16 * ((K + 79) / 80);
  if (grid == QL_GRID_I2) return K / 4;
  return 3 * K / 8;
}

// 4-bit container baseline: code c (-8..7) of row n, input k as a two's
// complement nibble.  Row bytes K/2; byte i of a row holds inputs 2i (low
// nibble) and 2i+1 (high nibble); rows are interleaved in 64-row slabs exactly
// like the packed layout (bytes 16c..16c+15 of slab row r at c*1024 + r*16).
__host__ __device__ inline int64_t c4_byte_offset(int64_t K, int64_t n, int64_t k) {
  const int64_t i = k >> 1;
  return (n / kSlab) * (int64_t)kSlab * (K / 2) + (i >> 4) * kSlabChunkBytes + (n % kSlab) * kChunkBytes + (i & 15);
}
__host__ __device__ inline int c4_code_at(const uint8_t* c4, int64_t K, int64_t n, int64_t k) {
  const uint32_t nib = (c4[c4_byte_offset(K, n, k)] >> (4 * (k & 1))) & 0xFu;
  return (int)nib - (int)((nib & 8u) << 1);
}

// Byte offset of slab `s` in a packed matrix (uniform grid, or per-block tables).
__device__ inline int64_t slab_offset(int64_t s, int64_t K, int grid, const int8_t* blk_grid,
                                      const int64_t* blk_off, int* grid_out) {
  if (grid == QL_GRID_MIXED) {
    // global-address-space reads: flat ones would also count against lgkmcnt, which the
    // decode loops wait on for their LDS reads
    const int g = ((const __attribute__((address_space(1))) int8_t*)blk_grid)[s >> 1];
    *grid_out = g;
    return ((const __attribute__((address_space(1))) int64_t*)blk_off)[s >> 1] +
           (s & 1) * (int64_t)kSlab * row_bytes(g, K);
  }
  *grid_out = grid;
  return s * (int64_t)kSlab * row_bytes(grid, K);
}

// Element index of scale (n, g) in the packed scale array.
__host__ __device__ inline int64_t pscale_index(int64_t n, int64_t g, int64_t G8) {
  return (((n / kSlab) * G8 + (g >> 3)) * kSlab + (n % kSlab)) * 8 + (g & 7);
}

__device__ inline float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ inline uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// bf16 bits of a small integer code (-4..3), exact.
__device__ inline uint32_t code_bf16(int c) { return (uint32_t)f32_to_bf16_bits((float)c); }

}  // namespace ql
