// Data validation: the products treat codes outside the grid and corrupt
// packed bytes as outside their contract (undefined results, never an
// out-of-bounds access).  These kernels find such data and count it in a
// device array the caller reads back.
//
// ThinkBit summary page (onedev.kr/papers/1416), section "How it works": the
// grids are ternary {-1,0,1}, 2-bit {-2..1} and 3-bit {-4..3}.  In the packed
// layout only ternary bytes can hold a value outside the grid (a base-3 byte
// of five trits is at most 242); every 2- and 3-bit field is a grid point.
// Padding (rows past N in the last slab, trits past K) must code c = 0.
#include "ql_internal.hpp"

namespace ql {
namespace {

enum { kBadCode = 0, kBadPadding = 1, kBadGrid = 2 };

__device__ __forceinline__ void count(uint32_t* counts, int what) { atomicAdd(counts + what, 1u); }

__device__ __forceinline__ bool grid_ok(int g) { return g == QL_GRID_T || g == QL_GRID_I2 || g == QL_GRID_I3; }

// One thread per (row, 128-input group) of the codes.
__global__ void __launch_bounds__(256) validate_codes_kernel(int64_t N, int64_t K, int grid,
                                                             const int8_t* __restrict__ blk_grid,
                                                             const int8_t* __restrict__ codes,
                                                             uint32_t* __restrict__ counts) {
  const int64_t G = K / kGroup;
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= N * G) return;
  const int64_t n = item / G, g = item % G;
  const int gr = grid == QL_GRID_MIXED ? blk_grid[n / kBlock] : grid;
  if (!grid_ok(gr)) {
    if (g == 0 && n % kBlock == 0) count(counts, kBadGrid);
    return;
  }
  const int cmin = grid_cmin(gr), cmax = grid_cmax(gr);
  uint32_t bad = 0;
  for (int k = 0; k < kGroup; ++k) {
    const int c = codes[n * K + g * kGroup + k];
    bad += (c < cmin || c > cmax) ? 1u : 0u;
  }
  if (bad) atomicAdd(counts + kBadCode, bad);
}

// Code u of input k of a 3-bit row (a little-endian bit stream, k at bits 3k..3k+2).
__device__ __forceinline__ uint32_t i3_digit(const uint8_t* __restrict__ slab, int64_t r, int64_t k) {
  const int64_t bit = 3 * k;
  auto byte = [&](int64_t jj) -> uint32_t {
    return slab[(jj >> 4) * kSlabChunkBytes + r * kChunkBytes + (jj & 15)];
  };
  uint32_t v = byte(bit >> 3);
  if ((bit & 7) > 5) v |= byte((bit >> 3) + 1) << 8;
  return (v >> (bit & 7)) & 7u;
}

// One thread per (padded row, 16-byte chunk) of the packed matrix.
__global__ void __launch_bounds__(256) validate_packed_kernel(int64_t N, int64_t K, int grid,
                                                              const int8_t* __restrict__ blk_grid,
                                                              const int64_t* __restrict__ blk_off,
                                                              const uint8_t* __restrict__ packed, int64_t max_chunks,
                                                              uint32_t* __restrict__ counts) {
  const int64_t S = (N + kSlab - 1) / kSlab;
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= S * kSlab * max_chunks) return;
  const int64_t np = item / max_chunks, c = item % max_chunks;
  const int64_t s = np / kSlab, r = np % kSlab;
  if (grid == QL_GRID_MIXED && !grid_ok(blk_grid[s >> 1])) {
    if (c == 0 && r == 0 && (s & 1) == 0) count(counts, kBadGrid);
    return;  // the block's offset and layout are unknown: nothing of it is read
  }
  int gr;
  const int64_t off = slab_offset(s, K, grid, blk_grid, blk_off, &gr);
  if (c >= row_bytes(gr, K) / kChunkBytes) return;
  const uint8_t* slab = packed + off;
  const bool pad_row = np >= N;
  if (gr == QL_GRID_T) {
    for (int b = 0; b < kChunkBytes; ++b) {
      const int64_t jj = 16 * c + b;
      const uint32_t v = slab[c * kSlabChunkBytes + r * kChunkBytes + b];
      if (v > 242u) {
        count(counts, kBadCode);
        continue;
      }
      uint32_t d = tern_to_input_order(v, jj);  // digit i = input 5 jj + i
      for (int i = 0; i < 5; ++i, d /= 3)
        if ((pad_row || 5 * jj + i >= K) && d % 3 != 1u) count(counts, kBadPadding);
    }
  } else if (pad_row) {
    const uint32_t want = (uint32_t)(-grid_cmin(gr));  // u of c = 0
    if (gr == QL_GRID_I2) {
      for (int b = 0; b < kChunkBytes; ++b)
        if (slab[c * kSlabChunkBytes + r * kChunkBytes + b] != 0xAAu) count(counts, kBadPadding);
    } else {
      // the chunk's 128 bits hold codes of inputs whose first bit falls in it
      const int64_t k0 = (128 * c + 2) / 3, k1 = (128 * (c + 1) + 2) / 3;
      for (int64_t k = k0; k < k1 && k < K; ++k)
        if (i3_digit(slab, r, k) != want) count(counts, kBadPadding);
    }
  }
}

}  // namespace

hipError_t launch_validate_codes(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int8_t* codes,
                                 uint32_t* counts, hipStream_t stream) {
  const int64_t items = N * (K / kGroup);
  hipLaunchKernelGGL(validate_codes_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, N, K, grid,
                     blk_grid, codes, counts);
  return hipGetLastError();
}

hipError_t launch_validate_packed(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                                  const uint8_t* packed, uint32_t* counts, hipStream_t stream) {
  const int64_t S = (N + kSlab - 1) / kSlab;
  const int64_t max_chunks = row_bytes(QL_GRID_I3, K) / kChunkBytes;  // the widest grid
  const int64_t items = S * kSlab * max_chunks;
  hipLaunchKernelGGL(validate_packed_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, N, K, grid,
                     blk_grid, blk_off, packed, max_chunks, counts);
  return hipGetLastError();
}

}  // namespace ql
