// Quantize, pack, unpack, scale re-layout and dequantize kernels.
//
// Weight format: ThinkBit summary page (onedev.kr/papers/1416), section "How it
// works" -- w = c * s, one bf16 scale per 128 input weights, grid ternary /
// 2-bit / 3-bit.  The packed layout is the library's own, documented in
// include/qlinear.h; this file writes it from codes and reads it back.
#include "ql_internal.hpp"

namespace ql {

// ---------------------------------------------------------------- quantize
// One wave per (row, group): 64 lanes x 2 weights, wave max, then per-weight
// rounding.  The quotient w/s is formed in fp64 (correctly rounded division),
// rounded half-to-even and clamped onto the grid.
__global__ void __launch_bounds__(256) quantize_kernel(int64_t N, int64_t K, int grid,
                                                       const int8_t* __restrict__ blk_grid,
                                                       const float* __restrict__ W, int8_t* __restrict__ codes,
                                                       uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t G = K / kGroup;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= N * G) return;
  const int64_t n = item / G, g = item % G;
  const int gr = grid == QL_GRID_MIXED ? blk_grid[n / kBlock] : grid;
  const int cmin = grid_cmin(gr), cmax = grid_cmax(gr);
  const float2 v = reinterpret_cast<const float2*>(W + n * K + g * kGroup)[lane];
  float a = fmaxf(fabsf(v.x), fabsf(v.y));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
  const uint16_t sb = f32_to_bf16_bits(a / (float)(-cmin));
  if (lane == 0) scales[n * G + g] = sb;
  const double s = (double)bf16_bits_to_f32(sb);
  int c0 = 0, c1 = 0;
  if (s != 0.0) {
    c0 = (int)fmin(fmax(rint((double)v.x / s), (double)cmin), (double)cmax);
    c1 = (int)fmin(fmax(rint((double)v.y / s), (double)cmin), (double)cmax);
  }
  char2 out;
  out.x = (signed char)c0;
  out.y = (signed char)c1;
  reinterpret_cast<char2*>(codes + n * K + g * kGroup)[lane] = out;
}

hipError_t launch_quantize(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const float* W, int8_t* codes,
                           uint16_t* scales, hipStream_t stream) {
  const int64_t items = N * (K / kGroup);
  const int64_t blocks = (items + 3) / 4;
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, N, K, grid, blk_grid, W, codes,
                     scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------- pack
// Where the packer reads codes: an int8 array [N][K], or a 4-bit container
// (the converter from container checkpoints).
struct I8Codes {
  const int8_t* __restrict__ p;
  __device__ int at(int64_t K, int64_t n, int64_t k) const { return p[n * K + k]; }
};
struct C4Codes {
  const uint8_t* __restrict__ p;
  __device__ int at(int64_t K, int64_t n, int64_t k) const { return c4_code_at(p, K, n, k); }
};

// Digit u = c - c_min of row n at input k; rows past N and trits past K are
// padding with c = 0.
template <class Src>
__device__ inline uint32_t digit(const Src& codes, int64_t N, int64_t K, int64_t n, int64_t k, int cmin) {
  const int c = (n < N && k < K) ? codes.at(K, n, k) : 0;
  return (uint32_t)(c - cmin);
}

// Byte jj of row n in its grid's row order.
template <class Src>
__device__ inline uint32_t row_byte_value(const Src& codes, int64_t N, int64_t K, int64_t n, int64_t jj, int gr) {
  const int cmin = grid_cmin(gr);
  if (gr == QL_GRID_T) {
    // five trits in input order (least significant = lowest k), then the
    // byte's stored digit order
    uint32_t v = 0;
#pragma unroll
    for (int i = 4; i >= 0; --i) v = v * 3 + digit(codes, N, K, n, 5 * jj + i, cmin);
    return tern_from_input_order(v, jj);
  }
  if (gr == QL_GRID_I2) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) v |= digit(codes, N, K, n, 4 * jj + i, cmin) << (2 * i);
    return v;
  }
  // 3-bit codes form one little-endian bit stream: code k at bits [3k, 3k+2].
  uint32_t v = 0;
  const int64_t bit0 = 8 * jj;
  const int64_t k_first = bit0 / 3, k_last = (bit0 + 7) / 3;
  for (int64_t k = k_first; k <= k_last; ++k) {
    const int64_t sh = 3 * k - bit0;  // may be negative for the first code
    const uint32_t u = digit(codes, N, K, n, k, cmin);
    v |= sh >= 0 ? (u << sh) : (u >> -sh);
  }
  return v & 0xFFu;
}

// One thread per (padded row, 16-byte chunk).
template <class Src>
__global__ void __launch_bounds__(256) pack_kernel(int64_t N, int64_t K, int grid, const int8_t* __restrict__ blk_grid,
                                                   const int64_t* __restrict__ blk_off, Src codes,
                                                   uint8_t* __restrict__ packed, int64_t max_chunks) {
  const int64_t S = (N + kSlab - 1) / kSlab;
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= S * kSlab * max_chunks) return;
  const int64_t np = item / max_chunks, c = item % max_chunks;
  const int64_t s = np / kSlab, r = np % kSlab;
  int gr;
  const int64_t off = slab_offset(s, K, grid, blk_grid, blk_off, &gr);
  if (c >= row_bytes(gr, K) / kChunkBytes) return;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) v |= row_byte_value(codes, N, K, np, 16 * c + 4 * q + b, gr) << (8 * b);
    w[q] = v;
  }
  *reinterpret_cast<uint4*>(packed + off + c * kSlabChunkBytes + r * kChunkBytes) = make_uint4(w[0], w[1], w[2], w[3]);
}

template <class Src>
static hipError_t launch_pack_from(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                                   Src codes, uint8_t* packed, hipStream_t stream) {
  const int64_t S = (N + kSlab - 1) / kSlab;
  const int64_t max_chunks = row_bytes(QL_GRID_I3, K) / kChunkBytes;  // the widest grid
  const int64_t items = S * kSlab * max_chunks;
  hipLaunchKernelGGL(pack_kernel<Src>, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, N, K, grid,
                     blk_grid, blk_off, codes, packed, max_chunks);
  return hipGetLastError();
}

hipError_t launch_pack(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                       const int8_t* codes, uint8_t* packed, hipStream_t stream) {
  return launch_pack_from(N, K, grid, blk_grid, blk_off, I8Codes{codes}, packed, stream);
}

hipError_t launch_c4_to_packed(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                               const uint8_t* c4, uint8_t* packed, hipStream_t stream) {
  return launch_pack_from(N, K, grid, blk_grid, blk_off, C4Codes{c4}, packed, stream);
}

// ---------------------------------------------------------------- 4-bit containers
// One thread per (padded row, 16-byte chunk = 32 codes): nibble i of word q
// holds input 32c + 8q + i.
__global__ void __launch_bounds__(256) c4_pack_kernel(int64_t N, int64_t K, const int8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ c4) {
  const int64_t nch = K / 32;
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= ((N + kSlab - 1) / kSlab) * kSlab * nch) return;
  const int64_t np = item / nch, c = item % nch;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int code = np < N ? codes[np * K + 32 * c + 8 * q + i] : 0;
      v |= ((uint32_t)code & 0xFu) << (4 * i);
    }
    w[q] = v;
  }
  *reinterpret_cast<uint4*>(c4 + c4_byte_offset(K, np, 32 * c)) = make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ void __launch_bounds__(256) c4_unpack_kernel(int64_t N, int64_t K, const uint8_t* __restrict__ c4,
                                                        int8_t* __restrict__ codes) {
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= N * K) return;
  codes[item] = (int8_t)c4_code_at(c4, K, item / K, item % K);
}

hipError_t launch_c4_pack(int64_t N, int64_t K, const int8_t* codes, uint8_t* c4, hipStream_t stream) {
  const int64_t items = ((N + kSlab - 1) / kSlab) * kSlab * (K / 32);
  hipLaunchKernelGGL(c4_pack_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, N, K, codes, c4);
  return hipGetLastError();
}

hipError_t launch_c4_unpack(int64_t N, int64_t K, const uint8_t* c4, int8_t* codes, hipStream_t stream) {
  const int64_t items = N * K;
  hipLaunchKernelGGL(c4_unpack_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, N, K, c4, codes);
  return hipGetLastError();
}

// ---------------------------------------------------------------- unpack / dequant
__device__ inline uint32_t packed_row_byte(const uint8_t* __restrict__ slab, int64_t r, int64_t jj) {
  return slab[(jj >> 4) * kSlabChunkBytes + r * kChunkBytes + (jj & 15)];
}

__device__ inline int decode_code(const uint8_t* __restrict__ slab, int64_t r, int64_t k, int64_t K, int gr) {
  uint32_t u;
  if (gr == QL_GRID_T) {
    uint32_t b = tern_to_input_order(packed_row_byte(slab, r, k / 5), k / 5);
    const int i = (int)(k % 5);
    for (int t = 0; t < i; ++t) b /= 3;
    u = b % 3;
  } else if (gr == QL_GRID_I2) {
    u = (packed_row_byte(slab, r, k >> 2) >> (2 * (k & 3))) & 3u;
  } else {
    const int64_t bit = 3 * k;
    uint32_t v = packed_row_byte(slab, r, bit >> 3);
    if ((bit & 7) > 5) v |= packed_row_byte(slab, r, (bit >> 3) + 1) << 8;
    u = (v >> (bit & 7)) & 7u;
  }
  return (int)u + grid_cmin(gr);
}

// mode 0: int8 codes; 1: fp32 c*s; 2: bf16 bits of c*s.  One thread per (row, k).
__global__ void __launch_bounds__(256) unpack_kernel(int64_t N, int64_t K, int grid, const int8_t* __restrict__ blk_grid,
                                                     const int64_t* __restrict__ blk_off,
                                                     const uint8_t* __restrict__ packed,
                                                     const uint16_t* __restrict__ pscales, int mode, void* out) {
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= N * K) return;
  const int64_t n = item / K, k = item % K;
  int gr;
  const int64_t off = slab_offset(n / kSlab, K, grid, blk_grid, blk_off, &gr);
  const int c = decode_code(packed + off, n % kSlab, k, K, gr);
  if (mode == 0) {
    static_cast<int8_t*>(out)[item] = (int8_t)c;
    return;
  }
  const int64_t G8 = (K / kGroup + 7) / 8;
  const float w = (float)c * bf16_bits_to_f32(pscales[pscale_index(n, k / kGroup, G8)]);
  if (mode == 1)
    static_cast<float*>(out)[item] = w;
  else
    static_cast<uint16_t*>(out)[item] = f32_to_bf16_bits(w);
}

hipError_t launch_unpack(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                         const uint8_t* packed, const uint16_t* pscales, int mode, void* out, hipStream_t stream) {
  const int64_t items = N * K;
  hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, N, K, grid, blk_grid,
                     blk_off, packed, pscales, mode, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- scales
// dir 0: scales [N][G] -> packed array; dir 1: packed array -> scales.
__global__ void __launch_bounds__(256) pack_scales_kernel(int64_t N, int64_t K, uint16_t* __restrict__ scales,
                                                          uint16_t* __restrict__ ps, int dir) {
  const int64_t G = K / kGroup, G8 = (G + 7) / 8;
  const int64_t S = (N + kSlab - 1) / kSlab;
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= S * kSlab * G8 * 8) return;
  const int64_t n = item / (G8 * 8), g = item % (G8 * 8);
  const int64_t idx = pscale_index(n, g, G8);
  if (dir == 0) {
    ps[idx] = (n < N && g < G) ? scales[n * G + g] : (uint16_t)0;
  } else if (n < N && g < G) {
    scales[n * G + g] = ps[idx];
  }
}

hipError_t launch_scales(int64_t N, int64_t K, uint16_t* scales, uint16_t* ps, int dir, hipStream_t stream) {
  const int64_t G8 = (K / kGroup + 7) / 8;
  const int64_t items = ((N + kSlab - 1) / kSlab) * kSlab * G8 * 8;
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, N, K, scales, ps,
                     dir);
  return hipGetLastError();
}

}  // namespace ql
