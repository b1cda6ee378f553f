// LDS decode tables of the batch-decode kernels (GEMV and its batched MFMA
// variant): each entry holds codes as bf16 in input order, so a table read
// turns packed bytes straight into bf16 operands.
#pragma once

#include "ql_device.hpp"

namespace ql {

// ---------------------------------------------------------------- LDS tables
// The 3-bit table sits at offset 0, so its addresses need no base; the other
// two bases fit the 16-bit immediate offset of the LDS read instructions.
constexpr int kI3Lut = 0;                   // 64 entries x 4 B
constexpr int kTLut = 64 * 4;               // 243 rows x 256 B (16 replicas x 16 B)
constexpr int kI2Lut = kTLut + 243 * 256;   // 256 rows x 32 B (4 replicas x 8 B)
constexpr int kLutBytes = kI2Lut + 256 * 32;  // 70656

__device__ inline void build_luts(uint8_t* smem) {
  for (int e = threadIdx.x; e < 243 * 16; e += blockDim.x) {
    const int b = e >> 4, r = e & 15;
    int c[5], v = b;
    for (int i = 0; i < 5; ++i) {
      c[i] = v % 3 - 1;
      v /= 3;
    }
    uint4 q;
    q.x = code_bf16(c[0]) | (code_bf16(c[1]) << 16);
    q.y = code_bf16(c[2]) | (code_bf16(c[3]) << 16);
    q.z = code_bf16(c[4]);
    q.w = code_bf16(c[4]) << 16;
    *reinterpret_cast<uint4*>(smem + kTLut + b * 256 + r * 16) = q;
  }
  for (int e = threadIdx.x; e < 256 * 4; e += blockDim.x) {
    const int b = e >> 2, r = e & 3;
    uint2 q;
    q.x = code_bf16((b & 3) - 2) | (code_bf16(((b >> 2) & 3) - 2) << 16);
    q.y = code_bf16(((b >> 4) & 3) - 2) | (code_bf16(((b >> 6) & 3) - 2) << 16);
    *reinterpret_cast<uint2*>(smem + kI2Lut + b * 32 + r * 8) = q;
  }
  for (int e = threadIdx.x; e < 64; e += blockDim.x)
    *reinterpret_cast<uint32_t*>(smem + kI3Lut + e * 4) = code_bf16((e & 7) - 4) | (code_bf16((e >> 3) - 4) << 16);
}

// 3-bit table address of field P of a 96-bit triple
// 4 * (6-bit field P of the 96-bit triple w0|w1<<32|w2<<64)
template <int P>
__device__ __forceinline__ uint32_t i3_field_x4(uint32_t w0, uint32_t w1, uint32_t w2) {
  constexpr int bit = 6 * P;
  if constexpr (bit == 0) {
    return (w0 << 2) & 0xFCu;
  } else if constexpr (bit + 6 <= 32) {
    return (w0 >> (bit - 2)) & 0xFCu;
  } else if constexpr (bit < 32) {
    return __builtin_amdgcn_alignbit(w1, w0, bit - 2) & 0xFCu;
  } else if constexpr (bit + 6 <= 64) {
    return (w1 >> (bit - 34)) & 0xFCu;
  } else if constexpr (bit < 64) {
    return __builtin_amdgcn_alignbit(w2, w1, bit - 34) & 0xFCu;
  } else {
    return (w2 >> (bit - 66)) & 0xFCu;
  }
}

}  // namespace ql
