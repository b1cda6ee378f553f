// LDS decode tables of the batch-decode kernels (GEMV and its batched MFMA
// variant): each entry holds codes as bf16 in input order, so a table read
// turns packed bytes straight into bf16 operands.
#pragma once

#include <utility>

#include "ql_device.hpp"

namespace ql {

// ---------------------------------------------------------------- LDS tables
// The 3-bit table sits at offset 0, so its addresses need no base; the other
// two bases fit the 16-bit immediate offset of the LDS read instructions.
constexpr int kI3Lut = 0;                   // 64 entries x 4 B
constexpr int kTLut = 64 * 4;               // 243 rows x 256 B (16 replicas x 16 B)
constexpr int kI2Lut = kTLut + 243 * 256;   // 256 rows x 32 B (4 replicas x 8 B)
constexpr int kLutBytes = kI2Lut + 256 * 32;  // 70656

typedef uint32_t lut_v4 __attribute__((ext_vector_type(4)));
typedef uint32_t lut_v2 __attribute__((ext_vector_type(2)));

// Replicas of one table: slot e (row e / REP, replica e % REP, SZ bytes each)
// takes replica 0 of its row.  Thread t copies slots t, t + NT, ...: all their
// reads are issued before the first write.
template <class V, int REP, int SZ, int SLOTS, int NT, int... I>
__device__ __forceinline__ void lut_copies(uint8_t* tab, int t, std::integer_sequence<int, I...>) {
  // (past the table: a row is read, never written)
  const V v[] = {*reinterpret_cast<const V*>(tab + ((t + I * NT < SLOTS ? t + I * NT : SLOTS - 1) / REP) * REP * SZ)...};
  ((t + I * NT < SLOTS && ((t + I * NT) % REP) != 0 ? (void)(*reinterpret_cast<V*>(tab + (t + I * NT) * SZ) = v[I])
                                                     : (void)0),
   ...);
}

// Every table row is computed once (replica 0), the rows of all three tables
// spread over all NT threads of the workgroup; after a barrier the other
// replicas are copied from them, consecutive threads writing consecutive
// slots, with each thread's copies unrolled so their LDS reads are in flight
// together.  Computing every slot separately cost about 2 us per launch, which
// is much of a short launch.
template <int NT>
__device__ inline void build_luts(uint8_t* smem) {
  const int t = threadIdx.x;
  for (int r = t; r < 243 + 256 + 64; r += NT) {
    if (r < 243) {
      int c[5], v = r;
      for (int i = 0; i < 5; ++i) {
        c[i] = v % 3 - 1;
        v /= 3;
      }
      uint4 q;
      q.x = code_bf16(c[0]) | (code_bf16(c[1]) << 16);
      q.y = code_bf16(c[2]) | (code_bf16(c[3]) << 16);
      q.z = code_bf16(c[4]);
      q.w = code_bf16(c[4]) << 16;
      *reinterpret_cast<uint4*>(smem + kTLut + r * 256) = q;
    } else if (r < 243 + 256) {
      const int b = r - 243;
      uint2 q;
      q.x = code_bf16((b & 3) - 2) | (code_bf16(((b >> 2) & 3) - 2) << 16);
      q.y = code_bf16(((b >> 4) & 3) - 2) | (code_bf16(((b >> 6) & 3) - 2) << 16);
      *reinterpret_cast<uint2*>(smem + kI2Lut + b * 32) = q;
    } else {
      const int e = r - 243 - 256;
      *reinterpret_cast<uint32_t*>(smem + kI3Lut + e * 4) = code_bf16((e & 7) - 4) | (code_bf16((e >> 3) - 4) << 16);
    }
  }
  __syncthreads();
  // ternary: 243 rows x 16 replicas x 16 B; 2-bit: 256 rows x 4 replicas x 8 B
  constexpr int kT = (243 * 16 + NT - 1) / NT, kI2 = (256 * 4 + NT - 1) / NT;
  lut_copies<lut_v4, 16, 16, 243 * 16, NT>(smem + kTLut, t, std::make_integer_sequence<int, kT>{});
  lut_copies<lut_v2, 4, 8, 256 * 4, NT>(smem + kI2Lut, t, std::make_integer_sequence<int, kI2>{});
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
