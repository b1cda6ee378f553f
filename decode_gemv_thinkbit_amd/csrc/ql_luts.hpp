// LDS decode tables of the batch-decode kernels (GEMV and its batched MFMA
// variant): each entry holds codes as bf16 in input order, so a table read
// turns packed bytes straight into bf16 operands.
#pragma once

#include "ql_device.hpp"

namespace ql {

// ---------------------------------------------------------------- LDS tables
// Each lane reads its own replica of a table row, so a wave's 64 data-dependent
// reads spread over the banks instead of piling onto the few that hold one
// copy.  The 3-bit table sits at offset 0, so its addresses need no base; the
// other two bases fit the 16-bit immediate offset of the LDS read instructions.
// Two workgroups' tables (2 x 78592 B) fit the 160 KB of LDS of a CU.
constexpr int kI3Lut = 0;                     // 64 rows x 128 B (32 replicas x 4 B)
constexpr int kI2Lut = 64 * 128;              // 256 rows x 32 B (4 replicas x 8 B)
constexpr int kTLut = kI2Lut + 256 * 32;      // 243 rows x 256 B (16 replicas x 16 B)
constexpr int kLutBytes = kTLut + 243 * 256;  // 78592
static_assert(kTLut < 65536 && kI2Lut < 65536, "table bases must fit the LDS immediate offset");

// Every table row is computed once, the rows of all three tables spread over
// all NT threads of the workgroup, and the thread that computes a row writes
// all its replicas, starting at replica (row mod REP): consecutive threads then
// write different banks at every step, and no barrier or copy pass separates
// computing from replicating.  (Computing every slot separately cost about
// 2 us per launch, which is much of a short launch.)  The caller's barrier
// follows.
template <int NT>
__device__ inline void build_luts(uint8_t* smem) {
  const int t = threadIdx.x;
  for (int r = t; r < 243 + 256 + 64; r += NT) {
    if (r < 243) {  // ternary: 243 rows x 16 replicas x 16 B
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
#pragma unroll
      for (int i = 0; i < 16; ++i) *reinterpret_cast<uint4*>(smem + kTLut + r * 256 + 16 * ((r + i) & 15)) = q;
    } else if (r < 243 + 256) {  // 2-bit: 256 rows x 4 replicas x 8 B
      const int b = r - 243;
      uint2 q;
      q.x = code_bf16((b & 3) - 2) | (code_bf16(((b >> 2) & 3) - 2) << 16);
      q.y = code_bf16(((b >> 4) & 3) - 2) | (code_bf16(((b >> 6) & 3) - 2) << 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<uint2*>(smem + kI2Lut + b * 32 + 8 * ((b + i) & 3)) = q;
    } else {  // 3-bit: 64 rows x 32 replicas x 4 B
      const int e = r - 243 - 256;
      const uint32_t q = code_bf16((e & 7) - 4) | (code_bf16((e >> 3) - 4) << 16);
#pragma unroll
      for (int i = 0; i < 32; ++i) *reinterpret_cast<uint32_t*>(smem + kI3Lut + e * 128 + 4 * ((e + i) & 31)) = q;
    }
  }
}

// Replica offset of a lane in the 3-bit table.
__device__ __forceinline__ uint32_t i3_lane_off(int lane) { return (uint32_t)(lane & 31) << 2; }

// 3-bit table address of field P of the 96-bit triple w0|w1<<32|w2<<64: the
// 6-bit field times the 128-byte row, plus the lane's replica offset (i3_lane_off).
// One shift or funnel shift brings the field to bits 7..12, one and-or adds the offset.
template <int P>
__device__ __forceinline__ uint32_t i3_addr(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t lane_off) {
  constexpr int bit = 6 * P;
  constexpr int s = bit - 7;  // right shift of the 96-bit value that puts the field at bit 7
  uint32_t v;
  if constexpr (s < 0) {
    v = w0 << -s;
  } else {
    constexpr int wi = s / 32, sh = s % 32;
    const uint32_t lo = wi == 0 ? w0 : wi == 1 ? w1 : w2;
    if constexpr (bit + 6 <= 32 * (wi + 1)) {
      v = lo >> sh;
    } else {
      static_assert(wi < 2, "a field past bit 96");
      v = __builtin_amdgcn_alignbit(wi == 0 ? w1 : w2, lo, sh);
    }
  }
  return (v & 0x1F80u) | lane_off;
}

}  // namespace ql
