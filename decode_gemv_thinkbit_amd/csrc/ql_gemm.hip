// Batched GEMM over ThinkBit-packed weights: LDS-staged bf16 code tiles + MFMA.
//
// For M tokens the product is a dense contraction, so it runs on the matrix
// cores.  A workgroup owns a 128-row grid block (one grid for all its rows)
// and up to 128 tokens.  Per 128-deep step (one scale group) the block's codes
// are decoded into LDS as bf16 integers (exact), the activation tile is staged
// beside it, and v_mfma_f32_16x16x32_bf16 accumulates the group's partial
// products in fp32; the group scale (ThinkBit summary page,
// onedev.kr/papers/1416, section "How it works": w = c * s, one scale per 128
// inputs) multiplies that partial once.  Computing on dequantized bf16 values
// reproduces the native low-bit result (k-quant calibration page,
// sotaaz.com/post/quantized-model-less-sure, section "Not just any noise");
// here the scale is kept out of the bf16 operand, so every product is exact.
//
// Matrices with few row blocks split K across workgroups; the partial sums go
// to the caller's workspace and a second kernel adds them in a fixed order, so
// results stay bitwise deterministic.
#include <algorithm>
#include <numeric>
#include <type_traits>
#include <utility>
#include <vector>

#include "ql_internal.hpp"

namespace ql {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef uint32_t u32x2g_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4g_t __attribute__((ext_vector_type(4)));

constexpr int kTileN = 128;    // rows per workgroup (one grid block)
constexpr int kPad = 136;      // bf16 per LDS tile row (128 + 8: rows start on different banks)
constexpr int kThreads = 512;  // 8 waves

// Decode tables (LDS), entries in input order:
//   ternary even / odd stored byte -> (c0,c1) (c2,c3) (c4,0) 0   [16 B]
//   2-bit byte -> (c0,c1) (c2,c3)                                [8 B]
//   3-bit 6-bit field -> (c0,c1)                                 [4 B]
constexpr int kLutT0 = 0;
constexpr int kLutT1 = 243 * 16;
constexpr int kLutI2 = 2 * 243 * 16;
constexpr int kLutI3 = kLutI2 + 256 * 8;
constexpr int kLutBytes = kLutI3 + 64 * 4;

template <class F, int... I>
__device__ __forceinline__ void gfor_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void gfor(F&& f) {
  gfor_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ void gemm_build_luts(uint8_t* lut) {
  for (int e = threadIdx.x; e < 2 * 243; e += blockDim.x) {
    const int odd = e >= 243, b = odd ? e - 243 : e;
    int d[5], v = b;
    for (int i = 0; i < 5; ++i) {
      d[i] = v % 3 - 1;
      v /= 3;
    }
    // input order: even bytes keep digit order; odd bytes hold input 0 as digit 4
    int c[5];
    for (int t = 0; t < 5; ++t) c[t] = odd ? (t == 0 ? d[4] : d[t - 1]) : d[t];
    uint4 q;
    q.x = code_bf16(c[0]) | (code_bf16(c[1]) << 16);
    q.y = code_bf16(c[2]) | (code_bf16(c[3]) << 16);
    q.z = code_bf16(c[4]);
    q.w = 0;
    *reinterpret_cast<uint4*>(lut + (odd ? kLutT1 : kLutT0) + b * 16) = q;
  }
  for (int b = threadIdx.x; b < 256; b += blockDim.x) {
    uint2 q;
    q.x = code_bf16((b & 3) - 2) | (code_bf16(((b >> 2) & 3) - 2) << 16);
    q.y = code_bf16(((b >> 4) & 3) - 2) | (code_bf16(((b >> 6) & 3) - 2) << 16);
    *reinterpret_cast<uint2*>(lut + kLutI2 + b * 8) = q;
  }
  for (int e = threadIdx.x; e < 64; e += blockDim.x)
    *reinterpret_cast<uint32_t*>(lut + kLutI3 + e * 4) = code_bf16((e & 7) - 4) | (code_bf16((e >> 3) - 4) << 16);
}

typedef const __attribute__((address_space(1))) u32x4g_t* gq4p;
// scales through a global-address-space pointer: a flat load would also count against
// the LDS counter, and the next LDS operand wait would then wait for it
typedef const __attribute__((address_space(1))) uint16_t* gu16g_p;
typedef const __attribute__((address_space(3))) u32x4g_t* lq4p;
typedef const __attribute__((address_space(3))) u32x2g_t* lq2p;
typedef const __attribute__((address_space(3))) uint32_t* lq1p;

// 16 bytes of a row: chunk c of row r of a slab (zero for a missing slab)
__device__ __forceinline__ u32x4g_t row_chunk(const uint8_t* slab, int r, int64_t c) {
  u32x4g_t v = {0u, 0u, 0u, 0u};
  if (slab) v = *(gq4p)(slab + c * kSlabChunkBytes + r * kChunkBytes);
  return v;
}

// byte offset b (4-aligned) of group bytes of a row -> the dword, zero for a missing slab
__device__ __forceinline__ uint32_t row_dword(const uint8_t* slab, int r, int64_t byte) {
  uint32_t v = 0u;
  if (slab) v = *(const __attribute__((address_space(1))) uint32_t*)(slab + (byte >> 4) * kSlabChunkBytes + r * kChunkBytes + (byte & 15));
  return v;
}
__device__ __forceinline__ u32x2g_t row_dword2(const uint8_t* slab, int r, int64_t byte) {
  u32x2g_t v = {0u, 0u};
  if (slab) v = *(const __attribute__((address_space(1))) u32x2g_t*)(slab + (byte >> 4) * kSlabChunkBytes + r * kChunkBytes + (byte & 15));
  return v;
}

// The same reads of an existing slab, unconditional: a load merged with a default value
// makes the compiler wait for it (and for every load issued before it) at the merge.
__device__ __forceinline__ u32x4g_t row_chunk_at(const uint8_t* slab, int r, int64_t c) {
  return *(gq4p)(slab + c * kSlabChunkBytes + r * kChunkBytes);
}
__device__ __forceinline__ uint32_t row_dword_at(const uint8_t* slab, int r, int64_t byte) {
  return *(const __attribute__((address_space(1))) uint32_t*)(slab + (byte >> 4) * kSlabChunkBytes + r * kChunkBytes + (byte & 15));
}
__device__ __forceinline__ u32x2g_t row_dword2_at(const uint8_t* slab, int r, int64_t byte) {
  return *(const __attribute__((address_space(1))) u32x2g_t*)(slab + (byte >> 4) * kSlabChunkBytes + r * kChunkBytes + (byte & 15));
}

__device__ __forceinline__ uint32_t dword_of(const u32x4g_t& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Write 16 dwords (32 bf16 codes) to an LDS tile row.
__device__ __forceinline__ void put32(uint16_t* dst, const uint32_t (&o)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<uint4*>(dst + 8 * q) = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
}

// Ternary: codes of period-local inputs [K0, K0+32) of one row (K0 even, compile-time)
// from the row's chunks (K0/5)/16 and ((K0+31)/5)/16 of the period, as 16 bf16 pairs.
template <int K0>
__device__ __forceinline__ void decode_t32(const u32x4g_t (&ch)[2], const uint8_t* lut, uint32_t (&o)[16]) {
  constexpr int J0 = K0 / 5, J1 = (K0 + 31) / 5;  // bytes covering the range
  constexpr int C0 = J0 / 16;
  u32x4g_t e[J1 - J0 + 1];
  gfor<J1 - J0 + 1>([&](auto ji) __attribute__((always_inline)) {
    constexpr int j = J0 + decltype(ji)::value;
    const uint32_t w = dword_of(ch[j / 16 - C0], (j & 15) >> 2);
    const uint32_t b = (w >> (8 * (j & 3))) & 0xFFu;
    e[decltype(ji)::value] = *(lq4p)(lut + ((j & 1) ? kLutT1 : kLutT0) + b * 16);
  });
  gfor<16>([&](auto pi) __attribute__((always_inline)) {
    constexpr int k = K0 + 2 * decltype(pi)::value;
    constexpr int j = k / 5 - J0, t = k % 5;
    if constexpr (t == 0) o[decltype(pi)::value] = e[j].x;
    else if constexpr (t == 2) o[decltype(pi)::value] = e[j].y;
    else if constexpr (t == 1) o[decltype(pi)::value] = __builtin_amdgcn_alignbit(e[j].y, e[j].x, 16);
    else if constexpr (t == 3) o[decltype(pi)::value] = __builtin_amdgcn_alignbit(e[j].z, e[j].y, 16);
    else o[decltype(pi)::value] = __builtin_amdgcn_perm(e[j + 1].x, e[j].z, 0x05040100u);
  });
}
template <int K0>
__device__ __forceinline__ void decode_t32(const u32x4g_t (&ch)[2], const uint8_t* lut, uint16_t* dst) {
  uint32_t o[16];
  decode_t32<K0>(ch, lut, o);
  put32(dst, o);
}

// 2-bit: codes [128g + 32q, +32) of one row = group bytes 8q..8q+7, staged as
// ch[0].x, ch[0].y.
__device__ __forceinline__ void decode_i2_32(const u32x4g_t (&ch)[2], const uint8_t* lut, uint32_t (&o)[16]) {
  const uint32_t wd[2] = {ch[0].x, ch[0].y};
  gfor<8>([&](auto bi) __attribute__((always_inline)) {
    constexpr int j = decltype(bi)::value;  // byte of the quarter
    const uint32_t b = (wd[j >> 2] >> (8 * (j & 3))) & 0xFFu;
    const u32x2g_t e = *(lq2p)(lut + kLutI2 + b * 8);
    o[2 * j] = e.x;
    o[2 * j + 1] = e.y;
  });
}
__device__ __forceinline__ void decode_i2_32(const u32x4g_t (&ch)[2], const uint8_t* lut, uint16_t* dst) {
  uint32_t o[16];
  decode_i2_32(ch, lut, o);
  put32(dst, o);
}

// 3-bit: codes [128g + 32q, +32) of one row = the 96-bit triple at group bytes
// 12q..12q+11, staged as ch[0].x, ch[0].y, ch[0].z (low word first).
__device__ __forceinline__ void decode_i3_32(const u32x4g_t (&ch)[2], const uint8_t* lut, uint32_t (&o)[16]) {
  const uint32_t w0 = ch[0].x, w1 = ch[0].y, w2 = ch[0].z;
  gfor<16>([&](auto pi) __attribute__((always_inline)) {
    constexpr int P = decltype(pi)::value;
    constexpr int bit = 6 * P;  // first bit of the 6-bit field
    uint32_t f;
    if constexpr (bit + 6 <= 32) f = (w0 >> bit) & 63u;
    else if constexpr (bit < 32) f = __builtin_amdgcn_alignbit(w1, w0, bit) & 63u;
    else if constexpr (bit + 6 <= 64) f = (w1 >> (bit - 32)) & 63u;
    else if constexpr (bit < 64) f = __builtin_amdgcn_alignbit(w2, w1, bit - 32) & 63u;
    else f = (w2 >> (bit - 64)) & 63u;
    o[P] = *(lq1p)(lut + kLutI3 + f * 4);
  });
}
__device__ __forceinline__ void decode_i3_32(const u32x4g_t (&ch)[2], const uint8_t* lut, uint16_t* dst) {
  uint32_t o[16];
  decode_i3_32(ch, lut, o);
  put32(dst, o);
}

// Selector tables of the large-tile kernel: the layout of the code tables above
// (ternary and 2-bit offsets identical, so decode_t32 / decode_i2_32 assemble
// selector pairs exactly as they assemble code pairs), but each 16-bit half is a
// v_perm byte selector that picks the bf16 value c * s of its code out of a
// register pair built once per group:
//   ternary, 2-bit: bytes 0-1 = s, 2-3 = -s, 4-5 = -2s (code 0 -> selector 0x0C, a zero byte);
//   3-bit: bytes 0-1 = s, 2-3 = 2s, 4-5 = 3s, 6-7 = 4s picked by |c|, with a
//   sign mask per code (entries 8 B: selector pair, sign pair).
// Each value is RNE(c * s) in bf16, so one v_perm per pair (and one xor for
// 3-bit) replaces the multiply and rounding of every pair.
constexpr int kSelI3 = kLutI2 + 256 * 8;
constexpr int kSelBytes = kSelI3 + 64 * 8;

__device__ __forceinline__ uint32_t sel_tern(int c) { return c == 1 ? 0x0100u : (c == -1 ? 0x0302u : (c == -2 ? 0x0504u : 0x0C0Cu)); }
__device__ __forceinline__ uint32_t sel_mag(int c) {
  const int m = c < 0 ? -c : c;
  return m == 0 ? 0x0C0Cu : (uint32_t)(((2 * m - 1) << 8) | (2 * m - 2));
}

__device__ void gemm2_build_luts(uint8_t* lut) {
  for (int e = threadIdx.x; e < 2 * 243; e += blockDim.x) {
    const int odd = e >= 243, b = odd ? e - 243 : e;
    int d[5], v = b;
    for (int i = 0; i < 5; ++i) {
      d[i] = v % 3 - 1;
      v /= 3;
    }
    int c[5];
    for (int t = 0; t < 5; ++t) c[t] = odd ? (t == 0 ? d[4] : d[t - 1]) : d[t];
    uint4 q;
    q.x = sel_tern(c[0]) | (sel_tern(c[1]) << 16);
    q.y = sel_tern(c[2]) | (sel_tern(c[3]) << 16);
    q.z = sel_tern(c[4]);
    q.w = 0;
    *reinterpret_cast<uint4*>(lut + (odd ? kLutT1 : kLutT0) + b * 16) = q;
  }
  for (int b = threadIdx.x; b < 256; b += blockDim.x) {
    uint2 q;
    q.x = sel_tern((b & 3) - 2) | (sel_tern(((b >> 2) & 3) - 2) << 16);
    q.y = sel_tern(((b >> 4) & 3) - 2) | (sel_tern(((b >> 6) & 3) - 2) << 16);
    *reinterpret_cast<uint2*>(lut + kLutI2 + b * 8) = q;
  }
  for (int e = threadIdx.x; e < 64; e += blockDim.x) {
    const int c0 = (e & 7) - 4, c1 = (e >> 3) - 4;
    uint2 q;
    q.x = sel_mag(c0) | (sel_mag(c1) << 16);
    q.y = (c0 < 0 ? 0x8000u : 0u) | (c1 < 0 ? 0x80000000u : 0u);
    *reinterpret_cast<uint2*>(lut + kSelI3 + e * 8) = q;
  }
}

// 3-bit through the selector table: magnitude selector pairs o and sign masks sg.
__device__ __forceinline__ void decode_i3_32_sel(const u32x4g_t (&ch)[2], const uint8_t* lut, uint32_t (&o)[16],
                                                 uint32_t (&sg)[16]) {
  const uint32_t w0 = ch[0].x, w1 = ch[0].y, w2 = ch[0].z;
  gfor<16>([&](auto pi) __attribute__((always_inline)) {
    constexpr int P = decltype(pi)::value;
    constexpr int bit = 6 * P;
    uint32_t f;
    if constexpr (bit + 6 <= 32) f = (w0 >> bit) & 63u;
    else if constexpr (bit < 32) f = __builtin_amdgcn_alignbit(w1, w0, bit) & 63u;
    else if constexpr (bit + 6 <= 64) f = (w1 >> (bit - 32)) & 63u;
    else if constexpr (bit < 64) f = __builtin_amdgcn_alignbit(w2, w1, bit - 32) & 63u;
    else f = (w2 >> (bit - 64)) & 63u;
    const u32x2g_t e = *(lq2p)(lut + kSelI3 + f * 8);
    o[P] = e.x;
    sg[P] = e.y;
  });
}

// Workgroup barrier that orders LDS only: the next group's global loads stay
// in flight across it (a plain __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

// One group's operands in registers, loaded a step ahead of their use.
struct Stage {
  u32x4g_t xv[4];  // 32 bf16 of one token
  u32x4g_t ch[2];  // code chunks covering this thread's quarter of the group
  uint32_t sc;     // bf16 scale of row tid (threads < 128)
};

// One workgroup: row block blockIdx.x (2 slabs), tokens [m0, m0 + MT), groups of split blockIdx.z.
// 8 waves: WR row slices of 128/WR rows x 8/WR token slices of 32 tokens... (MT = 256/WR).
// Per group: codes staged in registers are decoded into LDS with the x tile and
// scales; after one barrier the next group's global loads are issued and the
// MFMAs and the scale epilogue of this group run from LDS, so the loads' latency
// hides behind the matrix work.
#ifndef QL_GEMM_WAVES_PER_EU
#define QL_GEMM_WAVES_PER_EU 2
#endif
template <int WR>
__global__ void __launch_bounds__(kThreads, QL_GEMM_WAVES_PER_EU) gemm_kernel(MatArgs a, int M, int nsplit, float* __restrict__ part) {
  constexpr int WM = 8 / WR;         // token slices
  constexpr int RB = 8 / WR;         // 16-row blocks per wave (128 / WR rows)
  constexpr int MB = 2;              // 16-token blocks per wave
  constexpr int MT = 16 * MB * WM;   // tokens per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t wt[2][kTileN * kPad];
  __shared__ __attribute__((aligned(16))) uint16_t xt[2][MT * kPad];
  __shared__ __attribute__((aligned(16))) float sct[2][kTileN];
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLutBytes];
  gemm_build_luts(lut);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, G = K / kGroup, G8 = (G + 7) / 8;
  const int64_t nslabs = ((int64_t)a.N + kSlab - 1) / kSlab;
  const int64_t blk = blockIdx.x;
  const int m0 = blockIdx.y * MT;
  const int z = blockIdx.z;
  const int g_lo = (int)((int64_t)G * z / nsplit), g_hi = (int)((int64_t)G * (z + 1) / nsplit);
  int gr;
  const int64_t off0 = slab_offset(2 * blk, K, a.grid, a.blk_grid, a.blk_off, &gr);
  const uint8_t* slab0 = a.packed + off0;
  const uint8_t* slab1 = (2 * blk + 1 < nslabs) ? slab0 + (int64_t)kSlab * row_bytes(gr, K) : nullptr;

  // decode mapping: row dr, quarter dq (wave-uniform) of the group's 128 inputs
  const int dr = tid & 127, dq = __builtin_amdgcn_readfirstlane(tid >> 7);
  const uint8_t* dslab = dr < kSlab ? slab0 : slab1;
  const int dslab_r = dr & (kSlab - 1);
  const int drow_off = dr * kPad + 32 * dq;
  // x mapping: token xt_t, quarter xt_q
  const int xt_t = tid >> 2, xt_q = tid & 3;
  const bool x_ok = xt_t < MT && m0 + xt_t < M;
  const uint16_t* xrow = a.x + (int64_t)(x_ok ? m0 + xt_t : 0) * K + 32 * xt_q;
  const int64_t sc_n = blk * kTileN + tid;

  Stage st;
  auto load = [&](int g) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      st.xv[q] = u32x4g_t{0u, 0u, 0u, 0u};
      if (x_ok) st.xv[q] = *(gq4p)(xrow + (int64_t)g * kGroup + 8 * q);
    }
    if (gr == QL_GRID_T) {
      const int64_t p = g / 5;
      const int k0 = 128 * (g - 5 * (int)p) + 32 * dq;
      const int c0 = (k0 / 5) / 16, c1 = ((k0 + 31) / 5) / 16;
      st.ch[0] = row_chunk(dslab, dslab_r, 8 * p + c0);
      st.ch[1] = row_chunk(dslab, dslab_r, 8 * p + c1);
    } else if (gr == QL_GRID_I2) {
      // only the quarter's 8 bytes; every branch writes both slots: stores to one
      // slot or the other would be merged into one store with a computed address,
      // which keeps st in memory
      const u32x2g_t v = row_dword2(dslab, dslab_r, 32 * (int64_t)g + 8 * dq);
      st.ch[0] = u32x4g_t{v.x, v.y, 0u, 0u};
      st.ch[1] = u32x4g_t{0u, 0u, 0u, 0u};
    } else {
      // only the quarter's 12 bytes, as three aligned dwords (none straddles a chunk)
      const int64_t b0 = 48 * (int64_t)g + 12 * dq;
      st.ch[0] = u32x4g_t{row_dword(dslab, dslab_r, b0), row_dword(dslab, dslab_r, b0 + 4),
                          row_dword(dslab, dslab_r, b0 + 8), 0u};
      st.ch[1] = u32x4g_t{0u, 0u, 0u, 0u};
    }
    st.sc = 0;
    if (tid < kTileN && sc_n < a.N) st.sc = ((gu16g_p)a.pscales)[pscale_index(sc_n, g, G8)];
  };
  // x tile and scales of the staged group into LDS buffer b
  auto put_x = [&](int b) __attribute__((always_inline)) {
    if (xt_t < MT) {
      uint16_t* dst = xt[b] + xt_t * kPad + 32 * xt_q;
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4g_t*>(dst + 8 * q) = st.xv[q];
    }
    if (tid < kTileN) sct[b][tid] = bf16_bits_to_f32(st.sc);
  };

  // MFMA mapping: wave (wr, wm) computes rows (128/WR)wr.. x tokens 32wm..
  const int wr = wave % WR, wm = wave / WR;
  f32x4_t acc[RB][MB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[rb][mb] = f32x4_t{0, 0, 0, 0};

  // the MFMAs and scale epilogue of the group in LDS buffer b
  auto mma = [&](int b) __attribute__((always_inline)) {
    const uint16_t* wtb = wt[b];
    const uint16_t* xtb = xt[b];
    f32x4_t pr[RB][MB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) pr[rb][mb] = f32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kk = 32 * ks + 8 * (lane >> 4);
      bf16x8_t av[RB], bv[MB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        av[rb] = *reinterpret_cast<const bf16x8_t*>(wtb + ((128 / WR) * wr + 16 * rb + (lane & 15)) * kPad + kk);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        bv[mb] = *reinterpret_cast<const bf16x8_t*>(xtb + (32 * wm + 16 * mb + (lane & 15)) * kPad + kk);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          pr[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[rb], bv[mb], pr[rb][mb], 0, 0, 0);
    }
    // D lane l: rows 4*(l/16)+i of the 16-row block, token l%16 of the 16-token block
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const f32x4_t s4 = *reinterpret_cast<const f32x4_t*>(sct[b] + (128 / WR) * wr + 16 * rb + 4 * (lane >> 4));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[rb][mb][i] = fmaf(s4[i], pr[rb][mb][i], acc[rb][mb][i]);
    }
  };

  // decode of the staged group (dq is wave-uniform: one branch per wave)
  auto decode_t = [&](auto ii, int b) __attribute__((always_inline)) {
    constexpr int i = decltype(ii)::value;
    uint16_t* drow = wt[b] + drow_off;
    if (dq == 0) decode_t32<128 * i>(st.ch, lut, drow);
    else if (dq == 1) decode_t32<128 * i + 32>(st.ch, lut, drow);
    else if (dq == 2) decode_t32<128 * i + 64>(st.ch, lut, drow);
    else decode_t32<128 * i + 96>(st.ch, lut, drow);
  };
  auto decode_i2 = [&](int b) __attribute__((always_inline)) { decode_i2_32(st.ch, lut, wt[b] + drow_off); };
  auto decode_i3 = [&](int b) __attribute__((always_inline)) { decode_i3_32(st.ch, lut, wt[b] + drow_off); };

  // Two LDS buffers, one barrier per step: step d decodes group d (its codes
  // were loaded into registers one step earlier) into buffer (d - g_lo) & 1,
  // issues the loads of group d + 1, and runs the MFMAs of group d - 1 from the
  // other buffer.  Each grid keeps a single decode call site.
  __syncthreads();  // tables ready
  if (g_lo < g_hi) load(g_lo);
  auto step = [&](int d, auto&& decode) __attribute__((always_inline)) {
    const int b = (d - g_lo) & 1;
    if (d < g_hi) {
      decode(b);
      put_x(b);
      if (d + 1 < g_hi) load(d + 1);
    }
    if (d > g_lo) mma(b ^ 1);
    lds_barrier();
  };
  if (gr == QL_GRID_T) {
    // periods of 640 inputs: the byte positions of every group are compile-time
    for (int64_t p = g_lo / 5; 5 * p <= g_hi; ++p) {
      gfor<5>([&](auto ii) __attribute__((always_inline)) {
        const int d = (int)(5 * p) + decltype(ii)::value;
        if (d >= g_lo && d <= g_hi) step(d, [&](int b) __attribute__((always_inline)) { decode_t(ii, b); });
      });
    }
  } else if (gr == QL_GRID_I2) {
    for (int d = g_lo; d <= g_hi; ++d) step(d, decode_i2);
  } else {
    for (int d = g_lo; d <= g_hi; ++d) step(d, decode_i3);
  }

  // store: y directly, or this split's partial sums
  float* out = nsplit > 1 ? part + (int64_t)z * M * a.N : a.y;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t n = blk * kTileN + (128 / WR) * wr + 16 * rb + 4 * (lane >> 4);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int t = m0 + 32 * wm + 16 * mb + (lane & 15);
      if (t >= M) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n + i < a.N) out[(int64_t)t * a.N + n + i] = acc[rb][mb][i];
    }
  }
}

// ---------------------------------------------------------------- large-tile kernel
// The contraction of 16 and more tokens.  A workgroup of 8 waves owns 256
// weight rows (two grid blocks) x 64*TA tokens; each wave computes 64 rows x
// 32*TA tokens with v_mfma_f32_32x32x16_bf16 (x fragments as the first operand,
// weight fragments as the second, so the 32 lanes of a D register hold 32
// consecutive weight rows of one token and y is stored in 128-byte runs).
// Stages of 64 inputs are double-buffered in LDS with one barrier per stage:
// the waves decode stage s+1 into one buffer, issue the loads of stage s+2
// (codes, x, scales), and run the MFMAs of stage s from the other buffer.
//
// The weight operand is bf16 RNE(c * s), the group scale folded into the code
// (the dequantize-to-bf16 tile of the pages' BF16 reading: k-quant calibration
// page, section "Not just any noise").  For ternary and 2-bit codes, and 3-bit
// codes of magnitude 0, 1, 2 and 4, c * s is exact in bf16; only 3-bit codes of
// magnitude 3 are rounded.  Products are exact in fp32 and sums are fp32.
constexpr int kG2Rows = 256;  // weight rows per workgroup
constexpr int kG2K = 64;      // inputs per stage
constexpr int kG2Pad = 72;    // bf16 per LDS row: 64 + 8, so 16 lanes' 16-byte reads of 16 rows hit distinct banks
constexpr int kG2Threads = 512;

typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;


// LDS of one large-tile workgroup: double-buffered weight and activation stages
// and the selector tables.
template <int TA>
struct G2Smem {
  uint16_t wt[2][kG2Rows * kG2Pad];
  uint16_t xt[2][64 * TA * kG2Pad];
  uint8_t lut[kSelBytes];
};

// One tile: weight rows [256 bx, +256) x tokens [64 TA by, +64 TA) over stages of
// split z of nsplit (partial sums to part + z M N when nsplit > 1, else y).  The
// tables in sm.lut are built; the first barrier also separates this tile's LDS
// writes from the previous tile's last reads in a persistent launch.
template <int TA>
__device__ __forceinline__ void gemm2_tile(const MatArgs& a, int M, int nsplit, float* __restrict__ part, int bx,
                                           int by, int z, G2Smem<TA>& sm) {
  constexpr int MT = 64 * TA;         // tokens per workgroup
  constexpr int XQ = 8 / TA;          // threads per token row of a stage (16 * TA bytes each)
  auto& wt = sm.wt;
  auto& xt = sm.xt;
  const uint8_t* lut = sm.lut;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.K, G8 = (K / kGroup + 7) / 8;
  const int S = K / kG2K;  // stages of the row
  const int64_t n0 = (int64_t)bx * kG2Rows;
  const int m0 = by * MT;
  const int s_lo = (int)((int64_t)S * z / nsplit), s_hi = (int)((int64_t)S * (z + 1) / nsplit);
  const int64_t nslabs = ((int64_t)a.N + kSlab - 1) / kSlab;

  // decode mapping: row dr of the tile, half dh of the stage (wave-uniform), grid
  // block tid >> 8 of the tile (wave-uniform)
  const int dr = (tid & 127) + 128 * (tid >> 8);
  const int dh = __builtin_amdgcn_readfirstlane((tid >> 7) & 1);
  // Every load of the stage loop is unconditional: rows past the matrix's last slab read
  // its last row, and tokens past M read token 0; those rows and tokens are never stored,
  // and an output depends only on its own row and token.
  const int64_t dn = n0 + dr;
  const int64_t dn_c = dn < nslabs * kSlab ? dn : nslabs * kSlab - 1;
  int gr = QL_GRID_T;
  const uint8_t* dslab = a.packed + slab_offset(dn_c / kSlab, K, a.grid, a.blk_grid, a.blk_off, &gr);
  gr = __builtin_amdgcn_readfirstlane(gr);  // uniform: the wave's rows share one grid block
  const int dslab_r = (int)(dn_c & (kSlab - 1));
  // x mapping: token xr of the tile, piece xp (16 * TA bytes of the stage's 128)
  const int xr = tid / XQ, xp = tid % XQ;
  const uint16_t* xrow = a.x + (int64_t)(m0 + xr < M ? m0 + xr : 0) * K + 8 * TA * xp;

  struct Regs {
    u32x4g_t xv[TA];
    u32x4g_t ch[2];
    uint32_t sc;
  } st;
  auto load = [&](int s) __attribute__((always_inline)) {
    Regs& r = st;
#pragma unroll
    for (int q = 0; q < TA; ++q) r.xv[q] = *(gq4p)(xrow + (int64_t)s * kG2K + 8 * q);
    const int k0 = kG2K * s + 32 * dh;  // first input of this thread's 32
    if (gr == QL_GRID_T) {
      const int64_t p = k0 / kPeriodK;
      const int kp = k0 - (int)p * kPeriodK;
      r.ch[0] = row_chunk_at(dslab, dslab_r, 8 * p + (kp / 5) / 16);
      r.ch[1] = row_chunk_at(dslab, dslab_r, 8 * p + ((kp + 31) / 5) / 16);
    } else if (gr == QL_GRID_I2) {
      const u32x2g_t v = row_dword2_at(dslab, dslab_r, k0 / 4);
      r.ch[0] = u32x4g_t{v.x, v.y, 0u, 0u};
      r.ch[1] = u32x4g_t{0u, 0u, 0u, 0u};
    } else {
      const int64_t b0 = 3 * (int64_t)k0 / 8;
      r.ch[0] = u32x4g_t{row_dword_at(dslab, dslab_r, b0), row_dword_at(dslab, dslab_r, b0 + 4),
                          row_dword_at(dslab, dslab_r, b0 + 8), 0u};
      r.ch[1] = u32x4g_t{0u, 0u, 0u, 0u};
    }
    r.sc = (uint32_t)((gu16g_p)a.pscales)[pscale_index(dn_c, k0 / kGroup, G8)];
  };
  // decode the loaded stage s (bf16 c * s) and its x tile into buffer b
  auto put = [&](int s, int b) __attribute__((always_inline)) {
    const Regs& r = st;
    uint32_t o[16];
    const float sf = bf16_bits_to_f32(r.sc);
    if (gr == QL_GRID_T || gr == QL_GRID_I2) {
      // pair selectors, then v_perm from (s, -s | -2s, 0)
      if (gr == QL_GRID_T) {
      const int pos = (2 * ((kG2K * s) % kPeriodK) / kG2K) + dh;  // 32-input quarter within the period (0..19)
      switch (pos) {
#define QL_T_CASE(i) \
  case i:            \
    decode_t32<32 * i>(r.ch, lut, o); \
    break;
        QL_T_CASE(0) QL_T_CASE(1) QL_T_CASE(2) QL_T_CASE(3) QL_T_CASE(4) QL_T_CASE(5) QL_T_CASE(6)
        QL_T_CASE(7) QL_T_CASE(8) QL_T_CASE(9) QL_T_CASE(10) QL_T_CASE(11) QL_T_CASE(12) QL_T_CASE(13)
        QL_T_CASE(14) QL_T_CASE(15) QL_T_CASE(16) QL_T_CASE(17) QL_T_CASE(18)
        default: decode_t32<32 * 19>(r.ch, lut, o); break;
#undef QL_T_CASE
      }
      } else {
        decode_i2_32(r.ch, lut, o);
      }
      const uint32_t lo = r.sc | ((r.sc ^ 0x8000u) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_bits(2.0f * sf) ^ 0x8000u;
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] = __builtin_amdgcn_perm(hi, lo, o[i]);
    } else {
      uint32_t sg[16];
      decode_i3_32_sel(r.ch, lut, o, sg);
      const uint32_t lo = r.sc | ((uint32_t)f32_to_bf16_bits(2.0f * sf) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_bits(3.0f * sf) | ((uint32_t)f32_to_bf16_bits(4.0f * sf) << 16);
#pragma unroll
      for (int i = 0; i < 16; ++i) o[i] = __builtin_amdgcn_perm(hi, lo, o[i]) ^ sg[i];
    }
    uint16_t* dst = wt[b] + dr * kG2Pad + 32 * dh;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(dst + 8 * q) = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    uint16_t* xd = xt[b] + xr * kG2Pad + 8 * TA * xp;
#pragma unroll
    for (int q = 0; q < TA; ++q) *reinterpret_cast<u32x4g_t*>(xd + 8 * q) = r.xv[q];
  };

  // MFMA mapping: wave (th, rq) computes tokens [32 TA th, +32 TA) x rows [64 rq, +64)
  const int th = wave & 1, rq = wave >> 1;
  f32x16_t acc[TA][2];
#pragma unroll
  for (int ta = 0; ta < TA; ++ta)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ta][rb][r] = 0.0f;
  auto mma = [&](int b) __attribute__((always_inline)) {
    const uint16_t* xb = xt[b] + (32 * TA * th + (lane & 31)) * kG2Pad + 8 * (lane >> 5);
    const uint16_t* wb = wt[b] + (64 * rq + (lane & 31)) * kG2Pad + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < kG2K / 16; ++ks) {
      bf16x8_t av[TA], bv[2];
#pragma unroll
      for (int ta = 0; ta < TA; ++ta) av[ta] = *reinterpret_cast<const bf16x8_t*>(xb + 32 * ta * kG2Pad + 16 * ks);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) bv[rb] = *reinterpret_cast<const bf16x8_t*>(wb + 32 * rb * kG2Pad + 16 * ks);
#pragma unroll
      for (int ta = 0; ta < TA; ++ta)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[ta][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ta], bv[rb], acc[ta][rb], 0, 0, 0);
    }
  };

  // Per stage: decode stage s + 1 into the other buffer, issue the loads of stage
  // s + 2, then run the MFMAs of stage s.  The loads thus have the MFMAs, the
  // barrier and the next decode to arrive in (issued after the MFMAs, one stage
  // ahead, they had only the MFMAs: 433-439 against 480 us per Qwen3-8B layer at
  // 512 tokens).
  __syncthreads();  // tables ready
  if (s_lo < s_hi) {
    load(s_lo);
    put(s_lo, 0);
    if (s_lo + 1 < s_hi) load(s_lo + 1);
  }
  __syncthreads();
  // With 256 tokens per tile the two waves of a SIMD run the stage in opposite
  // orders (one MFMAs first, the other decode first), so one's matrix work overlaps
  // the other's decode between the barriers (same-box: 4.7 % faster on a Qwen3-8B
  // layer at 256 and 512 tokens; at 64 tokens, where a stage's MFMAs are few, 3 %
  // slower, so smaller tiles keep one order).
  // Each order is a loop of its own with one MFMA call site: with both orders in one loop
  // the accumulators took two register sets and were copied between them every stage.
  auto stages = [&](auto mf) __attribute__((always_inline)) {
    constexpr bool kMfmaFirst = decltype(mf)::value;
    for (int s = s_lo; s < s_hi; ++s) {
      const int b = (s - s_lo) & 1;
      if constexpr (kMfmaFirst) mma(b);
      if (s + 1 < s_hi) {
        put(s + 1, b ^ 1);
        if (s + 2 < s_hi) load(s + 2);
      }
      if constexpr (!kMfmaFirst) mma(b);
      lds_barrier();
    }
  };
  if (TA == 4 && __builtin_amdgcn_readfirstlane(wave) >= 4) stages(std::true_type{});
  else stages(std::false_type{});

  // D register r of lane l: token 8 (r / 4) + 4 (l / 32) + r % 4 of the 32-token block,
  // weight row l % 32 of the 32-row block (global stores: flat ones would also count
  // against the LDS counter, which the next tile's first waits use)
  __attribute__((address_space(1))) float* out =
      (__attribute__((address_space(1))) float*)(nsplit > 1 ? part + (int64_t)z * M * a.N : a.y);
#pragma unroll
  for (int ta = 0; ta < TA; ++ta)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int64_t n = n0 + 64 * rq + 32 * rb + (lane & 31);
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = m0 + 32 * TA * th + 32 * ta + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (t < M) out[(int64_t)t * a.N + n] = acc[ta][rb][r];
      }
    }
}

template <int TA>
__global__ void __launch_bounds__(kG2Threads, 2) gemm2_kernel(MatArgs a, int M, int nsplit, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) G2Smem<TA> sm;
  gemm2_build_luts(sm.lut);
  gemm2_tile<TA>(a, M, nsplit, part, blockIdx.x, blockIdx.y, blockIdx.z, sm);
}

// Many matrices at one M in one persistent launch: task t (tasks numbered by the
// host in descriptor order, longest tasks first) runs on workgroup t mod grid.
// Entry d's tasks are its row tiles x token tiles x d.kparts K splits, from task
// d.slab_begin on; a split entry's partial sums go to ws + d.ws_begin.  Entries
// whose partials would not fit ws_floats (a workspace smaller than prepare asked
// for, or another M) run nothing.
template <int TA>
__global__ void __launch_bounds__(kG2Threads, 2) gemm2_grouped_kernel(const ql_gemv_desc* __restrict__ descs,
                                                                     int count, int64_t total, int M,
                                                                     float* __restrict__ ws, int64_t ws_floats) {
  __shared__ __attribute__((aligned(16))) G2Smem<TA> sm;
  gemm2_build_luts(sm.lut);
  constexpr int MT = 64 * TA;
  const int64_t mt = (M + MT - 1) / MT;
  for (int64_t t = blockIdx.x; t < total; t += gridDim.x) {
    int lo = 0, hi = count - 1;  // the last entry whose first task is at or before t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (descs[mid].slab_begin <= t) lo = mid; else hi = mid - 1;
    }
    const ql_gemv_desc& d = descs[lo];
    const int64_t rt = ((int64_t)d.N + kG2Rows - 1) / kG2Rows;
    const int s = d.kparts > 1 ? d.kparts : 1;
    const int64_t local = t - d.slab_begin;
    if (local >= rt * mt * s) continue;  // past the entry's own tasks (a larger total than prepare's)
    if (s > 1 && d.ws_begin + (int64_t)s * M * d.N > ws_floats) continue;
    const MatArgs a{static_cast<const uint8_t*>(d.packed), d.pscales, d.blk_grid, d.blk_off, d.x, d.y, d.N, d.K,
                    d.grid};
    gemm2_tile<TA>(a, M, s, s > 1 ? ws + d.ws_begin : nullptr, (int)(local / s / mt), (int)(local / s % mt),
                   (int)(local % s), sm);
  }
}

// y = sum over splits of the partials, in split order, for every split entry of a
// grouped launch (blockIdx.y = entry).
__global__ void __launch_bounds__(256) gemm_reduce_grouped_kernel(const ql_gemv_desc* __restrict__ descs, int M,
                                                                  const float* __restrict__ ws, int64_t ws_floats) {
  const ql_gemv_desc& d = descs[blockIdx.y];
  const int s = d.kparts;
  if (s <= 1) return;
  const int64_t n = (int64_t)M * d.N;
  if (d.ws_begin + s * n > ws_floats) return;
  const float* part = ws + d.ws_begin;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    float v = part[i];
    for (int z = 1; z < s; ++z) v += part[(int64_t)z * n + i];
    d.y[i] = v;
  }
}

// y = sum over splits of the partials, in split order.
__global__ void __launch_bounds__(256) gemm_reduce_kernel(const float* __restrict__ part, float* __restrict__ y,
                                                          int64_t n, int nsplit) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    float s = part[i];
    for (int z = 1; z < nsplit; ++z) s += part[(int64_t)z * n + i];
    y[i] = s;
  }
}

namespace {
// row slices per workgroup of the small-batch kernel: 8 (32 tokens), 4 (64 tokens) or 2 (128 tokens)
int row_slices(int64_t M) { return M <= 32 ? 8 : (M <= 64 ? 4 : 2); }
int64_t tile_tokens(int64_t M) { return 256 / row_slices(M); }

// Batches of at least this many tokens run on the large-tile kernel.
constexpr int64_t kLargeM = 16;
// 32-token blocks per wave of the large-tile kernel (workgroup tokens 64 * TA)
int large_ta(int64_t M) { return M <= 64 ? 1 : (M <= 128 ? 2 : 4); }

// K splits.  Large-tile kernel (one workgroup per CU): the split count minimising a
// cost model of whole workgroup rounds times the stages each workgroup runs, plus the
// partial sums a split writes and the reduction reads back (8 bytes per output and
// split, at about 5 TB/s, against about 3 us per stage and round).  Small-batch
// kernel: enough splits for about two workgroups per CU.  At least two groups (or
// two stages) per split, at most 16 splits.
int choose_splits(int64_t M, int64_t N, int64_t K) {
  int64_t tiles, units, per_cu;
  if (M >= kLargeM) {
    const int64_t mt = 64 * large_ta(M);
    tiles = ((N + kG2Rows - 1) / kG2Rows) * ((M + mt - 1) / mt);
    units = K / kG2K;
    const int64_t slots = device_cu_count();
    int best = 1;
    double best_us = 0.0;
    for (int64_t s = 1; s <= 16 && s <= (units < 2 ? 1 : units / 2); ++s) {
      const int64_t rounds = (tiles * s + slots - 1) / slots;
      const double us = (double)rounds * (double)((units + s - 1) / s) * 3.0 +
                        (s > 1 ? (double)s * (double)M * (double)N * 8.0 / 5.0e6 : 0.0);
      if (s == 1 || us < best_us) {
        best = (int)s;
        best_us = us;
      }
    }
    return best;
  } else {
    const int64_t mt = tile_tokens(M);
    tiles = ((N + kTileN - 1) / kTileN) * ((M + mt - 1) / mt);
    units = K / kGroup;
  }
  per_cu = 2;
  const int64_t want = per_cu * (int64_t)device_cu_count();
  int64_t s = (want + tiles - 1) / tiles;
  if (s > units / 2) s = units / 2;
  if (s > 16) s = 16;
  return s < 1 ? 1 : (int)s;
}
}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int s = choose_splits(M, N, K);
  return s > 1 ? (size_t)s * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm(const MatArgs& a, int M, void* workspace, size_t ws_bytes, hipStream_t stream) {
  return launch_gemm_as(a, M, workspace, ws_bytes, M >= kLargeM, stream);
}

// large: the large-tile kernel (bf16 c*s operands); otherwise the small-batch kernel
// (bf16 codes, fp32 scale per group: every product exact).
hipError_t launch_gemm_as(const MatArgs& a, int M, void* workspace, size_t ws_bytes, bool large, hipStream_t stream) {
  int s = choose_splits(M, a.N, a.K);
  if (s > 1 && (!workspace || ws_bytes < (size_t)s * M * a.N * sizeof(float))) s = 1;
  float* part = static_cast<float*>(workspace);
  if (large) {
    const int ta = large_ta(M);
    const int64_t mt = 64 * ta;
    const dim3 grid((unsigned)((a.N + kG2Rows - 1) / kG2Rows), (unsigned)((M + mt - 1) / mt), (unsigned)s);
    if (ta == 1)
      hipLaunchKernelGGL(gemm2_kernel<1>, grid, dim3(kG2Threads), 0, stream, a, M, s, part);
    else if (ta == 2)
      hipLaunchKernelGGL(gemm2_kernel<2>, grid, dim3(kG2Threads), 0, stream, a, M, s, part);
    else
      hipLaunchKernelGGL(gemm2_kernel<4>, grid, dim3(kG2Threads), 0, stream, a, M, s, part);
  } else {
    const int wr = row_slices(M);
    const int64_t mt = tile_tokens(M);
    const dim3 grid((unsigned)((a.N + kTileN - 1) / kTileN), (unsigned)((M + mt - 1) / mt), (unsigned)s);
    if (wr == 8)
      hipLaunchKernelGGL(gemm_kernel<8>, grid, dim3(kThreads), 0, stream, a, M, s, part);
    else if (wr == 4)
      hipLaunchKernelGGL(gemm_kernel<4>, grid, dim3(kThreads), 0, stream, a, M, s, part);
    else
      hipLaunchKernelGGL(gemm_kernel<2>, grid, dim3(kThreads), 0, stream, a, M, s, part);
  }
  if (s > 1) {
    const int64_t n = (int64_t)M * a.N;
    const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3(blocks), dim3(256), 0, stream, part, a.y, n, s);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- grouped plan
// Split counts of a grouped large-tile launch.  Workgroups (one per CU) take tasks
// round-robin in descriptor order, longest first; the plan simulates that order
// with a cost per task of its stages (measured per-stage times of this kernel at
// 64 / 128 / 256 tokens per tile) plus a fixed part and, for split entries, the
// partial tile it writes, and adds the reduction pass (every split entry's
// partials read once, y written once).  It first tries every common task length
// L (each entry split into the fewest parts of at most L stages) and every pair
// of lengths over subsets of the entries, keeps the cheapest, then moves, one
// entry at a time, the split (up or down) that lowers the estimate most, until no
// move does.
namespace {
double g2_stage_us(int ta) { return ta == 1 ? 1.7 : (ta == 2 ? 2.0 : 2.6); }

struct PlanEntry {
  int64_t tiles, stages, mn;
  int splits;
  double task_us(int ta) const {
    const double st = (double)((stages + splits - 1) / splits);
    const double part = splits > 1 ? 256.0 * 64.0 * ta * 4.0 / 60.0e3 : 0.0;  // partial tile at ~60 GB/s per CU
    return st * g2_stage_us(ta) + 3.0 + part;
  }
};

double plan_cost(const std::vector<PlanEntry>& e, const std::vector<int>& order, int ta, int cus) {
  std::vector<double> load(cus, 0.0);
  int64_t t0 = 0;
  double red = 0.0;
  bool any = false;
  for (int i : order) {
    const int64_t n = e[i].tiles * e[i].splits;
    const double us = e[i].task_us(ta);
    const int64_t full = n / cus, rem = n % cus;
    const int64_t b = t0 % cus;
    if (full)
      for (int w = 0; w < cus; ++w) load[w] += full * us;
    for (int64_t k = 0; k < rem; ++k) load[(b + k) % cus] += us;
    t0 += n;
    if (e[i].splits > 1) {
      red += (double)(e[i].splits + 1) * e[i].mn * 4.0 / 5.0e6;  // bytes at ~5 TB/s, in us
      any = true;
    }
  }
  return *std::max_element(load.begin(), load.end()) + (any ? red + 5.0 : 0.0);
}

std::vector<int> plan_order(const std::vector<PlanEntry>& e, int ta) {
  std::vector<int> o(e.size());
  std::iota(o.begin(), o.end(), 0);
  std::stable_sort(o.begin(), o.end(), [&](int a, int b) { return e[a].task_us(ta) > e[b].task_us(ta); });
  return o;
}
}  // namespace

int64_t gemm_grouped_plan(ql_gemv_desc* descs, int32_t count, int64_t M, int64_t* ws_floats) {
  const int ta = large_ta(M);
  const int64_t mt = (M + 64 * ta - 1) / (64 * ta);
  const int cus = device_cu_count();
  std::vector<PlanEntry> e(count);
  for (int32_t i = 0; i < count; ++i)
    e[i] = PlanEntry{((descs[i].N + kG2Rows - 1) / kG2Rows) * mt, descs[i].K / kG2K, M * descs[i].N, 1};
  auto max_splits = [](const PlanEntry& p) { return (int)std::max<int64_t>(1, std::min<int64_t>(16, p.stages / 2)); };
  double cur = -1.0;
  std::vector<int> best_s(count, 1);
  int64_t longest = 0;
  for (const PlanEntry& p : e) longest = std::max(longest, p.stages);
  for (int64_t L = longest; L >= 2; --L) {
    for (int32_t i = 0; i < count; ++i)
      e[i].splits = (int)std::min<int64_t>(max_splits(e[i]), (e[i].stages + L - 1) / L);
    const double c = plan_cost(e, plan_order(e, ta), ta, cus);
    if (cur < 0.0 || c < cur - 0.25) {
      cur = c;
      for (int32_t i = 0; i < count; ++i) best_s[i] = e[i].splits;
    }
  }
  // Two task lengths: the entries of a subset cut to the shorter one (for instance the
  // tiles that overflow the first round split in halves while the others stay whole);
  // every subset when there are at most 10 entries.
  if (count <= 10) {
    std::vector<int64_t> Ls;
    for (const PlanEntry& p : e)
      for (int k = 1; k <= 16; ++k) Ls.push_back((p.stages + k - 1) / k);
    std::sort(Ls.begin(), Ls.end());
    Ls.erase(std::unique(Ls.begin(), Ls.end()), Ls.end());
    for (size_t a = 0; a + 1 < Ls.size(); ++a)
      for (size_t b = a + 1; b < Ls.size() && b <= a + 3; ++b)
        for (uint32_t mask = 1; mask + 1 < (1u << count); ++mask) {
          for (int32_t i = 0; i < count; ++i) {
            const int64_t L = (mask >> i) & 1 ? Ls[a] : Ls[b];
            e[i].splits = (int)std::min<int64_t>(max_splits(e[i]), (e[i].stages + L - 1) / L);
          }
          const double c = plan_cost(e, plan_order(e, ta), ta, cus);
          if (c < cur - 0.25) {
            cur = c;
            for (int32_t i = 0; i < count; ++i) best_s[i] = e[i].splits;
          }
        }
  }
  for (int32_t i = 0; i < count; ++i) e[i].splits = best_s[i];
  for (int it = 0; it < 4 * count * 16; ++it) {
    int best = -1, best_step = 0;
    double best_cost = cur;
    for (int32_t i = 0; i < count; ++i)
      for (int step : {1, -1}) {
        if (e[i].splits + step < 1 || e[i].splits + step > max_splits(e[i])) continue;
        e[i].splits += step;
        const double c = plan_cost(e, plan_order(e, ta), ta, cus);
        e[i].splits -= step;
        if (c < best_cost - 0.25) {
          best = i;
          best_step = step;
          best_cost = c;
        }
      }
    if (best < 0) break;
    e[best].splits += best_step;
    cur = best_cost;
  }
  const std::vector<int> order = plan_order(e, ta);
  std::vector<ql_gemv_desc> sorted(count);
  int64_t total = 0, ws = 0;
  for (int32_t j = 0; j < count; ++j) {
    const int i = order[j];
    ql_gemv_desc d = descs[i];
    d.kparts = e[i].splits;
    d.reserved = 0;
    d.slab_begin = (int32_t)total;
    total += e[i].tiles * e[i].splits;
    d.ws_begin = 0;
    if (e[i].splits > 1) {
      d.ws_begin = ws;
      ws += (int64_t)e[i].splits * e[i].mn;
      ws = (ws + 63) / 64 * 64;  // each entry's partials start 256-byte aligned
    }
    sorted[j] = d;
  }
  std::copy(sorted.begin(), sorted.end(), descs);
  if (ws_floats) *ws_floats = ws;
  return total;
}

hipError_t launch_gemm_grouped(const ql_gemv_desc* descs, int32_t count, int64_t total, int M, float* ws,
                               int64_t ws_floats, hipStream_t stream) {
  const int ta = large_ta(M);
  const int grid = (int)std::min<int64_t>(total, device_cu_count());
  if (ta == 1)
    hipLaunchKernelGGL(gemm2_grouped_kernel<1>, dim3(grid), dim3(kG2Threads), 0, stream, descs, count, total, M, ws, ws_floats);
  else if (ta == 2)
    hipLaunchKernelGGL(gemm2_grouped_kernel<2>, dim3(grid), dim3(kG2Threads), 0, stream, descs, count, total, M, ws, ws_floats);
  else
    hipLaunchKernelGGL(gemm2_grouped_kernel<4>, dim3(grid), dim3(kG2Threads), 0, stream, descs, count, total, M, ws, ws_floats);
  if (ws_floats > 0) {
    // a split entry holds at most half the workspace: about sixteen outputs per thread for it
    const int64_t bx = std::min<int64_t>(2048, std::max<int64_t>(128, ws_floats / 2 / (256 * 16)));
    hipLaunchKernelGGL(gemm_reduce_grouped_kernel, dim3((unsigned)bx, count), dim3(256), 0, stream, descs, M, ws,
                       ws_floats);
  }
  return hipGetLastError();
}

}  // namespace ql
