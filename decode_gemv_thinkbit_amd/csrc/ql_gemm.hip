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
#include <utility>

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
// from the row's chunks (K0/5)/16 and ((K0+31)/5)/16 of the period.
template <int K0>
__device__ __forceinline__ void decode_t32(const u32x4g_t (&ch)[2], const uint8_t* lut, uint16_t* dst) {
  constexpr int J0 = K0 / 5, J1 = (K0 + 31) / 5;  // bytes covering the range
  constexpr int C0 = J0 / 16;
  u32x4g_t e[J1 - J0 + 1];
  gfor<J1 - J0 + 1>([&](auto ji) __attribute__((always_inline)) {
    constexpr int j = J0 + decltype(ji)::value;
    const uint32_t w = dword_of(ch[j / 16 - C0], (j & 15) >> 2);
    const uint32_t b = (w >> (8 * (j & 3))) & 0xFFu;
    e[decltype(ji)::value] = *(lq4p)(lut + ((j & 1) ? kLutT1 : kLutT0) + b * 16);
  });
  uint32_t o[16];
  gfor<16>([&](auto pi) __attribute__((always_inline)) {
    constexpr int k = K0 + 2 * decltype(pi)::value;
    constexpr int j = k / 5 - J0, t = k % 5;
    if constexpr (t == 0) o[decltype(pi)::value] = e[j].x;
    else if constexpr (t == 2) o[decltype(pi)::value] = e[j].y;
    else if constexpr (t == 1) o[decltype(pi)::value] = __builtin_amdgcn_alignbit(e[j].y, e[j].x, 16);
    else if constexpr (t == 3) o[decltype(pi)::value] = __builtin_amdgcn_alignbit(e[j].z, e[j].y, 16);
    else o[decltype(pi)::value] = __builtin_amdgcn_perm(e[j + 1].x, e[j].z, 0x05040100u);
  });
  put32(dst, o);
}

// 2-bit: codes [128g + 32q, +32) of one row = group bytes 8q..8q+7, staged as
// ch[0].x, ch[0].y.
__device__ __forceinline__ void decode_i2_32(const u32x4g_t (&ch)[2], const uint8_t* lut, uint16_t* dst) {
  const uint32_t wd[2] = {ch[0].x, ch[0].y};
  uint32_t o[16];
  gfor<8>([&](auto bi) __attribute__((always_inline)) {
    constexpr int j = decltype(bi)::value;  // byte of the quarter
    const uint32_t b = (wd[j >> 2] >> (8 * (j & 3))) & 0xFFu;
    const u32x2g_t e = *(lq2p)(lut + kLutI2 + b * 8);
    o[2 * j] = e.x;
    o[2 * j + 1] = e.y;
  });
  put32(dst, o);
}

// 3-bit: codes [128g + 32q, +32) of one row = the 96-bit triple at group bytes
// 12q..12q+11, staged as ch[0].x, ch[0].y, ch[0].z (low word first).
__device__ __forceinline__ void decode_i3_32(const u32x4g_t (&ch)[2], const uint8_t* lut, uint16_t* dst) {
  const uint32_t w0 = ch[0].x, w1 = ch[0].y, w2 = ch[0].z;
  uint32_t o[16];
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
  put32(dst, o);
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
    if (tid < kTileN && sc_n < a.N) st.sc = a.pscales[pscale_index(sc_n, g, G8)];
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
// row slices per workgroup: 8 (32 tokens), 4 (64 tokens) or 2 (128 tokens)
int row_slices(int64_t M) { return M <= 32 ? 8 : (M <= 64 ? 4 : 2); }
int64_t tile_tokens(int64_t M) { return 256 / row_slices(M); }

// K splits that bring the launch to about two workgroups per CU (at least two
// groups per split); 1 when the matrix alone fills the device.
int choose_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t mt = tile_tokens(M);
  const int64_t tiles = ((N + kTileN - 1) / kTileN) * ((M + mt - 1) / mt);
  const int64_t want = 2 * (int64_t)device_cu_count();
  int64_t s = (want + tiles - 1) / tiles;
  const int64_t G = K / kGroup;
  if (s > G / 2) s = G / 2;
  if (s > 16) s = 16;
  return s < 1 ? 1 : (int)s;
}
}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int s = choose_splits(M, N, K);
  return s > 1 ? (size_t)s * M * N * sizeof(float) : 0;
}

hipError_t launch_gemm(const MatArgs& a, int M, void* workspace, size_t ws_bytes, hipStream_t stream) {
  int s = choose_splits(M, a.N, a.K);
  if (s > 1 && (!workspace || ws_bytes < (size_t)s * M * a.N * sizeof(float))) s = 1;
  const int wr = row_slices(M);
  const int64_t mt = tile_tokens(M);
  const dim3 grid((unsigned)((a.N + kTileN - 1) / kTileN), (unsigned)((M + mt - 1) / mt), (unsigned)s);
  float* part = static_cast<float*>(workspace);
  if (wr == 8)
    hipLaunchKernelGGL(gemm_kernel<8>, grid, dim3(kThreads), 0, stream, a, M, s, part);
  else if (wr == 4)
    hipLaunchKernelGGL(gemm_kernel<4>, grid, dim3(kThreads), 0, stream, a, M, s, part);
  else
    hipLaunchKernelGGL(gemm_kernel<2>, grid, dim3(kThreads), 0, stream, a, M, s, part);
  if (s > 1) {
    const int64_t n = (int64_t)M * a.N;
    const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3(blocks), dim3(256), 0, stream, part, a.y, n, s);
  }
  return hipGetLastError();
}

}  // namespace ql
