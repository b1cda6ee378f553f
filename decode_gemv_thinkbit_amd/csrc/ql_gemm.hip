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
constexpr int kThreads = 256;  // 4 waves: 2 row halves x 2 token halves

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

__device__ __forceinline__ uint32_t dword_of(const u32x4g_t& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Write 32 dwords (64 bf16 codes) to an LDS tile row.
__device__ __forceinline__ void put64(uint16_t* dst, const uint32_t (&o)[32]) {
#pragma unroll
  for (int q = 0; q < 8; ++q)
    *reinterpret_cast<uint4*>(dst + 8 * q) = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
}

// Ternary: codes of period-local inputs [K0, K0+64) of one row (K0 even, compile-time).
template <int K0>
__device__ __forceinline__ void decode_t64(const uint8_t* slab, int r, int64_t p, const uint8_t* lut, uint16_t* dst) {
  constexpr int J0 = K0 / 5, J1 = (K0 + 63) / 5;  // bytes covering the range
  constexpr int C0 = J0 / 16, C1 = J1 / 16;       // their chunks (at most two)
  u32x4g_t ch[2];
  ch[0] = row_chunk(slab, r, 8 * p + C0);
  ch[1] = C1 != C0 ? row_chunk(slab, r, 8 * p + C1) : ch[0];
  u32x4g_t e[J1 - J0 + 1];
  gfor<J1 - J0 + 1>([&](auto ji) __attribute__((always_inline)) {
    constexpr int j = J0 + decltype(ji)::value;
    const uint32_t w = dword_of(ch[j / 16 - C0], (j & 15) >> 2);
    const uint32_t b = (w >> (8 * (j & 3))) & 0xFFu;
    e[decltype(ji)::value] = *(lq4p)(lut + ((j & 1) ? kLutT1 : kLutT0) + b * 16);
  });
  uint32_t o[32];
  gfor<32>([&](auto pi) __attribute__((always_inline)) {
    constexpr int k = K0 + 2 * decltype(pi)::value;
    constexpr int j = k / 5 - J0, t = k % 5;
    if constexpr (t == 0) o[decltype(pi)::value] = e[j].x;
    else if constexpr (t == 2) o[decltype(pi)::value] = e[j].y;
    else if constexpr (t == 1) o[decltype(pi)::value] = __builtin_amdgcn_alignbit(e[j].y, e[j].x, 16);
    else if constexpr (t == 3) o[decltype(pi)::value] = __builtin_amdgcn_alignbit(e[j].z, e[j].y, 16);
    else o[decltype(pi)::value] = __builtin_amdgcn_perm(e[j + 1].x, e[j].z, 0x05040100u);
  });
  put64(dst, o);
}

// 2-bit: codes [128g + 64h, +64) of one row = chunk 2g+h.
__device__ __forceinline__ void decode_i2_64(const uint8_t* slab, int r, int64_t chunk, const uint8_t* lut,
                                             uint16_t* dst) {
  const u32x4g_t v = row_chunk(slab, r, chunk);
  uint32_t o[32];
  gfor<16>([&](auto bi) __attribute__((always_inline)) {
    constexpr int j = decltype(bi)::value;
    const uint32_t b = (dword_of(v, j >> 2) >> (8 * (j & 3))) & 0xFFu;
    const u32x2g_t q = *(lq2p)(lut + kLutI2 + b * 8);
    o[2 * j] = q.x;
    o[2 * j + 1] = q.y;
  });
  put64(dst, o);
}

// 3-bit: codes [128g + 64h, +64) of one row = two 96-bit triples (24 bytes).
template <int H>
__device__ __forceinline__ void decode_i3_64(const uint8_t* slab, int r, int64_t g, const uint8_t* lut, uint16_t* dst) {
  const u32x4g_t a = row_chunk(slab, r, 3 * g + H), b = row_chunk(slab, r, 3 * g + H + 1);
  // H = 0: bytes 0..23 of the group = a.xyzw, b.xy; H = 1: bytes 24..47 = a.zw, b.xyzw
  const uint32_t w[6] = {H ? a.z : a.x, H ? a.w : a.y, H ? b.x : a.z, H ? b.y : a.w, H ? b.z : b.x, H ? b.w : b.y};
  uint32_t o[32];
  gfor<32>([&](auto pi) __attribute__((always_inline)) {
    constexpr int P = decltype(pi)::value;
    constexpr int t = P / 16, bit = 6 * (P % 16);  // triple, first bit of the 6-bit field
    const uint32_t w0 = w[3 * t], w1 = w[3 * t + 1], w2 = w[3 * t + 2];
    uint32_t f;
    if constexpr (bit + 6 <= 32) f = (w0 >> bit) & 63u;
    else if constexpr (bit < 32) f = __builtin_amdgcn_alignbit(w1, w0, bit) & 63u;
    else if constexpr (bit + 6 <= 64) f = (w1 >> (bit - 32)) & 63u;
    else if constexpr (bit < 64) f = __builtin_amdgcn_alignbit(w2, w1, bit - 32) & 63u;
    else f = (w2 >> (bit - 64)) & 63u;
    o[P] = *(lq1p)(lut + kLutI3 + f * 4);
  });
  put64(dst, o);
}

// One workgroup: row block blockIdx.x (2 slabs), tokens [m0, m0 + 32*MB), groups of split blockIdx.z.
template <int MB>
__global__ void __launch_bounds__(kThreads, 2) gemm_kernel(MatArgs a, int M, int nsplit, float* __restrict__ part) {
  constexpr int MT = 32 * MB;  // tokens per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t wt[kTileN * kPad];
  __shared__ __attribute__((aligned(16))) uint16_t xt[MT * kPad];
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

  // decode mapping: waves 0,1 take inputs [0,64) of the group, waves 2,3 inputs [64,128)
  const int dr = tid & 127, dh = tid >> 7;
  const uint8_t* dslab = dr < kSlab ? slab0 : slab1;
  const int dslab_r = dr & (kSlab - 1);
  uint16_t* drow = wt + dr * kPad + 64 * dh;

  // MFMA mapping: wave (wr, wm) computes rows 64wr..64wr+63 x tokens (MT/2)wm..
  const int wr = wave & 1, wm = wave >> 1;
  f32x4_t acc[4][MB];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[rb][mb] = f32x4_t{0, 0, 0, 0};

  auto step = [&](int g) __attribute__((always_inline)) {
    // x tile: token t, half h -> 64 bf16 (8 x 16 B)
    for (int task = tid; task < 2 * MT; task += kThreads) {
      const int t = task >> 1, h = task & 1;
      uint16_t* dst = xt + t * kPad + 64 * h;
      const bool ok = m0 + t < M;
      const uint16_t* src = a.x + (int64_t)(ok ? m0 + t : 0) * K + (int64_t)g * kGroup + 64 * h;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        u32x4g_t v = {0u, 0u, 0u, 0u};
        if (ok) v = *(gq4p)(src + 8 * q);
        *reinterpret_cast<u32x4g_t*>(dst + 8 * q) = v;
      }
    }
    __syncthreads();
    f32x4_t pr[4][MB];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) pr[rb][mb] = f32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kk = 32 * ks + 8 * (lane >> 4);
      bf16x8_t av[4], bv[MB];
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
        av[rb] = *reinterpret_cast<const bf16x8_t*>(wt + (64 * wr + 16 * rb + (lane & 15)) * kPad + kk);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        bv[mb] = *reinterpret_cast<const bf16x8_t*>(xt + ((MT / 2) * wm + 16 * mb + (lane & 15)) * kPad + kk);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          pr[rb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[rb], bv[mb], pr[rb][mb], 0, 0, 0);
    }
    // D lane l: rows 4*(l/16)+i of the 16-row block, token l%16 of the 16-token block
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t n = blk * kTileN + 64 * wr + 16 * rb + 4 * (lane >> 4) + i;
        const float s = n < a.N ? bf16_bits_to_f32(a.pscales[pscale_index(n, g, G8)]) : 0.0f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[rb][mb][i] = fmaf(s, pr[rb][mb][i], acc[rb][mb][i]);
      }
    }
    __syncthreads();
  };

  __syncthreads();  // tables ready
  if (gr == QL_GRID_T) {
    // periods of 640 inputs: the byte positions of every group are compile-time
    for (int64_t p = g_lo / 5; 5 * p < g_hi; ++p) {
      gfor<5>([&](auto ii) __attribute__((always_inline)) {
        constexpr int i = decltype(ii)::value;
        const int g = (int)(5 * p) + i;
        if (g >= g_lo && g < g_hi) {
          if (dh == 0) decode_t64<128 * i>(dslab, dslab_r, p, lut, drow);
          else decode_t64<128 * i + 64>(dslab, dslab_r, p, lut, drow);
          step(g);
        }
      });
    }
  } else if (gr == QL_GRID_I2) {
    for (int g = g_lo; g < g_hi; ++g) {
      decode_i2_64(dslab, dslab_r, 2 * g + dh, lut, drow);
      step(g);
    }
  } else {
    for (int g = g_lo; g < g_hi; ++g) {
      if (dh == 0) decode_i3_64<0>(dslab, dslab_r, g, lut, drow);
      else decode_i3_64<1>(dslab, dslab_r, g, lut, drow);
      step(g);
    }
  }

  // store: y directly, or this split's partial sums
  float* out = nsplit > 1 ? part + (int64_t)z * M * a.N : a.y;
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    const int64_t n = blk * kTileN + 64 * wr + 16 * rb + 4 * (lane >> 4);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int t = m0 + (MT / 2) * wm + 16 * mb + (lane & 15);
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
int token_blocks(int64_t M) { return M <= 32 ? 1 : (M <= 64 ? 2 : 4); }

// K splits that bring the launch to about two workgroups per CU (at least two
// groups per split); 1 when the matrix alone fills the device.
int choose_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t mt = 32 * token_blocks(M);
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
  const int mbk = token_blocks(M);
  const dim3 grid((unsigned)((a.N + kTileN - 1) / kTileN), (unsigned)((M + 32 * mbk - 1) / (32 * mbk)), (unsigned)s);
  float* part = static_cast<float*>(workspace);
  if (mbk == 1)
    hipLaunchKernelGGL(gemm_kernel<1>, grid, dim3(kThreads), 0, stream, a, M, s, part);
  else if (mbk == 2)
    hipLaunchKernelGGL(gemm_kernel<2>, grid, dim3(kThreads), 0, stream, a, M, s, part);
  else
    hipLaunchKernelGGL(gemm_kernel<4>, grid, dim3(kThreads), 0, stream, a, M, s, part);
  if (s > 1) {
    const int64_t n = (int64_t)M * a.N;
    const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3(blocks), dim3(256), 0, stream, part, a.y, n, s);
  }
  return hipGetLastError();
}

}  // namespace ql
