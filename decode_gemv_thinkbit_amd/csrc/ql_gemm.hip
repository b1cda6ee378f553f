// Batched GEMM over ThinkBit-packed weights: LDS-staged bf16 code tiles + MFMA.
//
// For M tokens the product is a dense contraction, so it runs on the matrix
// cores.  Per 128-deep step (one scale group) a 64-row slab of codes is decoded
// into LDS as bf16 integers (exact), the activation tile is staged beside it,
// and v_mfma_f32_16x16x32_bf16 accumulates the group's partial products in
// fp32; the group scale (ThinkBit summary page, onedev.kr/papers/1416, section
// "How it works": w = c * s, one scale per 128 inputs) multiplies that partial
// once.  Computing on dequantized bf16 values reproduces the native low-bit
// result (k-quant calibration page, sotaaz.com/post/quantized-model-less-sure,
// section "Not just any noise"); here the scale is kept out of the bf16 operand,
// so every product is exact.
#include "ql_internal.hpp"

namespace ql {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kBM = 64;          // tokens per tile
constexpr int kRowPad = 136;     // bf16 per LDS row (128 + 8: rows land on different banks)

// Decode codes [k0, k0+32) of row r of a slab into 32 bf16 code bits.
__device__ __forceinline__ void decode32(const uint8_t* __restrict__ slab, int r, int gr, int64_t k0, int64_t K,
                                         uint16_t (&out)[32]) {
  auto rowbyte = [&](int64_t jj) -> uint32_t {
    return slab[(jj >> 4) * kSlabChunkBytes + r * kChunkBytes + (jj & 15)];
  };
  if (gr == QL_GRID_T) {
    int64_t j = k0 / 5;
    int i = (int)(k0 % 5);
    uint32_t b = tern_to_input_order(rowbyte(j), j);
    for (int t = 0; t < i; ++t) b /= 3;
    for (int q = 0; q < 32; ++q) {
      out[q] = code_bf16((int)(b % 3) - 1);
      b /= 3;
      if (++i == 5) {
        i = 0;
        ++j;
        b = (5 * j < K) ? tern_to_input_order(rowbyte(j), j) : 121u;
      }
    }
  } else if (gr == QL_GRID_I2) {
    const int64_t jj = k0 >> 2;  // 8 bytes, 8-byte aligned within one chunk
    const uint2 v = *reinterpret_cast<const uint2*>(slab + (jj >> 4) * kSlabChunkBytes + r * kChunkBytes + (jj & 15));
#pragma unroll
    for (int q = 0; q < 16; ++q) out[q] = code_bf16((int)((v.x >> (2 * q)) & 3u) - 2);
#pragma unroll
    for (int q = 0; q < 16; ++q) out[16 + q] = code_bf16((int)((v.y >> (2 * q)) & 3u) - 2);
  } else {
    const int64_t jj = (3 * k0) >> 3;  // 12 bytes, 4-byte aligned
    uint32_t w[3];
#pragma unroll
    for (int d = 0; d < 3; ++d) {
      const int64_t b = jj + 4 * d;
      w[d] = *reinterpret_cast<const uint32_t*>(slab + (b >> 4) * kSlabChunkBytes + r * kChunkBytes + (b & 15));
    }
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      const int bit = 3 * q;
      uint32_t u;
      if (bit + 3 <= 32)
        u = w[0] >> bit;
      else if (bit < 32)
        u = (w[0] >> bit) | (w[1] << (32 - bit));
      else if (bit + 3 <= 64)
        u = w[1] >> (bit - 32);
      else if (bit < 64)
        u = (w[1] >> (bit - 32)) | (w[2] << (64 - bit));
      else
        u = w[2] >> (bit - 64);
      out[q] = code_bf16((int)(u & 7u) - 4);
    }
  }
}

// grid: (ceil(M/64), slabs).  256 threads: wave w owns rows 16w..16w+15 of the slab.
__global__ void __launch_bounds__(256) gemm_kernel(MatArgs a, int M) {
  __shared__ __attribute__((aligned(16))) uint16_t ws[kSlab * kRowPad];
  __shared__ __attribute__((aligned(16))) uint16_t xs[kBM * kRowPad];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t slab = blockIdx.y;
  const int m0 = blockIdx.x * kBM;
  const int K = a.K, G = K / kGroup, G8 = (G + 7) / 8;
  int gr;
  const int64_t off = slab_offset(slab, K, a.grid, a.blk_grid, a.blk_off, &gr);
  const uint8_t* sp = a.packed + off;
  const uint16_t* ss = a.pscales + slab * (int64_t)G8 * kSlab * 8;
  f32x4_t acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) acc[mb] = f32x4_t{0, 0, 0, 0};
  const int dr = tid & 63, dq = tid >> 6;  // decode: row, 32-code quarter
  for (int g = 0; g < G; ++g) {
    // stage W codes (bf16) and the x tile
    uint16_t codes[32];
    decode32(sp, dr, gr, (int64_t)g * kGroup + 32 * dq, K, codes);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint4 v;
      v.x = codes[8 * q + 0] | ((uint32_t)codes[8 * q + 1] << 16);
      v.y = codes[8 * q + 2] | ((uint32_t)codes[8 * q + 3] << 16);
      v.z = codes[8 * q + 4] | ((uint32_t)codes[8 * q + 5] << 16);
      v.w = codes[8 * q + 6] | ((uint32_t)codes[8 * q + 7] << 16);
      *reinterpret_cast<uint4*>(&ws[dr * kRowPad + 32 * dq + 8 * q]) = v;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q;  // 1024 uint4 = 64 tokens x 16
      const int tm = e >> 4, kk = (e & 15) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m0 + tm < M) v = *reinterpret_cast<const uint4*>(a.x + (int64_t)(m0 + tm) * K + (int64_t)g * kGroup + kk);
      *reinterpret_cast<uint4*>(&xs[tm * kRowPad + kk]) = v;
    }
    __syncthreads();
    f32x4_t part[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) part[mb] = f32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kk = 32 * ks + 8 * (lane >> 4);
      const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(&ws[(16 * wave + (lane & 15)) * kRowPad + kk]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(&xs[(16 * mb + (lane & 15)) * kRowPad + kk]);
        part[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, part[mb], 0, 0, 0);
      }
    }
    // D lane l: rows 4*(l/16)+r of this wave's 16, token l%16 of the block
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rr = 16 * wave + 4 * (lane >> 4) + r;
      s[r] = bf16_bits_to_f32(ss[((g >> 3) * kSlab + rr) * 8 + (g & 7)]);
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mb][r] = fmaf(s[r], part[mb][r], acc[mb][r]);
    __syncthreads();
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int tm = m0 + 16 * mb + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t n = slab * kSlab + 16 * wave + 4 * (lane >> 4) + r;
      if (tm < M && n < a.N) a.y[(int64_t)tm * a.N + n] = acc[mb][r];
    }
  }
}

size_t gemm_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm(const MatArgs& a, int M, void*, size_t, hipStream_t stream) {
  const int64_t nslabs = ((int64_t)a.N + kSlab - 1) / kSlab;
  dim3 grid((unsigned)((M + kBM - 1) / kBM), (unsigned)nslabs);
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(256), 0, stream, a, M);
  return hipGetLastError();
}

}  // namespace ql
