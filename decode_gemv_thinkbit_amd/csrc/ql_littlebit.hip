// LittleBit two-path binary factorized GEMV (batch 1) on gfx950.
//
// LittleBit digest page (seosoyoung.eiaserinnys.me/digest/littlebit-ultra-
// low-bit-quantization), section "LittleBit's structure": a linear is the sum
// of a primary and a residual path, each diag(h) U_sign diag(l) V_sign^T
// diag(g) with +-1 matrices U_sign (d_out x r), V_sign (d_in x r) and 16-bit
// scale vectors h, g, l; the product never forms W:
//   z = ((x . g) V_sign) . l,   y = (z U_sign^T) . h,   summed over the paths.
// The page's own kernel packs the signs 32 to a word and flips the sign bit of
// 16-bit inputs instead of multiplying (section "Memory, KV cache, speed").
//
// Here, three launches:
//   lb_latent_kernel  one wave per (64 latent rows, slice of inputs): for each
//                     input pair a table turns a sign byte into four sign masks
//                     that flip the bf16 scales g, and v_dot2_f32_bf16 takes
//                     (+-g_i, +-g_i+1) . (x_i, x_i+1): exact products, fp32
//                     partial sums per slice;
//   lb_reduce_kernel  z = l . (sum of the slices, in slice order), split into
//                     three bf16 terms hi + mid + lo that reproduce z to fp32
//                     accuracy;
//   lb_output_kernel  one workgroup per 64 output rows, its waves splitting the
//                     latent dimension: a table turns a sign byte into four
//                     (+-1, +-1) bf16 pairs, dotted with the three z terms
//                     (exact), fp32 sums per path, times h.
// Every product is exact; only fp32 summation rounds, in a fixed order, so the
// result is deterministic.
#include "ql_internal.hpp"
#include "ql_stream.hpp"

namespace ql {

namespace {

constexpr int kLbWaves = 4;                 // waves per workgroup
constexpr int kLbLutBytes = 256 * 16 * 16;  // 256 byte values x 16 replicas x 16 B = 64 KB

__device__ __forceinline__ uint32_t bf16_one(int bit) { return bit ? 0xBF80u : 0x3F80u; }

// dword k of byte b's entry: sign masks of elements 2k (bit 15) and 2k+1 (bit 31)
__device__ void build_sign_masks(uint8_t* lut) {
  for (int e = threadIdx.x; e < 256 * 16; e += blockDim.x) {
    const int b = e >> 4;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = ((b >> (2 * k)) & 1 ? 0x8000u : 0u) | ((b >> (2 * k + 1)) & 1 ? 0x80000000u : 0u);
    *reinterpret_cast<uint4*>(lut + 16 * e) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// dword k of byte b's entry: the bf16 pair (+-1, +-1) of elements 2k, 2k+1
__device__ void build_pm_ones(uint8_t* lut) {
  for (int e = threadIdx.x; e < 256 * 16; e += blockDim.x) {
    const int b = e >> 4;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = bf16_one((b >> (2 * k)) & 1) | (bf16_one((b >> (2 * k + 1)) & 1) << 16);
    *reinterpret_cast<uint4*>(lut + 16 * e) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// table row of byte B (0..15) of a 16-byte chunk: byte << 8 | replica offset
__device__ __forceinline__ uint32_t lut_addr(const uint4& d, int B, uint32_t lane_off) {
  return __builtin_amdgcn_perm(word_of(d, B >> 2), lane_off, 0x0C0C0000u | ((4u + (B & 3)) << 8));
}

// partial[q][row] = sum over inputs of slice q of s(row, i) * g_i * x_i
__global__ void __launch_bounds__(kLbWaves * 64) lb_latent_kernel(int32_t d_in, int32_t RP, int32_t slice_chunks,
                                                                  int32_t nslices, const uint8_t* __restrict__ v_bits,
                                                                  const uint16_t* __restrict__ g,
                                                                  const uint16_t* __restrict__ x,
                                                                  float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLbLutBytes];
  build_sign_masks(lut);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ntasks = 2 * RP / kSlab * nslices;
  const int rb = d_in / 8, nchunks = rb / kChunkBytes;
  const cu32p xp = (cu32p)x;
  const uint32_t lane_off = (uint32_t)(lane & 15) << 4;
  // persistent: the table is built once per workgroup, tasks stride over the waves
  for (int task = blockIdx.x * kLbWaves + wave; task < ntasks; task += gridDim.x * kLbWaves) {
    const int slab = task / nslices, q = task % nslices;
    const int path = slab / (RP / kSlab);
    const int c0 = q * slice_chunks, c1 = (c0 + slice_chunks < nchunks) ? c0 + slice_chunks : nchunks;
    const ChunkSrc src(v_bits + (int64_t)slab * kSlab * rb, nchunks, lane);
    const cu32p gp = (cu32p)(g + (int64_t)path * d_in);
    float acc = 0.0f;
    for (int c = c0; c < c1; ++c) {
      const uint4 d = src.load(c);
#pragma unroll 8  // (full unrolling holds 128 x and g dwords in SGPRs and spills)
      for (int B = 0; B < 16; ++B) {
        const u32x4_t e = lds_b128(lut + lut_addr(d, B, lane_off));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int P = 64 * c + 4 * B + k;  // input pair (2P, 2P+1)
          acc = dot2(gp[P] ^ e[k], xp[P], acc);
        }
      }
    }
    partial[(int64_t)q * 2 * RP + slab * kSlab + lane] = acc;
  }
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) { return f32_to_bf16_bits(f); }

// z of latent pairs, as three bf16 terms per element: zs[(path*ZP + P)*3 + t]
// holds term t of elements 2P (low half) and 2P+1 (high half).
__global__ void __launch_bounds__(256) lb_reduce_kernel(int32_t r, int32_t RP, int32_t ZP, int32_t nslices,
                                                        const float* __restrict__ partial,
                                                        const uint16_t* __restrict__ l, uint32_t* __restrict__ zs) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= 2 * ZP) return;
  const int path = t / ZP, P = t % ZP;
  uint32_t term[3] = {0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int j = 2 * P + e;
    float z = 0.0f;
    if (j < r) {
      float s = 0.0f;
#pragma unroll 16  // loads issued ahead of the in-order adds
      for (int q = 0; q < nslices; ++q) s += partial[(int64_t)q * 2 * RP + path * RP + j];
      z = s * bf16_bits_to_f32(l[path * r + j]);
    }
    const uint32_t hi = bf16_rne_bits(z);
    const float r1 = z - bf16_bits_to_f32(hi);
    const uint32_t mid = bf16_rne_bits(r1);
    const float r2 = r1 - bf16_bits_to_f32(mid);
    const uint32_t lo = bf16_rne_bits(r2);
    term[0] |= hi << (16 * e);
    term[1] |= mid << (16 * e);
    term[2] |= lo << (16 * e);
  }
#pragma unroll
  for (int k = 0; k < 3; ++k) zs[(int64_t)t * 3 + k] = term[k];
}

// y[n] = h0[n] * sum_j s0(n, j) z0_j + h1[n] * sum_j s1(n, j) z1_j.  A
// workgroup owns one 64-row slab; its four waves split the row's latent chunks
// (path 0's, then path 1's) into contiguous quarters, so every wave's z
// operands stay wave-uniform (scalar loads), and the quarters' per-path sums
// are added through LDS in wave order.
__global__ void __launch_bounds__(kLbWaves * 64) lb_output_kernel(int32_t d_out, int32_t urb, int32_t ZP,
                                                                  const uint8_t* __restrict__ u_bits,
                                                                  const uint32_t* __restrict__ zs,
                                                                  const uint16_t* __restrict__ h,
                                                                  float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLbLutBytes];
  __shared__ float part[kLbWaves][2][kSlab];
  build_pm_ones(lut);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int half_chunks = urb / 2 / kChunkBytes;  // chunks of one path's part of a row
  const int nch = 2 * half_chunks;
  const int c0 = nch * wave / kLbWaves, c1 = nch * (wave + 1) / kLbWaves;
  const uint32_t lane_off = (uint32_t)(lane & 15) << 4;
  const int nslabs = (d_out + kSlab - 1) / kSlab;
  // persistent: the table is built once per workgroup, slabs stride over the workgroups
  for (int slab = blockIdx.x; slab < nslabs; slab += gridDim.x) {
  const ChunkSrc src(u_bits + (int64_t)slab * kSlab * urb, nch, lane);
  float acc[2] = {0.0f, 0.0f};
  for (int cc = c0; cc < c1; ++cc) {
    const int p = cc >= half_chunks, c = cc - p * half_chunks;
    const cu32p zp = (cu32p)(zs + (int64_t)p * ZP * 3);
    const uint4 d = src.load(cc);
    float a = 0.0f;
#pragma unroll 4  // (full unrolling keeps 192 z dwords of a chunk in SGPRs and spills)
    for (int B = 0; B < 16; ++B) {
      const u32x4_t e = lds_b128(lut + lut_addr(d, B, lane_off));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int P = 64 * c + 4 * B + k;  // latent pair (2P, 2P+1)
        a = dot2(e[k], zp[3 * P], a);
        a = dot2(e[k], zp[3 * P + 1], a);
        a = dot2(e[k], zp[3 * P + 2], a);
      }
    }
    if (p) acc[1] += a; else acc[0] += a;
  }
  part[wave][0][lane] = acc[0];
  part[wave][1][lane] = acc[1];
  __syncthreads();
  if (wave == 0) {
    float s0 = part[0][0][lane], s1 = part[0][1][lane];
#pragma unroll
    for (int w = 1; w < kLbWaves; ++w) {
      s0 += part[w][0][lane];
      s1 += part[w][1][lane];
    }
    const int64_t n = (int64_t)slab * kSlab + lane;
    if (n < d_out) y[n] = fmaf(bf16_bits_to_f32(h[n]), s0, bf16_bits_to_f32(h[d_out + n]) * s1);
  }
  __syncthreads();  // part is rewritten by the next slab
  }
}

// ---------------------------------------------------------------- packing
// One thread per (row, 16-byte chunk) of each buffer; bit t of byte B of a row
// is element 8B + t, set for a -1.
__global__ void __launch_bounds__(256) lb_pack_v_kernel(int32_t d_in, int32_t r, int32_t RP,
                                                        const int8_t* __restrict__ v_signs, uint8_t* __restrict__ v_bits) {
  const int64_t rb = d_in / 8, nchunks = rb / kChunkBytes;
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= 2 * RP * nchunks) return;
  const int64_t row = item / nchunks, c = item % nchunks;
  const int path = (int)(row / RP), j = (int)(row % RP);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (j < r)
    for (int bit = 0; bit < 128; ++bit) {
      const int64_t i = 128 * c + bit;
      if (v_signs[((int64_t)path * d_in + i) * r + j] < 0) w[bit >> 5] |= 1u << (bit & 31);
    }
  *reinterpret_cast<uint4*>(v_bits + (row / kSlab) * kSlab * rb + c * kSlabChunkBytes + (row % kSlab) * kChunkBytes) =
      make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ void __launch_bounds__(256) lb_pack_u_kernel(int32_t d_out, int32_t r, int32_t urb,
                                                        const int8_t* __restrict__ u_signs, uint8_t* __restrict__ u_bits) {
  const int64_t nchunks = urb / kChunkBytes, half_chunks = nchunks / 2;
  const int64_t rows = (int64_t)((d_out + kSlab - 1) / kSlab) * kSlab;
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= rows * nchunks) return;
  const int64_t n = item / nchunks, c = item % nchunks;
  const int path = (int)(c / half_chunks);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (n < d_out)
    for (int bit = 0; bit < 128; ++bit) {
      const int64_t j = 128 * (c % half_chunks) + bit;
      if (j < r && u_signs[((int64_t)path * d_out + n) * r + j] < 0) w[bit >> 5] |= 1u << (bit & 31);
    }
  *reinterpret_cast<uint4*>(u_bits + (n / kSlab) * kSlab * urb + c * kSlabChunkBytes + (n % kSlab) * kChunkBytes) =
      make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

int64_t lb_latent_rows(int64_t r) { return (r + 63) / 64 * 64; }
int64_t lb_u_row_bytes(int64_t r) { return 2 * ((r + 127) / 128) * 16; }
int64_t lb_z_pairs(int64_t r) { return (r + 127) / 128 * 64; }

// inputs per slice of the latent kernel: enough (row slab, slice) tasks to
// spread over the device, at most 16 chunks (2048 inputs) per task
static int lb_slice_chunks(int64_t d_in, int64_t r) {
  const int64_t nchunks = d_in / 128, slabs = 2 * lb_latent_rows(r) / 64;
  const int64_t want = 8 * (int64_t)device_cu_count();
  int64_t s = (nchunks * slabs + want - 1) / want;
  return (int)(s < 1 ? 1 : (s > 16 ? 16 : s));
}

size_t lb_workspace_bytes(int64_t d_out, int64_t d_in, int64_t r) {
  (void)d_out;
  const int64_t sc = lb_slice_chunks(d_in, r), nslices = (d_in / 128 + sc - 1) / sc;
  return (size_t)(nslices * 2 * lb_latent_rows(r) * 4 + 2 * lb_z_pairs(r) * 3 * 4 + 256);
}

hipError_t launch_lb_pack(int64_t d_out, int64_t d_in, int64_t r, const int8_t* u_signs, const int8_t* v_signs,
                          uint8_t* u_bits, uint8_t* v_bits, hipStream_t stream) {
  const int64_t RP = lb_latent_rows(r), urb = lb_u_row_bytes(r);
  const int64_t nv = 2 * RP * (d_in / 128);
  hipLaunchKernelGGL(lb_pack_v_kernel, dim3((unsigned)((nv + 255) / 256)), dim3(256), 0, stream, (int)d_in, (int)r,
                     (int)RP, v_signs, v_bits);
  const int64_t nu = ((d_out + 63) / 64) * 64 * (urb / 16);
  hipLaunchKernelGGL(lb_pack_u_kernel, dim3((unsigned)((nu + 255) / 256)), dim3(256), 0, stream, (int)d_out, (int)r,
                     (int)urb, u_signs, u_bits);
  return hipGetLastError();
}

hipError_t launch_lb_gemv(const ql_littlebit& w, const uint16_t* x, float* y, void* ws, hipStream_t stream) {
  const int64_t r = w.rank, RP = lb_latent_rows(r), ZP = lb_z_pairs(r);
  const int sc = lb_slice_chunks(w.d_in, r);
  const int nslices = (int)((w.d_in / 128 + sc - 1) / sc);
  float* partial = static_cast<float*>(ws);
  uint32_t* zs = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) +
                                             ((size_t)nslices * 2 * RP * 4 + 255) / 256 * 256);
  const int64_t tasks = 2 * RP / 64 * nslices, slots = 2 * (int64_t)device_cu_count();
  const int64_t wg_lat = (tasks + kLbWaves - 1) / kLbWaves;
  hipLaunchKernelGGL(lb_latent_kernel, dim3((unsigned)(wg_lat < slots ? wg_lat : slots)), dim3(kLbWaves * 64), 0,
                     stream, w.d_in, (int)RP, sc, nslices, static_cast<const uint8_t*>(w.v_bits), w.g, x, partial);
  hipLaunchKernelGGL(lb_reduce_kernel, dim3((unsigned)((2 * ZP + 255) / 256)), dim3(256), 0, stream, (int)r, (int)RP,
                     (int)ZP, nslices, partial, w.l, zs);
  const int64_t slabs = (w.d_out + 63) / 64;
  hipLaunchKernelGGL(lb_output_kernel, dim3((unsigned)(slabs < slots ? slabs : slots)), dim3(kLbWaves * 64), 0,
                     stream, w.d_out, (int)lb_u_row_bytes(r), (int)ZP, static_cast<const uint8_t*>(w.u_bits), zs, w.h,
                     y);
  return hipGetLastError();
}

}  // namespace ql
