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
// Here, two launches:
//   lb_latent_kernel  one wave per (64 latent rows, slice of inputs): for each
//                     input pair a table turns a sign byte into four sign masks
//                     that flip the bf16 scales g, and v_dot2_f32_bf16 takes
//                     (+-g_i, +-g_i+1) . (x_i, x_i+1): exact products, fp32
//                     partial sums per slice.  The wave that completes a slab's
//                     last slice (a counter per slab) forms its z = l . (sum of
//                     the slices, in slice order), split into three bf16 terms
//                     hi + mid + lo that reproduce z to fp32 accuracy;
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

// The tables: 256 byte values x 16 replicas of a 16-byte entry (byte b's replica q at
// b * 256 + q * 16; a lane reads replica lane % 16, so the 16 lanes a read serves at once
// hit distinct banks).  Built by 256 threads, thread b computing byte b's entry once and
// writing its replicas in the order (b + i) % 16, so that the 16 lanes of one write also
// hit distinct banks.
template <typename F>
__device__ __forceinline__ void build_replicated(uint8_t* lut, F entry_dword) {
  static_assert(kLbWaves * 64 == 256, "one thread per byte value");
  const int b = threadIdx.x;
  const uint4 v = make_uint4(entry_dword(b, 0), entry_dword(b, 1), entry_dword(b, 2), entry_dword(b, 3));
#pragma unroll
  for (int i = 0; i < 16; ++i) *reinterpret_cast<uint4*>(lut + 256 * b + 16 * ((b + i) & 15)) = v;
}

// dword k of byte b's entry: sign masks of elements 2k (bit 15) and 2k+1 (bit 31)
__device__ void build_sign_masks(uint8_t* lut) {
  build_replicated(lut, [](int b, int k) {
    return ((b >> (2 * k)) & 1 ? 0x8000u : 0u) | ((b >> (2 * k + 1)) & 1 ? 0x80000000u : 0u);
  });
}

// dword k of byte b's entry: the bf16 pair (+-1, +-1) of elements 2k, 2k+1
__device__ void build_pm_ones(uint8_t* lut) {
  build_replicated(lut, [](int b, int k) {
    return bf16_one((b >> (2 * k)) & 1) | (bf16_one((b >> (2 * k + 1)) & 1) << 16);
  });
}

// table row of byte B (0..15) of a 16-byte chunk: byte << 8 | replica offset
__device__ __forceinline__ uint32_t lut_addr(const uint4& d, int B, uint32_t lane_off) {
  return __builtin_amdgcn_perm(word_of(d, B >> 2), lane_off, 0x0C0C0000u | ((4u + (B & 3)) << 8));
}

// partial[q][row] = sum over inputs of slice q of s(row, i) * g_i * x_i
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) { return f32_to_bf16_bits(f); }

// z of the 64 latent rows of slab `slab` (lane = row) from the slab's input sum
// (ignored at rows past r), as three bf16 terms per element: zs[(path*ZP + P)*3 + t]
// holds term t of elements 2P (low half) and 2P+1 (high half).  Rows at or past r have
// z = 0; the path's last slab also zeroes the pairs between its padded row count and ZP.
__device__ __forceinline__ void lb_z_store(int slab, int lane, int r, int RP, int ZP, float sum,
                                           const uint16_t* __restrict__ l, uint32_t* __restrict__ zs) {
  const int spp = RP / kSlab;  // slabs per path
  const int path = slab / spp, j = (slab % spp) * kSlab + lane;
  const float z = j < r ? sum * bf16_bits_to_f32(l[path * r + j]) : 0.0f;
  const uint32_t hi = bf16_rne_bits(z);
  const float r1 = z - bf16_bits_to_f32(hi);
  const uint32_t mid = bf16_rne_bits(r1);
  const float r2 = r1 - bf16_bits_to_f32(mid);
  const uint32_t lo = bf16_rne_bits(r2);
  // the odd lane's halves join the even lane's
  const uint32_t ohi = __shfl_down(hi, 1, 64), omid = __shfl_down(mid, 1, 64), olo = __shfl_down(lo, 1, 64);
  if ((lane & 1) == 0) {
    uint32_t* d = zs + ((int64_t)path * ZP + (j >> 1)) * 3;
    d[0] = hi | (ohi << 16);
    d[1] = mid | (omid << 16);
    d[2] = lo | (olo << 16);
  }
  if (slab % spp == spp - 1)
    for (int P = RP / 2 + lane; P < ZP; P += 64)
      for (int t = 0; t < 3; ++t) zs[((int64_t)path * ZP + P) * 3 + t] = 0u;
}

// The split form's slab sum: the slices' partial sums in slice order, 32 loads in flight
// (a slice index past the last rereads the last slice and is not added).
__device__ __forceinline__ float lb_slice_sum(int slab, int lane, int RP, int nslices,
                                              const float* __restrict__ partial) {
  const float* p = partial + (int64_t)slab * kSlab + lane;  // slice q at p + q * 2 * RP
  float sum = 0.0f;
  for (int q0 = 0; q0 < nslices; q0 += 32) {
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int q = q0 + i < nslices ? q0 + i : nslices - 1;
      v[i] = __hip_atomic_load(p + (int64_t)q * 2 * RP, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (q0 + i < nslices) sum += v[i];
  }
  return sum;
}

typedef const __attribute__((address_space(1))) uint32_t* lb_gu32p;

// The inner loops read only LDS: the scales g, the activations x and the z terms a
// chunk needs are staged in a per-wave LDS buffer by vector loads issued one chunk
// ahead.  (Wave-uniform scalar loads inside these loops would share the LDS reads'
// completion counter and, returning out of order, force a full drain before every
// table read.)  A wave writes and then reads its own buffer, and LDS executes one
// wave's operations in order, so no barrier separates the two.
__global__ void __launch_bounds__(kLbWaves * 64) lb_latent_kernel(int32_t d_in, int32_t r, int32_t RP, int32_t ZP,
                                                                  int32_t slice_chunks, int32_t nslices,
                                                                  const uint8_t* __restrict__ v_bits,
                                                                  const uint16_t* __restrict__ g,
                                                                  const uint16_t* __restrict__ l,
                                                                  const uint16_t* __restrict__ x,
                                                                  float* __restrict__ partial,
                                                                  uint32_t* __restrict__ counters,
                                                                  uint32_t* __restrict__ zs) {
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLbLutBytes];
  // per wave, two chunk buffers of 64 input pairs: (g pair, x pair) dwords
  __shared__ __attribute__((aligned(16))) uint2 gxs[kLbWaves][2][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int ntasks = 2 * RP / kSlab * nslices, stride = gridDim.x * kLbWaves;
  const int rb = d_in / 8, nchunks = rb / kChunkBytes;
  const uint32_t lane_off = (uint32_t)(lane & 15) << 4;
  const lb_gu32p xw = (lb_gu32p)x;
  // chunk c of task t: its sign bits (lane = latent row) and the (g, x) dwords of its
  // input pair `lane`
  uint4 d = make_uint4(0u, 0u, 0u, 0u);
  uint32_t gv = 0u, xv = 0u;
  auto issue = [&](int t, int c) {
    const int slab = t / nslices, path = slab / (RP / kSlab);
    d = ChunkSrc(v_bits + (int64_t)slab * kSlab * rb, nchunks, lane).load(c);
    gv = ((lb_gu32p)(g + (int64_t)path * d_in))[64 * c + lane];
    xv = xw[64 * c + lane];
  };
  int task = blockIdx.x * kLbWaves + wave;
  if (task < ntasks) issue(task, (task % nslices) * slice_chunks);  // in flight during the table build
  build_sign_masks(lut);
  __syncthreads();
  int buf = 0;
  // persistent: the table is built once per workgroup, tasks stride over the waves
  for (; task < ntasks; task += stride) {
    const int slab = task / nslices, q = task % nslices;
    const int c0 = q * slice_chunks, c1 = (c0 + slice_chunks < nchunks) ? c0 + slice_chunks : nchunks;
    float acc = 0.0f;
    for (int c = c0; c < c1; ++c, buf ^= 1) {
      gxs[wave][buf][lane] = make_uint2(gv, xv);
      const uint4 dc = d;
      if (c + 1 < c1) issue(task, c + 1);
      else if (task + stride < ntasks) issue(task + stride, ((task + stride) % nslices) * slice_chunks);
      const uint8_t* gb = reinterpret_cast<const uint8_t*>(&gxs[wave][buf][0]);
      // step B reads the sign masks of byte B and the (g, x) of input pairs 4B .. 4B+3,
      // three steps ahead of their use (a ring of four operand sets)
      u32x4_t E[4], P0[4], P1[4];
#pragma unroll
      for (int B = 0; B < 3; ++B) {
        E[B] = lds_b128(lut + lut_addr(dc, B, lane_off));
        P0[B] = lds_b128(gb + 32 * B);
        P1[B] = lds_b128(gb + 32 * B + 16);
      }
#pragma unroll
      for (int B = 0; B < 16; ++B) {
        if (B + 3 < 16) {
          E[(B + 3) & 3] = lds_b128(lut + lut_addr(dc, B + 3, lane_off));
          P0[(B + 3) & 3] = lds_b128(gb + 32 * (B + 3));
          P1[(B + 3) & 3] = lds_b128(gb + 32 * (B + 3) + 16);
        }
        const u32x4_t e = E[B & 3], p0 = P0[B & 3], p1 = P1[B & 3];
        acc = dot2(p0[0] ^ e[0], p0[1], acc);
        acc = dot2(p0[2] ^ e[1], p0[3], acc);
        acc = dot2(p1[0] ^ e[2], p1[1], acc);
        acc = dot2(p1[2] ^ e[3], p1[3], acc);
      }
    }
    // partial sums travel at device scope (the XCDs' L2 caches are not coherent with
    // each other); the counter increment waits for this wave's stores, and the wave
    // that completes the slab reads them only after its increment has returned
    __hip_atomic_store(partial + (int64_t)q * 2 * RP + slab * kSlab + lane, acc, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (nslices > 1) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      uint32_t old = 0;
      if (lane == 0) old = __hip_atomic_fetch_add(counters + slab * 32, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old = __builtin_amdgcn_readfirstlane(old);
      if (old != (uint32_t)nslices - 1u) continue;
      asm volatile("" ::: "memory");
      if (lane == 0) __hip_atomic_store(counters + slab * 32, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    lb_z_store(slab, lane, r, RP, ZP, lb_slice_sum(slab, lane, RP, nslices, partial), l, zs);
  }
}

// y[n] = h0[n] * sum_j s0(n, j) z0_j + h1[n] * sum_j s1(n, j) z1_j.  A
// workgroup owns one 64-row slab; its four waves split the row's latent chunks
// (path 0's, then path 1's) into contiguous quarters, and the quarters' per-path
// sums are added through LDS in wave order.  A chunk's z terms (64 latent pairs x 3
// dwords) are staged in the wave's LDS buffer and read back as broadcasts.
__global__ void __launch_bounds__(kLbWaves * 64) lb_output_kernel(int32_t d_out, int32_t urb, int32_t ZP,
                                                                  const uint8_t* __restrict__ u_bits,
                                                                  const uint32_t* __restrict__ zs,
                                                                  const uint16_t* __restrict__ h,
                                                                  float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLbLutBytes];
  __shared__ float part[kLbWaves][2][kSlab];
  __shared__ __attribute__((aligned(16))) uint32_t zst[kLbWaves][2][kSlab * 3];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int half_chunks = urb / 2 / kChunkBytes;  // chunks of one path's part of a row
  const int nch = 2 * half_chunks;
  const int c0 = nch * wave / kLbWaves, c1 = nch * (wave + 1) / kLbWaves;
  const uint32_t lane_off = (uint32_t)(lane & 15) << 4;
  const int nslabs = (d_out + kSlab - 1) / kSlab;
  // chunk cc of slab s: its sign bits (lane = output row) and the three z dwords of latent
  // pair `lane` of the chunk
  uint4 d = make_uint4(0u, 0u, 0u, 0u);
  uint32_t z0 = 0u, z1 = 0u, z2 = 0u;
  auto issue = [&](int s, int cc) {
    const int p = cc >= half_chunks, c = cc - p * half_chunks;
    d = ChunkSrc(u_bits + (int64_t)s * kSlab * urb, nch, lane).load(cc);
    const lb_gu32p zp = (lb_gu32p)(zs + ((int64_t)p * ZP + 64 * c + lane) * 3);
    z0 = zp[0];
    z1 = zp[1];
    z2 = zp[2];
  };
  if (c0 < c1) issue(blockIdx.x, c0);  // in flight during the table build
  build_pm_ones(lut);
  __syncthreads();
  int buf = 0;
  // persistent: the table is built once per workgroup, slabs stride over the workgroups
  for (int slab = blockIdx.x; slab < nslabs; slab += gridDim.x) {
    float acc[2] = {0.0f, 0.0f};
    for (int cc = c0; cc < c1; ++cc, buf ^= 1) {
      const int p = cc >= half_chunks;
      uint32_t* zb = &zst[wave][buf][0];
      zb[3 * lane] = z0;
      zb[3 * lane + 1] = z1;
      zb[3 * lane + 2] = z2;
      const uint4 dc = d;
      if (cc + 1 < c1) issue(slab, cc + 1);
      else if (slab + (int)gridDim.x < nslabs) issue(slab + gridDim.x, c0);
      const uint8_t* zr = reinterpret_cast<const uint8_t*>(zb);
      float a = 0.0f;
      // step B reads the (+-1, +-1) pairs of byte B and the three terms of latent pairs
      // 4B .. 4B+3 (twelve dwords), two steps ahead of their use (a ring of three sets)
      u32x4_t E[3], W0[3], W1[3], W2[3];
#pragma unroll
      for (int B = 0; B < 2; ++B) {
        E[B] = lds_b128(lut + lut_addr(dc, B, lane_off));
        W0[B] = lds_b128(zr + 48 * B);
        W1[B] = lds_b128(zr + 48 * B + 16);
        W2[B] = lds_b128(zr + 48 * B + 32);
      }
#pragma unroll
      for (int B = 0; B < 16; ++B) {
        if (B + 2 < 16) {
          E[(B + 2) % 3] = lds_b128(lut + lut_addr(dc, B + 2, lane_off));
          W0[(B + 2) % 3] = lds_b128(zr + 48 * (B + 2));
          W1[(B + 2) % 3] = lds_b128(zr + 48 * (B + 2) + 16);
          W2[(B + 2) % 3] = lds_b128(zr + 48 * (B + 2) + 32);
        }
        const u32x4_t e = E[B % 3], w0 = W0[B % 3], w1 = W1[B % 3], w2 = W2[B % 3];
        a = dot2(e[0], w0[0], a);
        a = dot2(e[0], w0[1], a);
        a = dot2(e[0], w0[2], a);
        a = dot2(e[1], w0[3], a);
        a = dot2(e[1], w1[0], a);
        a = dot2(e[1], w1[1], a);
        a = dot2(e[2], w1[2], a);
        a = dot2(e[2], w1[3], a);
        a = dot2(e[2], w2[0], a);
        a = dot2(e[3], w2[1], a);
        a = dot2(e[3], w2[2], a);
        a = dot2(e[3], w2[3], a);
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
// spread over the device, at most 32 slices per slab (the slab's last wave reads
// every slice's partial sums at device scope: 64 slices of one chunk each ran
// 11.9 us against 11.2 us for 32 of two on 28672 x 8192 at 0.1 BPW, 16.0 against
// 13.8 us at 0.3 BPW), at most 16 chunks (2048 inputs) per task
static int lb_slice_chunks(int64_t d_in, int64_t r) {
  const int64_t nchunks = d_in / 128, slabs = 2 * lb_latent_rows(r) / 64;
  const int64_t want = 8 * (int64_t)device_cu_count();
  int64_t s = (nchunks * slabs + want - 1) / want;
  if (s < (nchunks + 31) / 32) s = (nchunks + 31) / 32;
  return (int)(s < 1 ? 1 : (s > 16 ? 16 : s));
}

// workspace: per-slab counters (one 128-byte line each), then the slices' partial
// sums, then the z terms
static size_t lb_counter_bytes(int64_t r) { return (size_t)(2 * lb_latent_rows(r) / 64) * 128; }
static size_t lb_partial_bytes(int64_t d_in, int64_t r) {
  const int64_t sc = lb_slice_chunks(d_in, r), nslices = (d_in / 128 + sc - 1) / sc;
  return ((size_t)nslices * 2 * lb_latent_rows(r) * 4 + 255) / 256 * 256;
}

size_t lb_workspace_bytes(int64_t d_out, int64_t d_in, int64_t r) {
  (void)d_out;
  return lb_counter_bytes(r) + lb_partial_bytes(d_in, r) + (size_t)(2 * lb_z_pairs(r) * 3 * 4);
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
  uint32_t* counters = static_cast<uint32_t*>(ws);
  float* partial = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + lb_counter_bytes(r));
  uint32_t* zs = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + lb_counter_bytes(r) +
                                             lb_partial_bytes(w.d_in, r));
  const int64_t tasks = 2 * RP / 64 * nslices, slots = 2 * (int64_t)device_cu_count();
  const int64_t wg_lat = (tasks + kLbWaves - 1) / kLbWaves;
  hipLaunchKernelGGL(lb_latent_kernel, dim3((unsigned)(wg_lat < slots ? wg_lat : slots)), dim3(kLbWaves * 64), 0,
                     stream, w.d_in, (int)r, (int)RP, (int)ZP, sc, nslices, static_cast<const uint8_t*>(w.v_bits),
                     w.g, w.l, x, partial, counters, zs);
  const int64_t slabs = (w.d_out + 63) / 64;
  hipLaunchKernelGGL(lb_output_kernel, dim3((unsigned)(slabs < slots ? slabs : slots)), dim3(kLbWaves * 64), 0,
                     stream, w.d_out, (int)lb_u_row_bytes(r), (int)ZP, static_cast<const uint8_t*>(w.u_bits), zs, w.h,
                     y);
  return hipGetLastError();
}

}  // namespace ql
