// Decode-time GEMV (1 <= M <= 8) over ThinkBit-packed weights on gfx950.
//
// The per-token weight stream is the bandwidth-bound step of decoding
// (ThinkBit summary page, onedev.kr/papers/1416, section "What it is"); the
// codes are read at 1.6 / 2 / 3 bits instead of 4-bit containers (same page,
// section "Premises & limits").  w = c * s with one bf16 scale per 128 inputs
// (section "How it works").
//
// Mapping: one wave owns a 64-row slab, lane r = row r.  The slab layout makes
// each 16-byte-per-lane load one contiguous 1 KB request.  Every lane walks the
// same input range, so activations are wave-uniform: they come through scalar
// loads into SGPRs and feed v_dot2_f32_bf16 as its second operand; no LDS or
// VGPR traffic is spent on x.  Codes are turned into exact bf16 code pairs by
// per-lane LDS lookup tables:
//   ternary: byte -> five codes (three bf16 pairs, 16-byte entry, 16 replicas
//            so a ds_read_b128 by 16 lanes touches distinct banks); the row
//            address is built by one v_perm (byte << 8 | replica offset);
//   2-bit:   byte -> four codes (two pairs);
//   3-bit:   6-bit field (two adjacent codes) -> one pair.
// Each product c * x is exact in fp32; sums are fp32 per 128-input group and
// the group scale is applied once per group.  Inputs are processed in
// "periods" of 640 (= 8 ternary chunks of 80 trits = 5 groups) so that every
// group boundary inside a ternary chunk is a compile-time position.
#include <utility>

#include "ql_internal.hpp"

namespace ql {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef const __attribute__((address_space(4))) uint32_t* cu32p;  // scalar-loaded x

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------- LDS tables
constexpr int kTLut = 0;                    // 243 rows x 256 B (16 replicas x 16 B)
constexpr int kI2Lut = 243 * 256;           // 256 rows x 32 B (4 replicas x 8 B)
constexpr int kI3Lut = kI2Lut + 256 * 32;   // 64 entries x 4 B
constexpr int kLutBytes = kI3Lut + 64 * 4;  // 70656

__device__ void build_luts(uint8_t* smem) {
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
    q.w = 0;
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

// ---------------------------------------------------------------- activations
// x dword i (two bf16) relative to the period base; the guarded form is used
// in the last, partial period where the trits past K are padding (c = 0) and
// the matching x must read as 0 without touching memory past x.
template <bool GUARD>
__device__ __forceinline__ uint32_t xdw(cu32p xb, int i, int kleft) {
  if constexpr (!GUARD) {
    return xb[i];
  } else {
    const int last = (kleft >> 1) - 1;
    const uint32_t v = xb[i < last ? i : last];
    return (2 * i < kleft) ? v : 0u;
  }
}

// (x_k, x_{k+1}) as a bf16 pair; odd k is re-aligned on the scalar unit.
template <int K0, bool GUARD>
__device__ __forceinline__ uint32_t xpair(cu32p xb, int kleft) {
  if constexpr ((K0 & 1) == 0) {
    return xdw<GUARD>(xb, K0 >> 1, kleft);
  } else {
    const uint32_t lo = xdw<GUARD>(xb, (K0 - 1) >> 1, kleft);
    const uint32_t hi = xdw<GUARD>(xb, (K0 + 1) >> 1, kleft);
    return (uint32_t)((((uint64_t)hi << 32) | lo) >> 16);
  }
}

// ---------------------------------------------------------------- ternary
// code pair a = (c_K0, c_K0+1) against x; split when a group boundary falls
// between the two codes.
template <int M, int K0, bool GUARD>
__device__ __forceinline__ void t_pair(uint32_t a, const cu32p (&xb)[M], int kleft, float (&acc)[M][5]) {
  constexpr int g0 = K0 / 128, g1 = (K0 + 1) / 128;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint32_t xp = xpair<K0, GUARD>(xb[m], kleft);
    if constexpr (g0 == g1) {
      acc[m][g0] = dot2(a, xp, acc[m][g0]);
    } else {
      acc[m][g0] = dot2(a, xp & 0x0000FFFFu, acc[m][g0]);
      acc[m][g1] = dot2(a, xp & 0xFFFF0000u, acc[m][g1]);
    }
  }
}

// a = (c_K0, 0): the fifth trit of a byte.  Only x_K0 is read (into the low
// half); the high half is zeroed so nothing past the period is touched.
template <int M, int K0, bool GUARD>
__device__ __forceinline__ void t_single(uint32_t a, const cu32p (&xb)[M], int kleft, float (&acc)[M][5]) {
  constexpr int g0 = K0 / 128;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint32_t xp = (K0 & 1) ? (xdw<GUARD>(xb[m], K0 >> 1, kleft) >> 16)
                                 : (xdw<GUARD>(xb[m], K0 >> 1, kleft) & 0xFFFFu);
    acc[m][g0] = dot2(a, xp, acc[m][g0]);
  }
}

template <int M, int CH, int J, bool GUARD>
__device__ __forceinline__ void t_byte(uint32_t wj, const uint8_t* lut, uint32_t lane_off, const cu32p (&xb)[M],
                                       int kleft, float (&acc)[M][5]) {
  // address = (byte J&3 of wj) << 8 | lane_off, in one v_perm
  const uint32_t addr = __builtin_amdgcn_perm(wj, lane_off, 0x0C0C0000u | ((4u + (J & 3)) << 8));
  const uint4 e = *reinterpret_cast<const uint4*>(lut + kTLut + addr);
  constexpr int k0 = CH * 80 + 5 * J;
  t_pair<M, k0, GUARD>(e.x, xb, kleft, acc);
  t_pair<M, k0 + 2, GUARD>(e.y, xb, kleft, acc);
  t_single<M, k0 + 4, GUARD>(e.z, xb, kleft, acc);
}

template <int M, int CH, bool GUARD, int... J>
__device__ __forceinline__ void t_chunk(const uint4 d, const uint8_t* lut, uint32_t lane_off, const cu32p (&xb)[M],
                                        int kleft, float (&acc)[M][5], std::integer_sequence<int, J...>) {
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
  (t_byte<M, CH, J, GUARD>(w[J >> 2], lut, lane_off, xb, kleft, acc), ...);
}

template <int M, int CH, bool GUARD>
__device__ __forceinline__ void t_chunk_if(const uint4 d, int nch, const uint8_t* lut, uint32_t lane_off,
                                           const cu32p (&xb)[M], int kleft, float (&acc)[M][5]) {
  if (GUARD && CH >= nch) return;
  t_chunk<M, CH, GUARD>(d, lut, lane_off, xb, kleft, acc, std::make_integer_sequence<int, 16>{});
}

template <int M, bool GUARD, int... CH>
__device__ __forceinline__ void t_period(const uint4 (&d)[8], int nch, const uint8_t* lut, uint32_t lane_off,
                                         const cu32p (&xb)[M], int kleft, float (&acc)[M][5],
                                         std::integer_sequence<int, CH...>) {
  (t_chunk_if<M, CH, GUARD>(d[CH], nch, lut, lane_off, xb, kleft, acc), ...);
}

// ---------------------------------------------------------------- 2-bit
template <int M, int K0, int J>
__device__ __forceinline__ void i2_byte(uint32_t wj, const uint8_t* lut, uint32_t lane_off, const cu32p (&xb)[M],
                                        float (&acc)[M]) {
  const uint32_t b = (wj >> (8 * (J & 3))) & 0xFFu;
  const uint2 e = *reinterpret_cast<const uint2*>(lut + kI2Lut + ((b << 5) | lane_off));
  constexpr int k = K0 + 4 * J;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    acc[m] = dot2(e.x, xpair<k, false>(xb[m], 0), acc[m]);
    acc[m] = dot2(e.y, xpair<k + 2, false>(xb[m], 0), acc[m]);
  }
}

template <int M, int K0, int... J>
__device__ __forceinline__ void i2_chunk(const uint4 d, const uint8_t* lut, uint32_t lane_off, const cu32p (&xb)[M],
                                         float (&acc)[M], std::integer_sequence<int, J...>) {
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
  (i2_byte<M, K0, J>(w[J >> 2], lut, lane_off, xb, acc), ...);
}

// ---------------------------------------------------------------- 3-bit
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

template <int M, int K0, int P>
__device__ __forceinline__ void i3_pair(uint32_t w0, uint32_t w1, uint32_t w2, const uint8_t* lut,
                                        const cu32p (&xb)[M], float (&acc)[M]) {
  const uint32_t a = *reinterpret_cast<const uint32_t*>(lut + kI3Lut + i3_field_x4<P>(w0, w1, w2));
  constexpr int k = K0 + 2 * P;
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = dot2(a, xpair<k, false>(xb[m], 0), acc[m]);
}

template <int M, int K0, int... P>
__device__ __forceinline__ void i3_triple(uint32_t w0, uint32_t w1, uint32_t w2, const uint8_t* lut,
                                          const cu32p (&xb)[M], float (&acc)[M], std::integer_sequence<int, P...>) {
  (i3_pair<M, K0, P>(w0, w1, w2, lut, xb, acc), ...);
}

// ---------------------------------------------------------------- per-slab drivers
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// streamed once: non-temporal 128-bit load
__device__ __forceinline__ uint4 ld_chunk(const uint8_t* __restrict__ p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float ld_scale(const uint16_t* __restrict__ ss, int g, int lane) {
  return bf16_bits_to_f32(ss[((g >> 3) * kSlab + lane) * 8 + (g & 7)]);
}

template <int M>
struct SlabCtx {
  const uint8_t* codes;      // slab base + lane * 16
  const uint16_t* scales;    // slab's scale block
  const uint16_t* x;         // x row 0
  int K, G, Mact, lane;
  const uint8_t* lut;
};

template <int M>
__device__ __forceinline__ void set_xb(cu32p (&xb)[M], const SlabCtx<M>& c, int kbase) {
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int mm = m < c.Mact ? m : c.Mact - 1;
    xb[m] = (cu32p)(c.x + (int64_t)mm * c.K + kbase);
  }
}

template <int M>
__device__ void run_t(const SlabCtx<M>& c, int p0, int p1, float (&y)[M]) {
  const int nchunks = (c.K + 79) / 80;
  const uint32_t lane_off = (uint32_t)(c.lane & 15) << 4;
  uint4 cur[8], nxt[8];
  auto load = [&](uint4(&d)[8], int p) {
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
      const int cc = 8 * p + ch;
      d[ch] = cc < nchunks ? ld_chunk(c.codes + (int64_t)cc * kSlabChunkBytes) : make_uint4(0, 0, 0, 0);
    }
  };
  if (p0 < p1) load(cur, p0);
  for (int p = p0; p < p1; ++p) {
    if (p + 1 < p1) load(nxt, p + 1);
    float sc[5];
#pragma unroll
    for (int gl = 0; gl < 5; ++gl) sc[gl] = (5 * p + gl < c.G) ? ld_scale(c.scales, 5 * p + gl, c.lane) : 0.0f;
    float acc[M][5];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int gl = 0; gl < 5; ++gl) acc[m][gl] = 0.0f;
    cu32p xb[M];
    set_xb(xb, c, kPeriodK * p);
    const int kleft = c.K - kPeriodK * p;
    if (kleft >= kPeriodK) {
      t_period<M, false>(cur, 8, c.lut, lane_off, xb, kleft, acc, std::make_integer_sequence<int, 8>{});
    } else {
      const int nch = (kleft + 79) / 80;
      t_period<M, true>(cur, nch, c.lut, lane_off, xb, kleft, acc, std::make_integer_sequence<int, 8>{});
    }
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int gl = 0; gl < 5; ++gl) y[m] = fmaf(sc[gl], acc[m][gl], y[m]);
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) cur[ch] = nxt[ch];
  }
}

template <int M, int GL>
__device__ __forceinline__ void i2_group(const uint4 d0, const uint4 d1, const SlabCtx<M>& c, uint32_t lane_off,
                                         const cu32p (&xb)[M], float (&acc)[M]) {
  i2_chunk<M, 128 * GL>(d0, c.lut, lane_off, xb, acc, std::make_integer_sequence<int, 16>{});
  i2_chunk<M, 128 * GL + 64>(d1, c.lut, lane_off, xb, acc, std::make_integer_sequence<int, 16>{});
}

template <int M>
__device__ void run_i2(const SlabCtx<M>& c, int p0, int p1, float (&y)[M]) {
  const uint32_t lane_off = (uint32_t)(c.lane & 3) << 3;
  uint4 cur[10], nxt[10];
  auto load = [&](uint4(&d)[10], int p) {
#pragma unroll
    for (int ch = 0; ch < 10; ++ch) {
      const int g = 5 * p + (ch >> 1);
      d[ch] = g < c.G ? ld_chunk(c.codes + (int64_t)(10 * p + ch) * kSlabChunkBytes) : make_uint4(0, 0, 0, 0);
    }
  };
  if (p0 < p1) load(cur, p0);
  for (int p = p0; p < p1; ++p) {
    if (p + 1 < p1) load(nxt, p + 1);
    cu32p xb[M];
    set_xb(xb, c, kPeriodK * p);
#define QL_I2_GROUP(GL)                                                  \
    if (5 * p + GL < c.G) {                                              \
      const float s = ld_scale(c.scales, 5 * p + GL, c.lane);            \
      float acc[M];                                                      \
      _Pragma("unroll") for (int m = 0; m < M; ++m) acc[m] = 0.0f;       \
      i2_group<M, GL>(cur[2 * GL], cur[2 * GL + 1], c, lane_off, xb, acc); \
      _Pragma("unroll") for (int m = 0; m < M; ++m) y[m] = fmaf(s, acc[m], y[m]); \
    }
    QL_I2_GROUP(0) QL_I2_GROUP(1) QL_I2_GROUP(2) QL_I2_GROUP(3) QL_I2_GROUP(4)
#undef QL_I2_GROUP
#pragma unroll
    for (int ch = 0; ch < 10; ++ch) cur[ch] = nxt[ch];
  }
}

template <int M, int GL>
__device__ __forceinline__ void i3_group(const uint4 d0, const uint4 d1, const uint4 d2, const SlabCtx<M>& c,
                                         const cu32p (&xb)[M], float (&acc)[M]) {
  const uint32_t w[12] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w, d2.x, d2.y, d2.z, d2.w};
  i3_triple<M, 128 * GL + 0>(w[0], w[1], w[2], c.lut, xb, acc, std::make_integer_sequence<int, 16>{});
  i3_triple<M, 128 * GL + 32>(w[3], w[4], w[5], c.lut, xb, acc, std::make_integer_sequence<int, 16>{});
  i3_triple<M, 128 * GL + 64>(w[6], w[7], w[8], c.lut, xb, acc, std::make_integer_sequence<int, 16>{});
  i3_triple<M, 128 * GL + 96>(w[9], w[10], w[11], c.lut, xb, acc, std::make_integer_sequence<int, 16>{});
}

template <int M>
__device__ void run_i3(const SlabCtx<M>& c, int p0, int p1, float (&y)[M]) {
  uint4 cur[15], nxt[15];
  auto load = [&](uint4(&d)[15], int p) {
#pragma unroll
    for (int ch = 0; ch < 15; ++ch) {
      const int g = 5 * p + ch / 3;
      d[ch] = g < c.G ? ld_chunk(c.codes + (int64_t)(15 * p + ch) * kSlabChunkBytes) : make_uint4(0, 0, 0, 0);
    }
  };
  if (p0 < p1) load(cur, p0);
  for (int p = p0; p < p1; ++p) {
    if (p + 1 < p1) load(nxt, p + 1);
    cu32p xb[M];
    set_xb(xb, c, kPeriodK * p);
#define QL_I3_GROUP(GL)                                                        \
    if (5 * p + GL < c.G) {                                                    \
      const float s = ld_scale(c.scales, 5 * p + GL, c.lane);                  \
      float acc[M];                                                            \
      _Pragma("unroll") for (int m = 0; m < M; ++m) acc[m] = 0.0f;             \
      i3_group<M, GL>(cur[3 * GL], cur[3 * GL + 1], cur[3 * GL + 2], c, xb, acc); \
      _Pragma("unroll") for (int m = 0; m < M; ++m) y[m] = fmaf(s, acc[m], y[m]); \
    }
    QL_I3_GROUP(0) QL_I3_GROUP(1) QL_I3_GROUP(2) QL_I3_GROUP(3) QL_I3_GROUP(4)
#undef QL_I3_GROUP
#pragma unroll
    for (int ch = 0; ch < 15; ++ch) cur[ch] = nxt[ch];
  }
}

template <int M>
__device__ __forceinline__ void run_slab(int gr, const SlabCtx<M>& c, int p0, int p1, float (&y)[M]) {
  if (gr == QL_GRID_T)
    run_t<M>(c, p0, p1, y);
  else if (gr == QL_GRID_I2)
    run_i2<M>(c, p0, p1, y);
  else
    run_i3<M>(c, p0, p1, y);
}

// ---------------------------------------------------------------- kernels
constexpr int kWaves = 4;

// Single matrix.  Each workgroup iteration takes kWaves/KS slabs; the KS waves
// of a slab split its periods and are summed in LDS in fixed order.
template <int M>
__global__ void __launch_bounds__(kWaves * 64, 2) gemv_kernel(MatArgs a, int Mact, int KS, int64_t nslabs) {
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLutBytes];
  __shared__ float red[kWaves][M][64];
  build_luts(lut);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int spw = kWaves / KS;
  const int64_t ntasks = (nslabs + spw - 1) / spw;
  const int P = (a.K + kPeriodK - 1) / kPeriodK;
  const int kpart = wave % KS;
  const int p0 = P * kpart / KS, p1 = P * (kpart + 1) / KS;
  const int G = a.K / kGroup, G8 = (G + 7) / 8;
  for (int64_t t = blockIdx.x; t < ntasks; t += gridDim.x) {
    const int64_t slab = t * spw + wave / KS;
    float y[M];
#pragma unroll
    for (int m = 0; m < M; ++m) y[m] = 0.0f;
    if (slab < nslabs) {
      int gr;
      const int64_t off = slab_offset(slab, a.K, a.grid, a.blk_grid, a.blk_off, &gr);
      SlabCtx<M> c{a.packed + off + lane * kChunkBytes, a.pscales + slab * (int64_t)G8 * kSlab * 8, a.x, a.K, G,
                   Mact, lane, lut};
      run_slab<M>(gr, c, p0, p1, y);
    }
    const int64_t row = slab * kSlab + lane;
    if (KS > 1) {
#pragma unroll
      for (int m = 0; m < M; ++m) red[wave][m][lane] = y[m];
      __syncthreads();
      if (kpart == 0 && slab < nslabs && row < a.N) {
        for (int m = 0; m < Mact; ++m) {
          float s = red[wave][m][lane];
          for (int q = 1; q < KS; ++q) s += red[wave + q][m][lane];
          a.y[(int64_t)m * a.N + row] = s;
        }
      }
      __syncthreads();
    } else if (slab < nslabs && row < a.N) {
      for (int m = 0; m < Mact; ++m) a.y[(int64_t)m * a.N + row] = y[m];
    }
  }
}

// Many independent matrices in one persistent launch; one slab per wave task.
template <int M>
__global__ void __launch_bounds__(kWaves * 64, 2) gemv_grouped_kernel(const ql_gemv_desc* __restrict__ descs,
                                                                      int count, int64_t total, int Mact) {
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLutBytes];
  build_luts(lut);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t < total; t += (int64_t)gridDim.x * kWaves) {
    // descriptor holding slab t: last d with slab_begin <= t
    int lo = 0, hi = count - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (descs[mid].slab_begin <= t) lo = mid; else hi = mid - 1;
    }
    const ql_gemv_desc& d = descs[lo];
    const int64_t slab = t - d.slab_begin;
    const int K = d.K, G = K / kGroup, G8 = (G + 7) / 8;
    int gr;
    const int64_t off = slab_offset(slab, K, d.grid, d.blk_grid, d.blk_off, &gr);
    float y[M];
#pragma unroll
    for (int m = 0; m < M; ++m) y[m] = 0.0f;
    SlabCtx<M> c{static_cast<const uint8_t*>(d.packed) + off + lane * kChunkBytes,
                 d.pscales + slab * (int64_t)G8 * kSlab * 8, d.x, K, G, Mact, lane, lut};
    run_slab<M>(gr, c, 0, (K + kPeriodK - 1) / kPeriodK, y);
    const int64_t row = slab * kSlab + lane;
    if (row < d.N)
      for (int m = 0; m < Mact; ++m) d.y[(int64_t)m * d.N + row] = y[m];
  }
}

// ---------------------------------------------------------------- launchers
static int cu_count_cached = 0;

int device_cu_count() {
  if (!cu_count_cached) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                 hipSuccess && n > 0)
      cu_count_cached = n;
    else
      return 256;
  }
  return cu_count_cached;
}

template <int M>
static hipError_t launch_gemv_m(const MatArgs& a, int Mact, hipStream_t stream) {
  const int64_t nslabs = ((int64_t)a.N + kSlab - 1) / kSlab;
  const int P = (a.K + kPeriodK - 1) / kPeriodK;
  const int slots = device_cu_count() * 2;  // two resident workgroups per CU
  // split the periods of a slab over waves when there are too few slabs to fill the chip
  int KS = 1;
  while (KS < kWaves && (nslabs * KS) < (int64_t)slots * kWaves && P >= 2 * KS) KS *= 2;
  const int64_t ntasks = (nslabs + (kWaves / KS) - 1) / (kWaves / KS);
  const int grid = (int)(ntasks < slots ? ntasks : slots);
  hipLaunchKernelGGL(gemv_kernel<M>, dim3(grid), dim3(kWaves * 64), 0, stream, a, Mact, KS, nslabs);
  return hipGetLastError();
}

hipError_t launch_gemv(const MatArgs& a, int M, hipStream_t stream) {
  if (M == 1) return launch_gemv_m<1>(a, M, stream);
  if (M == 2) return launch_gemv_m<2>(a, M, stream);
  if (M <= 4) return launch_gemv_m<4>(a, M, stream);
  return launch_gemv_m<8>(a, M, stream);
}

template <int M>
static hipError_t launch_grouped_m(const ql_gemv_desc* descs, int32_t count, int64_t total, int Mact,
                                   hipStream_t stream) {
  const int slots = device_cu_count() * 2;
  const int64_t wg_needed = (total + kWaves - 1) / kWaves;
  const int grid = (int)(wg_needed < slots ? wg_needed : slots);
  hipLaunchKernelGGL(gemv_grouped_kernel<M>, dim3(grid), dim3(kWaves * 64), 0, stream, descs, count, total, Mact);
  return hipGetLastError();
}

hipError_t launch_gemv_grouped(const ql_gemv_desc* descs, int32_t count, int64_t total_slabs, int M,
                               hipStream_t stream) {
  if (M == 1) return launch_grouped_m<1>(descs, count, total_slabs, M, stream);
  if (M == 2) return launch_grouped_m<2>(descs, count, total_slabs, M, stream);
  if (M <= 4) return launch_grouped_m<4>(descs, count, total_slabs, M, stream);
  return launch_grouped_m<8>(descs, count, total_slabs, M, stream);
}

}  // namespace ql
