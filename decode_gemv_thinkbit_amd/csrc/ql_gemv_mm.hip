// Batched decode, 2 <= M <= 16 tokens, over ThinkBit-packed weights (gfx950).
//
// At a decode batch of a few tokens the product is still a weight stream: every
// packed byte is read once per step and used M times (ThinkBit summary page,
// onedev.kr/papers/1416, section "What it is": the decode step is bound by
// reading the weights; w = c * s with one bf16 scale per 128 inputs, section
// "How it works").  The batch-1 kernel multiplies with v_dot2 and would need
// M times the arithmetic; here the M-fold work goes to the matrix cores
// instead, so the cost per packed byte stays that of decoding it once.
//
// Mapping.  One wave owns a 64-row slab of the packed layout (four blocks of
// 16 rows).  For v_mfma_f32_16x16x32_bf16 lane l = (i = l & 15, q = l >> 4)
// supplies k-slots 8q..8q+7 of row i of the first operand and of column i of
// the second.  The first operand is x (row i = token i, tokens past M read as
// zero) and the second the decoded codes (column i = weight row 16 * block + i),
// so D[t][i] = sum_k x_t[k] c_i[k]: lane l ends up holding tokens 4q..4q+3 of
// one weight row, and the group scale of that row multiplies its four values.
// The slot order inside a group is free as long as both operands use it: lane
// q decodes whole stored bytes from the dword q of each 16-byte chunk it loads,
// and the matching x dwords are loaded next to each other.
//
// Decode.  The same LDS tables as the batch-1 kernel turn bytes into bf16 codes:
//   ternary: one 16-byte entry per byte, (d0,d1) (d2,d3) (d4,0) (0,d4), used
//            whole as the 4-dword code operand of one MFMA; the x operand puts
//            zero against the unused dword (even bytes .w, odd bytes .z);
//   2-bit:   two bytes (8 codes) per MFMA operand;
//   3-bit:   four 6-bit fields (8 codes) per MFMA operand.
// Each product c * x is exact and MFMA accumulates in fp32; partial sums are
// kept per 128-input group and scaled in fp32, as in the batch-1 kernel.
//
// Group edges.  2- and 3-bit chunks never straddle a 128-input group.  A
// ternary chunk holds 80 inputs, and in four of the eight chunks of a 640-input
// period a group edge falls inside it: there the x operand is split by lane
// (dwords before the edge / after it; the edges are even, so no dword straddles
// one) and each window runs two MFMAs, one into each group's accumulator.
#include "ql_internal.hpp"
#include "ql_luts.hpp"
#include "ql_stream.hpp"

namespace ql {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kMmWaves = 8;   // waves per workgroup
constexpr int kMmWgPerCu = 2;  // resident workgroups per CU (LDS tables: 69 KB each)
constexpr int kRB = kSlab / 16;  // 16-row blocks per slab

__device__ __forceinline__ f32x4_t mma(const u32x4_t& xa, const u32x4_t& cb, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xa), __builtin_bit_cast(bf16x8_t, cb), c,
                                                 0, 0, 0);
}

// Code dwords of one slab: dword q of 16-byte chunk `chunk` of row 16 * rb + i.
// Chunks past the slab's range read as zero without a memory access.
struct CodeDw {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t lane_off;
  __device__ __forceinline__ CodeDw(const uint8_t* slab, int nchunks, int lane)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(uniform_ptr(slab), (short)0,
                                               __builtin_amdgcn_readfirstlane(nchunks * kSlabChunkBytes), 0x00020000)),
        lane_off((uint32_t)(lane & 15) * kChunkBytes + (uint32_t)(lane >> 4) * 4u) {}
  __device__ __forceinline__ uint32_t load(int chunk, int rb) const {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc, lane_off + (uint32_t)chunk * kSlabChunkBytes + rb * 256u,
                                                          0, 2);
  }
};

// Activations of the batch: token t = lane & 15 of an M x K bf16 matrix; rows
// past M (and anything past the matrix) read as zero.
struct XSrc {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t base;  // byte offset of this lane's token row (past the end for t >= M)
  __device__ __forceinline__ XSrc(const uint16_t* x, int M, int K, int lane)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(uniform_ptr(x), (short)0,
                                               __builtin_amdgcn_readfirstlane(2 * M * K), 0x00020000)) {
    const int t = lane & 15;
    base = t < M ? (uint32_t)(2 * t * K) : (uint32_t)(2 * M * K);
  }
  __device__ __forceinline__ u32x4_t b128(uint32_t off) const {
    const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, base + off, 0, 0);
    return u32x4_t{(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
  }
  __device__ __forceinline__ u32x2_t b64(uint32_t off) const {
    typedef int i32x2_t __attribute__((ext_vector_type(2)));
    const i32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, base + off, 0, 0);
    return u32x2_t{(uint32_t)v.x, (uint32_t)v.y};
  }
};

struct Acc {
  f32x4_t v[kRB];
};

__device__ __forceinline__ void zero(Acc& a) {
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) a.v[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// y += s(row, g) * D for the slab's rows; lane l holds weight row 16 rb + (l & 15)
__device__ __forceinline__ void flush(Acc& y, const Acc& d, const uint16_t* scales, int g, int G, int lane) {
  if (g >= G) return;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float s = ld_scale(scales, g, 16 * rb + (lane & 15));
#pragma unroll
    for (int i = 0; i < 4; ++i) y.v[rb][i] = fmaf(s, d.v[rb][i], y.v[rb][i]);
  }
}

// ---------------------------------------------------------------- ternary
// Chunk phase c (0..7) of a 640-input period; an edge at input offset e inside it
// (0 = none).  Lane q's x dwords cover chunk inputs 20q .. 20q+19.
constexpr int t_edge(int c) { return c == 1 ? 48 : c == 3 ? 16 : c == 4 ? 64 : c == 6 ? 32 : 0; }
// chunk phases after which a group ends (its accumulator is scaled and cleared)
constexpr bool t_flush_after(int c) { return c == 1 || c == 3 || c == 4 || c == 6 || c == 7; }

// the 4-dword x operand of window w (byte 4q + w of the lane's chunk dword)
template <int W>
__device__ __forceinline__ u32x4_t t_xop(const uint32_t (&X)[10]) {
  constexpr int u = W >> 1;
  if constexpr ((W & 1) == 0)
    return u32x4_t{X[5 * u], X[5 * u + 1], X[5 * u + 2], 0u};
  else
    return u32x4_t{X[5 * u + 3], X[5 * u + 4], 0u, X[5 * u + 2]};
}

// the same with the dwords at or past the edge (index >= nlo) zeroed
template <int W>
__device__ __forceinline__ u32x4_t t_xop_lo(const uint32_t (&X)[10], int nlo) {
  constexpr int u = W >> 1;
  auto lo = [&](int i) __attribute__((always_inline)) { return i < nlo ? X[i] : 0u; };
  if constexpr ((W & 1) == 0)
    return u32x4_t{lo(5 * u), lo(5 * u + 1), lo(5 * u + 2), 0u};
  else
    return u32x4_t{lo(5 * u + 3), lo(5 * u + 4), 0u, lo(5 * u + 2)};
}

struct TWinE {
  u32x4_t e[kRB];
};

// table entries of window W from the chunk's code dwords (one per row block)
template <int W>
__device__ __forceinline__ void t_read(TWinE& b, const uint32_t (&cd)[kRB], uint32_t lane_off, const uint8_t* lut) {
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const uint32_t addr = __builtin_amdgcn_perm(cd[rb], lane_off, 0x0C0C0000u | ((4u + W) << 8));
    b.e[rb] = lds_b128(lut + kTLut + addr);
  }
}

__device__ void run_t(const uint8_t* codes, const uint16_t* scales, const XSrc& xs, int K, int G, int lane,
                      const uint8_t* lut, Acc& y) {
  const int nchunks = (K + 79) / 80;
  const int nper = (nchunks + 7) / 8;
  const CodeDw src(codes, nchunks, lane);
  const int q = lane >> 4;
  const uint32_t lane_off = (uint32_t)(lane & 15) << 4;
  Acc cur, nxt;
  zero(cur);
  zero(nxt);
  // ring of code dwords: chunk ch lives in slot ch % 4 (a period is 8 chunks), two ahead
  uint32_t cd[4][kRB];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) cd[s][rb] = src.load(s, rb);
  for (int p = 0; p < nper; ++p) {
    const bool tail = p == nper - 1;
    sfor<8>([&](auto c_) __attribute__((always_inline)) {
      constexpr int C = decltype(c_)::value;
      const int ch = 8 * p + C;
      sched_fence();
      if (ch < nchunks) {
        // prefetch chunk ch + 2 (slot (ch + 2) % 4; chunk ch - 2 is done with it)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) cd[(C + 2) & 3][rb] = src.load(ch + 2, rb);
        // x dwords of this chunk: inputs 80 ch + 20 q .. + 19
        uint32_t X[10];
        {
          const uint32_t off = (uint32_t)(160 * ch + 40 * q);
          const u32x4_t a = xs.b128(off), b = xs.b128(off + 16);
          const u32x2_t c2 = xs.b64(off + 32);
          X[0] = a.x; X[1] = a.y; X[2] = a.z; X[3] = a.w;
          X[4] = b.x; X[5] = b.y; X[6] = b.z; X[7] = b.w;
          X[8] = c2.x; X[9] = c2.y;
        }
        if (tail) {  // inputs past K meet zero codes; keep them zero on this side too
          const int left = K - (80 * ch + 20 * q);
#pragma unroll
          for (int i = 0; i < 10; ++i) X[i] = 2 * i < left ? X[i] : 0u;
        }
        constexpr int E = t_edge(C);
        // edge chunk: how many of the lane's 10 x dwords lie before the edge
        const int nlo = E == 0 ? 10 : ((E - 20 * q) / 2 < 0 ? 0 : (E - 20 * q) / 2);
        sfor<4>([&](auto w_) __attribute__((always_inline)) {
          constexpr int W = decltype(w_)::value;
          TWinE cur_e;
          sched_fence();
          t_read<W>(cur_e, cd[C & 3], lane_off, lut);
          lgkm_wait0();
          const u32x4_t xo = t_xop<W>(X);
          if constexpr (E == 0) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) cur.v[rb] = mma(xo, cur_e.e[rb], cur.v[rb]);
          } else {
            const u32x4_t xl = t_xop_lo<W>(X, nlo);
            const u32x4_t xh = xo ^ xl;
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
              cur.v[rb] = mma(xl, cur_e.e[rb], cur.v[rb]);
              nxt.v[rb] = mma(xh, cur_e.e[rb], nxt.v[rb]);
            }
          }
        });
      }
      if constexpr (t_flush_after(C)) {
        constexpr int gl = C == 1 ? 0 : C == 3 ? 1 : C == 4 ? 2 : C == 6 ? 3 : 4;
        flush(y, cur, scales, 5 * p + gl, G, lane);
        cur = nxt;
        zero(nxt);
      }
    });
  }
}

// ---------------------------------------------------------------- 2-bit
// A group is 32 bytes = 2 chunks of 64 inputs.  Lane q's chunk dword holds
// bytes 4q..4q+3 (inputs 16q .. 16q+15 of the chunk); window w takes bytes
// 4q + 2w, 4q + 2w + 1, whose x dwords are 8q + 4w .. + 3 of the chunk.
__device__ void run_i2(const uint8_t* codes, const uint16_t* scales, const XSrc& xs, int K, int G, int lane,
                       const uint8_t* lut, Acc& y) {
  const int nchunks = 2 * G;
  const CodeDw src(codes, nchunks, lane);
  const int q = lane >> 4;
  const uint32_t lane_off = (uint32_t)(lane & 3) << 3;
  uint32_t cd[2][kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) cd[0][rb] = src.load(0, rb);
  for (int g = 0; g < G; ++g) {
    Acc d;
    zero(d);
    sfor<2>([&](auto h_) __attribute__((always_inline)) {
      constexpr int H = decltype(h_)::value;
      const int ch = 2 * g + H;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) cd[H ^ 1][rb] = src.load(ch + 1, rb);
      const uint32_t off = (uint32_t)(128 * ch + 32 * q);
      const u32x4_t x0 = xs.b128(off), x1 = xs.b128(off + 16);
      u32x2_t e[2][kRB][2];
      sfor<2>([&](auto w_) __attribute__((always_inline)) {
        constexpr int W = decltype(w_)::value;
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const uint32_t bv = (cd[H][rb] >> (8 * (2 * W + j))) & 0xFFu;
            e[W][rb][j] = lds_b64(lut + kI2Lut + ((bv << 5) | lane_off));
          }
      });
      lgkm_wait0();
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        d.v[rb] = mma(x0, u32x4_t{e[0][rb][0].x, e[0][rb][0].y, e[0][rb][1].x, e[0][rb][1].y}, d.v[rb]);
        d.v[rb] = mma(x1, u32x4_t{e[1][rb][0].x, e[1][rb][0].y, e[1][rb][1].x, e[1][rb][1].y}, d.v[rb]);
      }
    });
    flush(y, d, scales, g, G, lane);
  }
}

// ---------------------------------------------------------------- 3-bit
// A group is 48 bytes = four 96-bit triples of 32 codes.  Lane q decodes triple
// q of its row (three aligned dwords, each inside one chunk); window w takes
// fields 4w .. 4w+3 (codes 32q + 8w ..), whose x dwords are 16q + 4w .. + 3.
__device__ void run_i3(const uint8_t* codes, const uint16_t* scales, const XSrc& xs, int K, int G, int lane,
                       const uint8_t* lut, Acc& y) {
  const int nchunks = 3 * G;
  const CodeDw src(codes, nchunks, lane);
  const int q = lane >> 4;
  // the triple's three dwords: group-relative bytes 12 q + 4 j (each inside one chunk)
  uint32_t toff[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int byte = 12 * q + 4 * j;
    toff[j] = (uint32_t)(byte >> 4) * kSlabChunkBytes + (uint32_t)(byte & 15) - (uint32_t)(lane >> 4) * 4u;
  }
  auto load_tr = [&](int g, uint32_t (&t)[kRB][3]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb)
        t[rb][j] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
            src.rsrc, src.lane_off + toff[j] + (uint32_t)(3 * g) * kSlabChunkBytes + rb * 256u, 0, 2);
  };
  uint32_t tw[2][kRB][3];
  load_tr(0, tw[0]);
  for (int gb = 0; gb < G; gb += 2) {
    sfor<2>([&](auto s_) __attribute__((always_inline)) {
      constexpr int S = decltype(s_)::value;
      const int g = gb + S;
      if (g < G) {
        load_tr(g + 1, tw[S ^ 1]);  // past the last group: reads zero, no memory access
        const uint32_t off = (uint32_t)(256 * g + 64 * q);
        u32x4_t xo[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) xo[w] = xs.b128(off + 16 * w);
        Acc d;
        zero(d);
        sfor<4>([&](auto w_) __attribute__((always_inline)) {
          constexpr int W = decltype(w_)::value;
          sched_fence();
          uint32_t e[kRB][4];
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb) {
            const uint32_t w0 = tw[S][rb][0], w1 = tw[S][rb][1], w2 = tw[S][rb][2];
            e[rb][0] = lds_b32(lut + kI3Lut + i3_field_x4<4 * W + 0>(w0, w1, w2));
            e[rb][1] = lds_b32(lut + kI3Lut + i3_field_x4<4 * W + 1>(w0, w1, w2));
            e[rb][2] = lds_b32(lut + kI3Lut + i3_field_x4<4 * W + 2>(w0, w1, w2));
            e[rb][3] = lds_b32(lut + kI3Lut + i3_field_x4<4 * W + 3>(w0, w1, w2));
          }
          lgkm_wait0();
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
            d.v[rb] = mma(xo[W], u32x4_t{e[rb][0], e[rb][1], e[rb][2], e[rb][3]}, d.v[rb]);
        });
        flush(y, d, scales, g, G, lane);
      }
    });
  }
}

// One task: one 64-row slab of one descriptor, all M tokens.
__device__ __forceinline__ void mm_task(const ql_gemv_desc* __restrict__ descs, int count, int64_t t, int M,
                                        const uint8_t* lut, int lane) {
  const ql_gemv_desc& d = descs[find_desc(descs, count, t)];
  const int64_t slab = t - d.slab_begin;
  const int K = d.K, G = K / kGroup, G8 = (G + 7) / 8;
  int gr;
  const int64_t off = slab_offset(slab, K, d.grid, d.blk_grid, d.blk_off, &gr);
  const uint8_t* codes = static_cast<const uint8_t*>(d.packed) + off;
  const uint16_t* scales = d.pscales + slab * (int64_t)G8 * kSlab * 8;
  const XSrc xs(d.x, M, K, lane);
  Acc y;
  zero(y);
  if (gr == QL_GRID_T)
    run_t(codes, scales, xs, K, G, lane, lut, y);
  else if (gr == QL_GRID_I2)
    run_i2(codes, scales, xs, K, G, lane, lut, y);
  else
    run_i3(codes, scales, xs, K, G, lane, lut, y);
  // lane l: tokens 4q .. 4q+3 of weight row 16 rb + (l & 15)
  const int q = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int64_t row = slab * kSlab + 16 * rb + (lane & 15);
    if (row < d.N)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * q + i < M) d.y[(int64_t)(4 * q + i) * d.N + row] = y.v[rb][i];
  }
}

__global__ void __launch_bounds__(kMmWaves * 64, 4) gemv_mm_grouped_kernel(const ql_gemv_desc* __restrict__ descs,
                                                                         int count, int64_t total, int M,
                                                                         uint32_t* __restrict__ sched) {
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLutBytes];
  build_luts(lut);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  TaskQueues tq(sched, total, (int64_t)gridDim.x * kMmWaves);
  int64_t t = (int64_t)blockIdx.x * kMmWaves + wave;
  if (t >= total) t = tq.next(lane);
  while (t >= 0) {
    const uint32_t claim = tq.claim(lane);
    mm_task(descs, count, t, M, lut, lane);
    t = tq.resolve(claim, lane);
  }
  tq.checkout(lane);
}

}  // namespace

hipError_t launch_gemv_mm_grouped(const ql_gemv_desc* descs, int32_t count, int64_t total_slabs, int M,
                                  uint32_t* sched, hipStream_t stream) {
  if (M < 2 || M > 16) return hipErrorInvalidValue;
  const int slots = device_cu_count() * kMmWgPerCu;
  const int64_t wg_needed = (total_slabs + kMmWaves - 1) / kMmWaves;
  const int grid = (int)(wg_needed < slots ? wg_needed : slots);
  hipLaunchKernelGGL(gemv_mm_grouped_kernel, dim3(grid), dim3(kMmWaves * 64), 0, stream, descs, count, total_slabs, M,
                     sched);
  return hipGetLastError();
}

}  // namespace ql
