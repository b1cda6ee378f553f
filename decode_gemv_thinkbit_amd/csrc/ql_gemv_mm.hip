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

#ifndef QL_MM_WAVES
#define QL_MM_WAVES 6
#endif
#ifndef QL_MM_WAVES_PER_EU
#define QL_MM_WAVES_PER_EU 3
#endif
constexpr int kMmWaves = QL_MM_WAVES;  // waves per workgroup
constexpr int kMmWgPerCu = 2;  // resident workgroups per CU (LDS tables: 77 KB each; 168 VGPRs: 3 waves per SIMD)
constexpr int kRB = kSlab / 16;  // 16-row blocks per slab
static_assert(kRB * 4 * 64 <= kPartWords, "a split part stores 4 tokens x kRB rows per lane");

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
};

struct Acc {
  f32x4_t v[kRB];
};

__device__ __forceinline__ void zero(Acc& a) {
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) a.v[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// Group scales of the slab's four row blocks (row 16 rb + (lane & 15)), read as
// aligned dwords that hold groups 2k and 2k+1, one pair of groups ahead of use
// (a scale read right before its multiply would stall the wave on memory at
// every group).
struct Scales {
  uint32_t cur[kRB], nxt[kRB];  // pairs k and k + 1
  const uint16_t* ss;
  int G, lane;  // G: end of the groups this task sums (groups from G on are dropped)
  __device__ __forceinline__ void load(uint32_t (&v)[kRB], int k) const {
    int g = 2 * k;
    g = g < G ? g : G - 1;  // past the row: any in-range pair (never used)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) v[rb] = ld_scale_pair(ss, g, 16 * rb + (lane & 15));
  }
  // groups g0 .. g_end - 1 (pairs are aligned: g0 may be odd)
  __device__ __forceinline__ Scales(const uint16_t* s, int g0, int g_end, int l) : ss(s), G(g_end), lane(l) {
    load(cur, g0 >> 1);
    load(nxt, (g0 >> 1) + 1);
  }
  // after the last group of pair k: move to pair k + 1 and start reading pair k + 2
  __device__ __forceinline__ void advance(int k) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) cur[rb] = nxt[rb];
    load(nxt, k + 2);
  }
  __device__ __forceinline__ float get(int rb, int g) const {
    return __uint_as_float((g & 1) ? (cur[rb] & 0xFFFF0000u) : (cur[rb] << 16));
  }
};

// y += s(row, g) * D; lane l holds weight row 16 rb + (l & 15).  Moves the
// scale window on after the second group of a pair.
__device__ __forceinline__ void flush(Acc& y, const Acc& d, Scales& sc, int g) {
  if (g < sc.G) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const float s = sc.get(rb, g);
#pragma unroll
      for (int i = 0; i < 4; ++i) y.v[rb][i] = fmaf(s, d.v[rb][i], y.v[rb][i]);
    }
  }
  if (g & 1) sc.advance(g >> 1);
}

// ---------------------------------------------------------------- ternary
// Chunk phase c (0..7) of a 640-input period; an edge at input offset e inside it
// (0 = none).  Lane q's x dwords cover chunk inputs 20q .. 20q+19.
constexpr int t_edge(int c) { return c == 1 ? 48 : c == 3 ? 16 : c == 4 ? 64 : c == 6 ? 32 : 0; }
// chunk phases after which a group ends (its accumulator is scaled and cleared)
constexpr bool t_flush_after(int c) { return c == 1 || c == 3 || c == 4 || c == 6 || c == 7; }

struct TWinE {
  u32x4_t e[kRB];
};

// table entries of window W (byte W of each code dword; one per row block)
template <int W>
__device__ __forceinline__ void t_read(TWinE& b, const uint32_t (&cd)[kRB], uint32_t lane_off, const uint8_t* lut) {
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const uint32_t addr = __builtin_amdgcn_perm(cd[rb], lane_off, 0x0C0C0000u | ((4u + W) << 8));
    b.e[rb] = lds_b128(lut + kTLut + addr);
  }
}

// x of byte pair u (0, 1) of the lane's chunk dword: five dwords, inputs 10u .. 10u+9
// of the lane's 20 (byte offset 160 ch + 40 q + 20 u of the token row)
struct X5 {
  uint32_t d[5];
};
__device__ __forceinline__ void load_x5(X5& x, const XSrc& xs, uint32_t off) {
  const u32x4_t a = xs.b128(off);
  x.d[0] = a.x; x.d[1] = a.y; x.d[2] = a.z; x.d[3] = a.w;
  x.d[4] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(xs.rsrc, xs.base + off + 16, 0, 0);
}

// Periods [p0, p1) of the slab's rows (the whole row, or one split part).
__device__ void run_t(const uint8_t* codes, const uint16_t* scales, const XSrc& xs, int K, int G, int p0, int p1,
                      int lane, const uint8_t* lut, Acc& y) {
  Scales sc(scales, 5 * p0, 5 * p1 < G ? 5 * p1 : G, lane);
  const int nchunks = (K + 79) / 80;
  const int nper = (nchunks + 7) / 8;
  // chunks past the part (or the row) read as zero without memory traffic
  const CodeDw src(codes, nchunks < 8 * p1 ? nchunks : 8 * p1, lane);
  const int q = lane >> 4;
  const uint32_t lane_off = (uint32_t)(lane & 15) << 4;
  Acc cur, nxt;
  zero(cur);
  zero(nxt);
  // code dwords: chunk ch in slot ch % 4, loaded two chunks ahead.  Every load
  // is unconditional (past the slab or x it reads zero), which keeps the
  // compiler's wait counts exact.
  uint32_t cd[4][kRB];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) cd[s][rb] = src.load(8 * p0 + s, rb);
  // x pair P (global: 2 ch + U) in slot P % 4, three pairs ahead
  X5 xw[4];
  auto xoff = [&](int P) __attribute__((always_inline)) { return (uint32_t)(160 * (P >> 1) + 40 * q + 20 * (P & 1)); };
#pragma unroll
  for (int i = 0; i < 3; ++i) load_x5(xw[i], xs, xoff(16 * p0 + i));
  // table entries, one window ahead (window w of a chunk in buffer w % 2)
  TWinE ent[2];
  t_read<0>(ent[0], cd[0], lane_off, lut);
  // The last period skips its second half when the row ends in the first:
  // no group still inside K ends after chunk 4 of such a period (K is a
  // multiple of 128).
  const bool short_last = nchunks - 8 * (nper - 1) <= 4;
  for (int p = p0; p < p1; ++p) {
    const bool tail = p == nper - 1;
    auto chunk = [&](auto c_) __attribute__((always_inline)) {
      constexpr int C = decltype(c_)::value;
      constexpr int E = t_edge(C);
      const int ch = 8 * p + C;
      sched_fence();
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) cd[(C + 2) & 3][rb] = src.load(ch + 2, rb);
      sfor<2>([&](auto u_) __attribute__((always_inline)) {
        constexpr int U = decltype(u_)::value;
        constexpr int P = 2 * C + U;  // pair within the period (the period holds 16)
        load_x5(xw[(P + 3) & 3], xs, xoff(2 * ch + U + 3));
        X5 x = xw[P & 3];
        if (tail) {  // inputs past K meet padding codes; keep them zero on this side too
          const int left = K - (80 * ch + 20 * q + 10 * U);
#pragma unroll
          for (int i = 0; i < 5; ++i) x.d[i] = 2 * i < left ? x.d[i] : 0u;
        }
        // edge chunk: how many of this pair's five dwords lie before the edge
        int nlo = 5;
        if constexpr (E != 0) {
          const int v = (E - 20 * q - 10 * U) / 2;
          nlo = v < 0 ? 0 : (v > 5 ? 5 : v);
        }
        sfor<2>([&](auto h_) __attribute__((always_inline)) {
          constexpr int H = decltype(h_)::value;  // even / odd byte of the pair
          constexpr int W = 2 * U + H;
          // this window's entries were read one window earlier; read the next
          // window's now (the last window of a chunk reads window 0 of the next
          // chunk, whose code dwords are already in the ring)
          if constexpr (W < 3)
            t_read<W + 1>(ent[(W + 1) & 1], cd[C & 3], lane_off, lut);
          else
            t_read<0>(ent[0], cd[(C + 1) & 3], lane_off, lut);
          const TWinE& cur_e = ent[W & 1];
          // even byte: (x0,x1) (x2,x3) (x4,x5) 0; odd byte: (x6,x7) (x8,x9) 0 (x4,x5)
          const u32x4_t xo = H == 0 ? u32x4_t{x.d[0], x.d[1], x.d[2], 0u} : u32x4_t{x.d[3], x.d[4], 0u, x.d[2]};
          if constexpr (E == 0) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) cur.v[rb] = mma(xo, cur_e.e[rb], cur.v[rb]);
          } else {
            auto lo = [&](int i) __attribute__((always_inline)) { return i < nlo ? x.d[i] : 0u; };
            const u32x4_t xl = H == 0 ? u32x4_t{lo(0), lo(1), lo(2), 0u} : u32x4_t{lo(3), lo(4), 0u, lo(2)};
            const u32x4_t xh = xo ^ xl;
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
              cur.v[rb] = mma(xl, cur_e.e[rb], cur.v[rb]);
              nxt.v[rb] = mma(xh, cur_e.e[rb], nxt.v[rb]);
            }
          }
        });
      });
      if constexpr (t_flush_after(C)) {
        constexpr int gl = C == 1 ? 0 : C == 3 ? 1 : C == 4 ? 2 : C == 6 ? 3 : 4;
        flush(y, cur, sc, 5 * p + gl);
        cur = nxt;
        zero(nxt);
      }
    };
    sfor<4>(chunk);
    if (!(tail && short_last)) sfor_from<4, 4>(chunk);
  }
}

// ---------------------------------------------------------------- 2-bit
// A group is 32 bytes = 2 chunks of 64 inputs.  Lane q's chunk dword holds
// bytes 4q..4q+3 (inputs 16q .. 16q+15 of the chunk); window w takes bytes
// 4q + 2w, 4q + 2w + 1, whose x dwords are 8q + 4w .. + 3 of the chunk
// (byte offset 128 ch + 32 q + 16 w of the token row).
// Group pairs [k0, k1) of the slab's rows (groups 2 k0 .. min(2 k1, G) - 1).
__device__ void run_i2(const uint8_t* codes, const uint16_t* scales, const XSrc& xs, int k0, int k1, int G, int lane,
                       const uint8_t* lut, Acc& y) {
  const int g0 = 2 * k0, g1 = 2 * k1 < G ? 2 * k1 : G;
  Scales sc(scales, g0, g1, lane);
  const int nchunks = 2 * g1;
  const CodeDw src(codes, nchunks, lane);
  const int q = lane >> 4;
  const uint32_t lane_off = (uint32_t)(lane & 3) << 3;
  // table entries of window W (bytes 2W, 2W+1) of a chunk's code dwords
  struct E2 {
    u32x2_t e[kRB][2];
  };
  auto read = [&](E2& b, const uint32_t (&c)[kRB], int W) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t bv = (c[rb] >> (8 * (2 * W + j))) & 0xFFu;
        b.e[rb][j] = lds_b64(lut + kI2Lut + ((bv << 5) | lane_off));
      }
  };
  // code dwords of chunk ch in slot ch % 4, two chunks ahead; table entries one
  // window ahead
  uint32_t cd[4][kRB];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) cd[s][rb] = src.load(2 * g0 + s, rb);
  // x of window wi (global: 2 ch + W) in slot wi % 4, three windows ahead
  u32x4_t xw[4];
  auto xoff2 = [&](int wi) __attribute__((always_inline)) { return (uint32_t)(128 * (wi >> 1) + 32 * q + 16 * (wi & 1)); };
#pragma unroll
  for (int i = 0; i < 3; ++i) xw[i] = xs.b128(xoff2(4 * g0 + i));
  E2 ent[2];
  read(ent[0], cd[0], 0);
  for (int k = k0; k < k1; ++k) {  // two groups (4 chunks) per pass; an odd last one is dropped by flush
    sfor<2>([&](auto s_) __attribute__((always_inline)) {
      constexpr int S = decltype(s_)::value;
      const int g = 2 * k + S;
      Acc d;
      zero(d);
      sfor<2>([&](auto h_) __attribute__((always_inline)) {
        constexpr int H = decltype(h_)::value;
        constexpr int CS = 2 * S + H;  // chunk slot
        const int ch = 2 * g + H;
        sched_fence();
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) cd[(CS + 2) & 3][rb] = src.load(ch + 2, rb);
        sfor<2>([&](auto w_) __attribute__((always_inline)) {
          constexpr int W = decltype(w_)::value;
          constexpr int WI = 2 * CS + W;  // window index within the pass
          xw[(WI + 3) & 3] = xs.b128(xoff2(2 * ch + W + 3));
          if constexpr (W == 0)
            read(ent[(WI + 1) & 1], cd[CS], 1);
          else
            read(ent[(WI + 1) & 1], cd[(CS + 1) & 3], 0);
          const u32x4_t xo = xw[WI & 3];
          const E2& e = ent[WI & 1];
#pragma unroll
          for (int rb = 0; rb < kRB; ++rb)
            d.v[rb] = mma(xo, u32x4_t{e.e[rb][0].x, e.e[rb][0].y, e.e[rb][1].x, e.e[rb][1].y}, d.v[rb]);
        });
      });
      flush(y, d, sc, g);
    });
  }
}

// ---------------------------------------------------------------- 3-bit
// A group is 48 bytes = four 96-bit triples of 32 codes.  Lane q decodes triple
// q of its row (three aligned dwords, each inside one chunk); window w takes
// fields 4w .. 4w+3 (codes 32q + 8w ..), whose x dwords are 16q + 4w .. + 3
// (byte offset 256 g + 64 q + 16 w of the token row).
// Group pairs [k0, k1) of the slab's rows (groups 2 k0 .. min(2 k1, G) - 1).
__device__ void run_i3(const uint8_t* codes, const uint16_t* scales, const XSrc& xs, int k0, int k1, int G, int lane,
                       const uint8_t* lut, Acc& y) {
  const int g0 = 2 * k0, g1 = 2 * k1 < G ? 2 * k1 : G;
  Scales sc(scales, g0, g1, lane);
  const int nchunks = 3 * g1;
  const CodeDw src(codes, nchunks, lane);
  const int q = lane >> 4;
  const uint32_t i3_off = i3_lane_off(lane);
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
  // triples of group g in slot g % 2, one group ahead; table entries one window
  // ahead
  struct E3 {
    uint32_t e[kRB][4];
  };
  auto read = [&](E3& b, const uint32_t (&t)[kRB][3], auto w_) __attribute__((always_inline)) {
    constexpr int W = decltype(w_)::value;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const uint32_t w0 = t[rb][0], w1 = t[rb][1], w2 = t[rb][2];
      b.e[rb][0] = lds_b32(lut + kI3Lut + i3_addr<4 * W + 0>(w0, w1, w2, i3_off));
      b.e[rb][1] = lds_b32(lut + kI3Lut + i3_addr<4 * W + 1>(w0, w1, w2, i3_off));
      b.e[rb][2] = lds_b32(lut + kI3Lut + i3_addr<4 * W + 2>(w0, w1, w2, i3_off));
      b.e[rb][3] = lds_b32(lut + kI3Lut + i3_addr<4 * W + 3>(w0, w1, w2, i3_off));
    }
  };
  uint32_t tw[2][kRB][3];
  load_tr(g0, tw[0]);
  // x of window wi (global: 4 g + W) in slot wi % 4, three windows ahead
  u32x4_t xw[4];
  auto xoff3 = [&](int wi) __attribute__((always_inline)) { return (uint32_t)(256 * (wi >> 2) + 64 * q + 16 * (wi & 3)); };
#pragma unroll
  for (int i = 0; i < 3; ++i) xw[i] = xs.b128(xoff3(4 * g0 + i));
  E3 ent[2];
  read(ent[0], tw[0], std::integral_constant<int, 0>{});
  for (int k = k0; k < k1; ++k) {  // an odd last group runs past the row and is dropped by flush
    sfor<2>([&](auto s_) __attribute__((always_inline)) {
      constexpr int S = decltype(s_)::value;
      const int g = 2 * k + S;
      sched_fence();
      load_tr(g + 1, tw[S ^ 1]);
      Acc d;
      zero(d);
      sfor<4>([&](auto w_) __attribute__((always_inline)) {
        constexpr int W = decltype(w_)::value;
        constexpr int WI = 4 * S + W;
        xw[(W + 3) & 3] = xs.b128(xoff3(4 * g + W + 3));
        if constexpr (W < 3)
          read(ent[(WI + 1) & 1], tw[S], std::integral_constant<int, W + 1>{});
        else
          read(ent[(WI + 1) & 1], tw[S ^ 1], std::integral_constant<int, 0>{});
        const u32x4_t xo = xw[W];
        const E3& e = ent[WI & 1];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          d.v[rb] = mma(xo, u32x4_t{e.e[rb][0], e.e[rb][1], e.e[rb][2], e.e[rb][3]}, d.v[rb]);
      });
      flush(y, d, sc, g);
    });
  }
}

// One task: one 64-row slab of one descriptor (or one part of its input when
// the entry is split), all M tokens.
__device__ __forceinline__ void mm_task(const ql_gemv_desc* __restrict__ descs, int count, int64_t t, int M,
                                        const uint8_t* lut, int lane, uint32_t* state) {
  const ql_gemv_desc& d = descs[find_desc(descs, count, t)];
  if (!task_in_entry(d, t)) return;
  const SplitTask st(d, t);
  const int K = d.K, G = K / kGroup, G8 = (G + 7) / 8;
  int gr;
  const int64_t off = slab_offset(st.slab, K, d.grid, d.blk_grid, d.blk_off, &gr);
  const uint8_t* codes = static_cast<const uint8_t*>(d.packed) + off;
  const uint16_t* scales = d.pscales + (int64_t)st.slab * G8 * kSlab * 8;
  const XSrc xs(d.x, M, K, lane);
  Acc y;
  zero(y);
  if (gr == QL_GRID_T)
    run_t(codes, scales, xs, K, G, st.p0(K), st.p1(K), lane, lut, y);
  else if (gr == QL_GRID_I2)
    run_i2(codes, scales, xs, st.k0(K), st.k1(K), G, lane, lut, y);
  else
    run_i3(codes, scales, xs, st.k0(K), st.k1(K), G, lane, lut, y);
  const int q = lane >> 4;
  if (st.split()) {
    float* sl = st.slots(d, state);
    // partial sum (rb, i) of lane l at word (4 rb + i) * 64 + l of the part's
    // slot; lanes whose tokens are all past M hold nothing and skip the exchange
    float v[4 * kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[4 * rb + i] = y.v[rb][i];
    if (4 * q < M)
#pragma unroll
      for (int j = 0; j < 4 * kRB; ++j) st.put(sl, 64 * j + lane, v[j]);
    if (!st.arrive(st.counter(d, state), lane)) return;
    if (4 * q < M) st.totals<4 * kRB, 4>(sl, v, lane);
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) y.v[rb][i] = v[4 * rb + i];
  }
  // lane l: tokens 4q .. 4q+3 of weight row 16 rb + (l & 15)
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int64_t row = (int64_t)st.slab * kSlab + 16 * rb + (lane & 15);
    if (row < d.N)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * q + i < M) d.y[(int64_t)(4 * q + i) * d.N + row] = y.v[rb][i];
  }
}

__global__ void __launch_bounds__(kMmWaves * 64, QL_MM_WAVES_PER_EU) gemv_mm_grouped_kernel(const ql_gemv_desc* __restrict__ descs,
                                                                         int count, int64_t total, int M,
                                                                         uint32_t* __restrict__ sched) {
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLutBytes];
  build_luts<kMmWaves * 64>(lut);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  TaskQueues tq(sched, total, (int64_t)gridDim.x * kMmWaves);
  int64_t t = (int64_t)blockIdx.x * kMmWaves + wave;
  if (t >= total) t = tq.next(lane);
  while (t >= 0) {
    const uint32_t claim = tq.claim(lane);
    mm_task(descs, count, t, M, lut, lane, sched);
    t = tq.resolve(claim, lane);
  }
  tq.checkout(lane);
}

}  // namespace

int64_t mm_wave_slots() { return (int64_t)device_cu_count() * kMmWgPerCu * kMmWaves; }

hipError_t launch_gemv_mm_grouped(const ql_gemv_desc* descs, int32_t count, int64_t total_tasks, int M,
                                  uint32_t* sched, hipStream_t stream) {
  if (M < 2 || M > 16) return hipErrorInvalidValue;
  const int slots = device_cu_count() * kMmWgPerCu;
  const int64_t wg_needed = (total_tasks + kMmWaves - 1) / kMmWaves;
  const int grid = (int)(wg_needed < slots ? wg_needed : slots);
  hipLaunchKernelGGL(gemv_mm_grouped_kernel, dim3(grid), dim3(kMmWaves * 64), 0, stream, descs, count, total_tasks, M,
                     sched);
  return hipGetLastError();
}

}  // namespace ql
