// Decode-time GEMV, 1 <= M <= 16 tokens, over ThinkBit-packed weights (gfx950):
// one lane per weight row, codes decoded through per-lane LDS tables, products
// on the matrix cores.  One kernel serves a single matrix (qlinear_gemv) and
// the grouped pass (qlinear_gemv_grouped).
//
// A decode step at a small batch is still one pass over the weights: each
// packed byte is read once and used by every token (ThinkBit summary page,
// onedev.kr/papers/1416, section "What it is"; w = c * s with one bf16 scale
// per 128 inputs, section "How it works").
//
// Mapping.  One wave owns a 64-row slab and lane r is row r: it streams its
// row's code bytes and turns them into bf16 codes with per-lane LDS tables.  The products run on
// v_mfma_f32_4x4x4_16b_bf16, whose 64 lanes form 16 blocks of four: lane
// 4b + j supplies four inputs of weight row 4b + j (the second operand, so
// lane = row holds) and receives the four token sums of that row.  The first
// operand, x (4 tokens x 4 inputs), is broadcast from one block to all sixteen
// (CBSZ = 4, ABID = the source block), so per 128-input group one 16-byte load
// per lane holds every activation the group needs: lane 4b + t holds token t's
// inputs 8b .. 8b+7, and MFMA j of the group (inputs 4j .. 4j+3) takes block
// j / 2, half j % 2.  Tokens past M read as zero.  Up to 16 tokens run as
// token groups of four: every code operand feeds one MFMA per group.
//
// Per stored byte the VALU issues only the table address (and, for ternary,
// one OR per byte pair and the copies that pair operands across entries); the
// products leave the VALU entirely.
//
// Decode operands (four consecutive inputs per MFMA):
//   ternary: a byte pair covers 10 inputs.  The table entry of a byte is
//            (d0,d1) (d2,d3) (d4,0) (0,d4); with the stored digit order the
//            even byte E covers inputs 0..4 and the odd byte O inputs 6..9 and
//            5, so two pairs (20 inputs) are five MFMAs:
//              (E1.x, E1.y) (E1.z|O1.w, O1.x) (O1.y, E2.x) (E2.y, E2.z|O2.w) (O2.x, O2.y);
//   2-bit:   one byte = four codes = one MFMA (8-byte entry);
//   3-bit:   two 6-bit fields = four codes = one MFMA (two 4-byte entries).
// Group edges (every 128 inputs) fall on MFMA boundaries in all three grids,
// so each group is summed by its own MFMA chains and scaled once, in fp32.
#include "ql_internal.hpp"
#include "ql_luts.hpp"
#include "ql_stream.hpp"

namespace ql {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Token groups: TG groups of four tokens (M <= 4 TG), one MFMA per group per code
// operand, all against the same decoded codes.  Up to two groups the kernel keeps
// the batch-1 occupancy (8-wave workgroups, 4 waves per SIMD); three and four
// groups need more registers for activations and sums (6-wave workgroups, 3 per SIMD).
constexpr int gemv_waves(int TG) { return TG <= 2 ? 8 : 6; }
constexpr int gemv_waves_per_eu(int TG) { return TG <= 2 ? 4 : 3; }
constexpr int kWgPerCu = 2;  // resident workgroups per CU (LDS tables: 77 KB each)
constexpr int kMaxTG = 4;
static_assert(4 * kMaxTG * 64 <= kPartWords, "a split part stores 16 tokens per lane");
// MFMA chains per token group within one 128-input group: one group of tokens
// alternates two chains, so that consecutive MFMAs do not wait on each other;
// with several token groups their chains interleave instead.
constexpr int gemv_chains(int TG) { return TG == 1 ? 2 : 1; }

// acc + x(block ABID, broadcast) * codes(lane's row): one MFMA of four inputs.
template <int ABID>
__device__ __forceinline__ f32x4_t mma4(uint32_t x0, uint32_t x1, uint32_t c0, uint32_t c1, const f32x4_t& acc) {
  const u32x2_t a = {x0, x1}, b = {c0, c1};
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), acc, 4,
                                                ABID, 0);
}

// Sums of one 128-input group: chain c of token group tg.
template <int TG>
struct Chains {
  f32x4_t v[TG][gemv_chains(TG)];
};

// MFMA jj (0..31) of a group, for every token group: x half jj % 2 of block
// jj / 2, into chain jj % chains; the first MFMA of each chain starts from zero.
template <int TG, int JJ>
__device__ __forceinline__ void group_mma(const u32x4_t (&xg)[TG], uint32_t c0, uint32_t c1, Chains<TG>& ch) {
  constexpr int NC = gemv_chains(TG);
  constexpr f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int tg = 0; tg < TG; ++tg) {
    const uint32_t x0 = (JJ & 1) ? xg[tg].z : xg[tg].x, x1 = (JJ & 1) ? xg[tg].w : xg[tg].y;
    ch.v[tg][JJ % NC] = mma4<(JJ >> 1)>(x0, x1, c0, c1, JJ < NC ? z : ch.v[tg][JJ % NC]);
  }
}

// y[4 tg + t] += s * (sum of token group tg's chains), token t = component t.
template <int TG>
__device__ __forceinline__ void flush(float s, const Chains<TG>& ch, float (&y)[4 * TG]) {
#pragma unroll
  for (int tg = 0; tg < TG; ++tg)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float v = ch.v[tg][0][t];
#pragma unroll
      for (int c = 1; c < gemv_chains(TG); ++c) v += ch.v[tg][c][t];
      y[4 * tg + t] = fmaf(s, v, y[4 * tg + t]);
    }
}

// Activations: token 4 tg + (lane & 3) of the M x K bf16 batch, inputs
// 8 (lane >> 2) .. +7 of each 128-input group.  Tokens past M, and groups at
// or past G, read as zero through the buffer's range check.
template <int TG>
struct XSrc {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t base;  // token (lane & 3) of token group 0
  int M, G, K;
  __device__ __forceinline__ XSrc(const uint16_t* x, int M_, int K_, int lane)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(uniform_ptr(x), (short)0,
                                               __builtin_amdgcn_readfirstlane(2 * M_ * K_), 0x00020000)),
        M(M_), G(K_ / kGroup), K(K_) {
    base = (uint32_t)(2 * (lane & 3) * K) + 16u * (uint32_t)(lane >> 2);
  }
  // token group tg's x of group g (tokens past M land past the buffer's range)
  __device__ __forceinline__ u32x4_t load(int g, int tg) const {
    const uint32_t off = g < G ? 256u * (uint32_t)g + (uint32_t)(8 * tg * K) : 0x80000000u;
    const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, base + off, 0, 0);
    return u32x4_t{(uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w};
  }
  __device__ __forceinline__ void group(u32x4_t (&xg)[TG], int g) const {
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) xg[tg] = load(g, tg);
  }
};

template <int TG>
struct Ctx {
  const uint8_t* codes;    // slab base
  const uint16_t* scales;  // slab's scale block
  XSrc<TG> xs;
  int K, G, lane;
  const uint8_t* lut;
};

// ---------------------------------------------------------------- ternary
// A 640-input period = 8 chunks = 128 bytes per row = 160 MFMAs = 5 groups;
// a unit is kTU bytes (kTU / 4 quads of 20 inputs, five MFMAs each).
#ifndef QL_T_UNIT
#define QL_T_UNIT 4
#endif
constexpr int kTU = QL_T_UNIT;                // bytes per unit (whole 4-byte quads)
constexpr int kTUnits = 128 / kTU;
constexpr int kTMfma = 5 * kTU / 4;           // MFMAs per unit
static_assert(kTU % 4 == 0 && 128 % kTU == 0, "units of whole quads");

struct TEnt {
  u32x4_t e[kTU];
};

template <int U, int R>
__device__ __forceinline__ void t_lds(TEnt& b, const uint4 (&d)[R], uint32_t lane_off, const uint8_t* lut) {
  sfor<kTU>([&](auto bi) __attribute__((always_inline)) {
    constexpr int j = U * kTU + decltype(bi)::value;  // byte within the period
    const uint32_t w = word_of(d[(j >> 4) % R], (j & 15) >> 2);
    const uint32_t addr = __builtin_amdgcn_perm(w, lane_off, 0x0C0C0000u | ((4u + (j & 3)) << 8));
    b.e[decltype(bi)::value] = lds_b128(lut + kTLut + addr);
  });
}

// Code operand of MFMA M5 (0..4) of quad Q (0, 1) of a unit.
template <int Q, int M5>
__device__ __forceinline__ u32x2_t t_code(const TEnt& b) {
  const u32x4_t& E1 = b.e[4 * Q];
  const u32x4_t& O1 = b.e[4 * Q + 1];
  const u32x4_t& E2 = b.e[4 * Q + 2];
  const u32x4_t& O2 = b.e[4 * Q + 3];
  if constexpr (M5 == 0) return u32x2_t{E1.x, E1.y};
  if constexpr (M5 == 1) return u32x2_t{E1.z | O1.w, O1.x};
  if constexpr (M5 == 2) return u32x2_t{O1.y, E2.x};
  if constexpr (M5 == 3) return u32x2_t{E2.y, E2.z | O2.w};
  return u32x2_t{O2.x, O2.y};
}

// The five scales of a period whose first group sits at position S0 of its
// 8-group scale block (sa: that block, sb: the first half of the next).
template <int S0>
__device__ __forceinline__ void t_pick(const u32x4_t& sa, const u32x2_t& sb, int g_left, float (&sc)[5]) {
  sfor<5>([&](auto gl_) __attribute__((always_inline)) {
    constexpr int gl = decltype(gl_)::value, q = S0 + gl;
    const uint32_t w = q < 8 ? sa[q >> 1] : sb[(q - 8) >> 1];
    sc[gl] = gl < g_left ? scale_of_pair<q & 1>(w) : 0.0f;
  });
}

__device__ __forceinline__ void t_scales(const u32x4_t& sa, const u32x2_t& sb, int s0, int g_left, float (&sc)[5]) {
  switch (s0) {
    case 0: t_pick<0>(sa, sb, g_left, sc); break;
    case 1: t_pick<1>(sa, sb, g_left, sc); break;
    case 2: t_pick<2>(sa, sb, g_left, sc); break;
    case 3: t_pick<3>(sa, sb, g_left, sc); break;
    case 4: t_pick<4>(sa, sb, g_left, sc); break;
    case 5: t_pick<5>(sa, sb, g_left, sc); break;
    case 6: t_pick<6>(sa, sb, g_left, sc); break;
    default: t_pick<7>(sa, sb, g_left, sc); break;
  }
}

#ifndef QL_T_RING
#define QL_T_RING 4
#endif

// Periods p0..p1-1 of the slab (the last may be partial).
template <int TG>
__device__ void run_t(const Ctx<TG>& c, int p0, int p1, float (&y)[4 * TG]) {
  if (p0 >= p1) return;
  const int nchunks = (c.K + 79) / 80;
  const bool last_half = nchunks - 8 * (p1 - 1) <= 4;  // the row ends in the first half of period p1 - 1
  uint32_t lane_off = (uint32_t)(c.lane & 15) << 4;
  const ChunkSrc src(c.codes, nchunks < 8 * p1 ? nchunks : 8 * p1, c.lane);
  constexpr int R = QL_T_RING;
  static_assert(8 % R == 0, "the ring must divide a period's 8 chunks");
  uint4 d[R];
  sfor<R>([&](auto ch) __attribute__((always_inline)) { d[decltype(ch)::value] = src.load(8 * p0 + decltype(ch)::value); });
  const int G8 = (c.G + 7) >> 3;
  // scale blocks of period p0 (later periods: loaded one period ahead)
  u32x4_t sa = ld_scale_blk(c.scales, (5 * p0) >> 3, c.lane);
  u32x2_t sb = ld_scale_blk_lo(c.scales, ((5 * p0) >> 3) + 1 < G8 ? ((5 * p0) >> 3) + 1 : (5 * p0) >> 3, c.lane);
  // x of group gl of the period lives in xg[gl & 1]; group 5 (the next
  // period's group 0) lands in xg[1] and moves to xg[0] at the period's end
  u32x4_t xg[2][TG];
  c.xs.group(xg[0], 5 * p0);
  TEnt A, B;
  t_lds<0, R>(A, d, lane_off, c.lut);
  lgkm_wait0();
  for (int p = p0; p < p1; ++p) {
    const bool more = p + 1 < p1;
    float sc[5];
    Chains<TG> ch;
    auto step = [&](auto u) __attribute__((always_inline)) {
      constexpr int U = decltype(u)::value;
      constexpr bool odd = (U & 1) != 0;
      auto& cur = odd ? B : A;
      auto& nxt = odd ? A : B;
      __builtin_amdgcn_s_setprio(1);
      if constexpr (U + 1 < kTUnits) {
        t_lds<U + 1, R>(nxt, d, lane_off, c.lut);
        constexpr int last_byte = (U + 1) * kTU + kTU - 1;
        if constexpr ((last_byte & 15) == 15) {
          constexpr int chn = last_byte >> 4;
          d[chn % R] = src.load(chn + R < 8 ? 8 * p + chn + R : 8 * (p + 1) + chn + R - 8);
        }
      } else {
        if (more) t_lds<0, R>(nxt, d, lane_off, c.lut);
      }
      __builtin_amdgcn_s_setprio(0);
      sched_fence();
      sfor<kTMfma>([&](auto m_) __attribute__((always_inline)) {
        constexpr int m = decltype(m_)::value;
        constexpr int j = kTMfma * U + m;  // MFMA within the period
        constexpr int gl = j / 32, jj = j % 32;
        if constexpr (jj == 0) c.xs.group(xg[(gl + 1) & 1], 5 * p + gl + 1);  // next group's x
        const u32x2_t cv = t_code<m / 5, m % 5>(cur);
        group_mma<TG, jj>(xg[gl & 1], cv.x, cv.y, ch);
        if constexpr (j == 31) {
          // the period's scales, needed from here on; then the next period's blocks
          // (loaded a period ahead, so the first flush of a period never waits on them)
          t_scales(sa, sb, (5 * p) & 7, c.G - 5 * p, sc);
          const int bn = (5 * (more ? p + 1 : p)) >> 3;
          sa = ld_scale_blk(c.scales, bn, c.lane);
          sb = ld_scale_blk_lo(c.scales, bn + 1 < G8 ? bn + 1 : bn, c.lane);
        }
        if constexpr (jj == 31) flush(sc[gl], ch, y);
      });
      after(lane_off, y);
      sched_fence();
      lgkm_wait0();
    };
    sfor<kTUnits / 2>(step);
    if (more || !last_half) sfor_from<kTUnits / 2, kTUnits / 2>(step);
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) xg[0][tg] = xg[1][tg];
  }
}

// ---------------------------------------------------------------- 2-bit
// A group is 32 bytes = 2 chunks = 32 MFMAs; a unit is 8 bytes.
struct I2E {
  u32x2_t e[8];
};

// ring: 4 chunks = 2 groups; group slot S holds chunks 2S, 2S+1
template <int S, int U>
__device__ __forceinline__ void i2_lds(I2E& b, const uint4 (&d)[4], uint32_t lane_off, const uint8_t* lut) {
  sfor<8>([&](auto bi) __attribute__((always_inline)) {
    constexpr int j = U * 8 + decltype(bi)::value;  // byte within the group
    const uint32_t w = word_of(d[2 * S + (j >> 4)], (j & 15) >> 2);
    const uint32_t bv = (w >> (8 * (j & 3))) & 0xFFu;
    b.e[decltype(bi)::value] = lds_b64(lut + kI2Lut + ((bv << 5) | lane_off));
  });
}

template <int TG>
__device__ void run_i2(const Ctx<TG>& c, int g0, int g1, float (&y)[4 * TG]) {
  if (g0 >= g1) return;
  uint32_t lane_off = (uint32_t)(c.lane & 3) << 3;
  const ChunkSrc src(c.codes, 2 * g1, c.lane);
  uint4 d[4];
  sfor<4>([&](auto q) __attribute__((always_inline)) { d[decltype(q)::value] = src.load(2 * g0 + decltype(q)::value); });
  u32x4_t xg[2][TG];
  c.xs.group(xg[0], g0);
  I2E A, B;
  i2_lds<0, 0>(A, d, lane_off, c.lut);
  lgkm_wait0();
  for (int gb = g0; gb < g1; gb += 2) {
    sfor<2>([&](auto s_) __attribute__((always_inline)) {
      constexpr int S = decltype(s_)::value;
      const int g = gb + S;
      if (g < g1) {
        const float sc = ld_scale(c.scales, g, c.lane);
        c.xs.group(xg[S ^ 1], g + 1);
        const bool more = g + 1 < g1;
        Chains<TG> ch;
        sfor<4>([&](auto u) __attribute__((always_inline)) {
          constexpr int U = decltype(u)::value;
          constexpr bool even = ((4 * S + U) & 1) == 0;  // buffer of this unit
          auto& cur = even ? A : B;
          auto& nxt = even ? B : A;
          if constexpr (U + 1 < 4) {
            i2_lds<S, U + 1>(nxt, d, lane_off, c.lut);
          } else {
            if (more) i2_lds<S ^ 1, 0>(nxt, d, lane_off, c.lut);
            // every byte of this group is addressed: its slot takes group g + 2
            d[2 * S] = src.load(2 * (g + 2));
            d[2 * S + 1] = src.load(2 * (g + 2) + 1);
          }
          sched_fence();
          sfor<8>([&](auto bi) __attribute__((always_inline)) {
            constexpr int jj = 8 * U + decltype(bi)::value;
            group_mma<TG, jj>(xg[S], cur.e[decltype(bi)::value].x, cur.e[decltype(bi)::value].y, ch);
          });
          after(lane_off, y);
          sched_fence();
          lgkm_wait0();
        });
        flush(sc, ch, y);
      }
    });
  }
}

// ---------------------------------------------------------------- 3-bit
// A group is 4 triples (96 bits = 32 codes each) = 3 chunks = 32 MFMAs; a unit
// is one triple (16 six-bit fields, 8 MFMAs).
struct I3E {
  uint32_t e[16];
};

// triple U of group slot S: words 3U..3U+2 of the slot's 3 chunks
template <int S, int U>
__device__ __forceinline__ void i3_lds(I3E& b, const uint4 (&d)[6], const uint8_t* lut, uint32_t tok,
                                       uint32_t lane_off) {
  constexpr int wb = 3 * U;
  uint32_t w0 = word_of(d[3 * S + (wb >> 2)], wb & 3);
  uint32_t w1 = word_of(d[3 * S + ((wb + 1) >> 2)], (wb + 1) & 3);
  uint32_t w2 = word_of(d[3 * S + ((wb + 2) >> 2)], (wb + 2) & 3);
  asm volatile("" : "+v"(w0), "+v"(w1), "+v"(w2) : "v"(tok));  // table reads stay in this step
  sfor<16>([&](auto pi) __attribute__((always_inline)) {
    constexpr int P = decltype(pi)::value;
    b.e[P] = lds_b32(lut + kI3Lut + i3_addr<P>(w0, w1, w2, lane_off));
  });
}

template <int TG>
__device__ void run_i3(const Ctx<TG>& c, int g0, int g1, float (&y)[4 * TG]) {
  if (g0 >= g1) return;
  const ChunkSrc src(c.codes, 3 * g1, c.lane);
  uint4 d[6];
  sfor<6>([&](auto q) __attribute__((always_inline)) { d[decltype(q)::value] = src.load(3 * g0 + decltype(q)::value); });
  u32x4_t xg[2][TG];
  c.xs.group(xg[0], g0);
  const uint32_t lane_off = i3_lane_off(c.lane);
  uint32_t tok = 0;  // step token: rewritten (as far as the compiler knows) after each step's arithmetic
  I3E A, B;
  i3_lds<0, 0>(A, d, c.lut, tok, lane_off);
  lgkm_wait0();
  for (int gb = g0; gb < g1; gb += 2) {
    sfor<2>([&](auto s_) __attribute__((always_inline)) {
      constexpr int S = decltype(s_)::value;
      const int g = gb + S;
      if (g < g1) {
        const float sc = ld_scale(c.scales, g, c.lane);
        c.xs.group(xg[S ^ 1], g + 1);
        const bool more = g + 1 < g1;
        Chains<TG> ch;
        sfor<4>([&](auto u) __attribute__((always_inline)) {
          constexpr int U = decltype(u)::value;
          constexpr bool even = ((4 * S + U) & 1) == 0;
          auto& cur = even ? A : B;
          auto& nxt = even ? B : A;
          __builtin_amdgcn_s_setprio(1);
          if constexpr (U + 1 < 4) {
            i3_lds<S, U + 1>(nxt, d, c.lut, tok, lane_off);
          } else {
            if (more) i3_lds<S ^ 1, 0>(nxt, d, c.lut, tok, lane_off);
#pragma unroll
            for (int q = 0; q < 3; ++q) d[3 * S + q] = src.load(3 * (g + 2) + q);
          }
          __builtin_amdgcn_s_setprio(0);
          sched_fence();
          sfor<8>([&](auto m_) __attribute__((always_inline)) {
            constexpr int m = decltype(m_)::value;
            constexpr int jj = 8 * U + m;
            group_mma<TG, jj>(xg[S], cur.e[2 * m], cur.e[2 * m + 1], ch);
          });
          after(tok, y);
          sched_fence();
          lgkm_wait0();
        });
        flush(sc, ch, y);
      }
    });
  }
}

// ---------------------------------------------------------------- task, kernel
// One wave task: one 64-row slab of one descriptor, all tokens, or one part of
// its input when the entry is split (partial sums meet in the state buffer).
// `done` runs once the sums are complete and before anything is stored: the
// grouped launch reads its next task's draw there, so that wait (which covers
// every vector memory operation in flight) does not also wait for this task's
// stores to reach memory.
template <int TG, class Done>
__device__ __forceinline__ void gemv_task(const ql_gemv_desc* __restrict__ descs, const TaskLoc& loc, int64_t t, int M,
                                          const uint8_t* lut, int lane, uint32_t* state, Done&& done) {
  constexpr int NT = 4 * TG;
  const ql_gemv_desc& d = descs[loc.di];
  if (!task_in_entry(d, t)) return done();
  const SplitTask st(d, t);
  const int K = d.K, G = K / kGroup, G8 = (G + 7) / 8;
  float y[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) y[i] = 0.0f;
  const Ctx<TG> c{static_cast<const uint8_t*>(d.packed) + loc.off, d.pscales + st.slab * (int64_t)G8 * kSlab * 8,
                  XSrc<TG>(d.x, M, K, lane), K, G, lane, lut};
  if (loc.gr == QL_GRID_T) {
    run_t<TG>(c, st.p0(K), st.p1(K), y);
  } else {
    const int k0 = st.k0(K), k1 = st.k1(K);
    const int g0 = 2 * k0, g1 = (2 * k1 < G) ? 2 * k1 : G;
    if (loc.gr == QL_GRID_I2)
      run_i2<TG>(c, g0, g1, y);
    else
      run_i3<TG>(c, g0, g1, y);
  }
  done();
  if (st.split()) {
    float* sl = st.slots(d, state);
#pragma unroll
    for (int i = 0; i < NT; ++i) st.put(sl, 64 * i + lane, y[i]);  // all slots, straight-line before the wait
    if (!st.arrive(st.counter(d, state), lane)) return;
    st.totals<NT, (NT == 4 ? 8 : 4)>(sl, y, lane);  // 8 parts per load round at batch <= 4
  }
  const int64_t row = (int64_t)st.slab * kSlab + lane;
  // a global store (a flat one would also hold up the next task's lgkmcnt waits)
  typedef __attribute__((address_space(1))) float* gf32p;
  if (row < d.N)
#pragma unroll
    for (int i = 0; i < NT; ++i)
      if (i < M) ((gf32p)d.y)[(int64_t)i * d.N + row] = y[i];
}

// A single matrix: all slabs cost the same, so waves stride over them (no task
// queues, no split).  The descriptor travels in the kernel arguments; `count`
// (always 1) is a runtime value so its reads stay inside the task loop instead
// of being hoisted and kept live across it.
template <int TG>
__global__ void __launch_bounds__(gemv_waves(TG) * 64, gemv_waves_per_eu(TG)) gemv_kernel(ql_gemv_desc desc, int count,
                                                                                       int64_t total, int M) {
  constexpr int kWaves = gemv_waves(TG);
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLutBytes];
  build_luts<kWaves * 64>(lut);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t < total; t += (int64_t)gridDim.x * kWaves)
    gemv_task<TG>(&desc, locate_task(&desc, count, t), t, M, lut, lane, nullptr, [] {});
}

// Many independent matrices in one persistent launch.  Slab costs differ (row
// length, grid), so after its first task a wave keeps drawing tasks from the
// task queues: list scheduling over tasks that the host numbered longest-first.
// The next task is drawn when the current one starts and read when it ends, so
// the atomic's round trip is hidden behind the task instead of stalling the
// wave between tasks; a wave then holds at most one task ahead, which costs
// little balance because the last tasks are the shortest.  The first task's
// descriptor loads are in flight while the tables are built.
template <int TG>
__global__ void __launch_bounds__(gemv_waves(TG) * 64, gemv_waves_per_eu(TG)) gemv_grouped_kernel(
    const ql_gemv_desc* __restrict__ descs, int count, int64_t total, int M, uint32_t* __restrict__ sched) {
  constexpr int kWaves = gemv_waves(TG);
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLutBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int64_t t = (int64_t)blockIdx.x * kWaves + wave;
  const TaskLoc first = locate_task(descs, count, t < total ? t : total - 1);
  build_luts<kWaves * 64>(lut);
  __syncthreads();
  TaskQueues tq(sched, total, (int64_t)gridDim.x * kWaves);
  TaskLoc loc = first;
  if (t >= total) {
    t = tq.next(lane);
    if (t >= 0) loc = locate_task(descs, count, t);
  }
  while (t >= 0) {
    const uint32_t claim = tq.claim(lane);
    int64_t tn = -1;
    gemv_task<TG>(descs, loc, t, M, lut, lane, sched, [&]() __attribute__((always_inline)) { tn = tq.drawn(claim); });
    if (tn < 0) tn = tq.next(lane);  // the home queue was dry: scan the others
    t = tn;
    if (t >= 0) loc = locate_task(descs, count, t);
  }
  tq.checkout(lane);
}

}  // namespace

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

int64_t grouped_wave_slots(int M) {
  return (int64_t)device_cu_count() * kWgPerCu * gemv_waves((M + 3) / 4);
}

template <int TG>
static hipError_t launch_tg(const ql_gemv_desc* descs, int32_t count, int64_t total_tasks, int M, uint32_t* sched,
                            hipStream_t stream) {
  constexpr int W = gemv_waves(TG);
  const int slots = device_cu_count() * kWgPerCu;
  const int64_t wg_needed = (total_tasks + W - 1) / W;
  const int grid = (int)(wg_needed < slots ? wg_needed : slots);
  hipLaunchKernelGGL(gemv_grouped_kernel<TG>, dim3(grid), dim3(W * 64), 0, stream, descs, count, total_tasks, M,
                     sched);
  return hipGetLastError();
}

hipError_t launch_gemv_grouped(const ql_gemv_desc* descs, int32_t count, int64_t total_tasks, int M,
                                  uint32_t* sched, hipStream_t stream) {
  switch ((M + 3) / 4) {
    case 1: return launch_tg<1>(descs, count, total_tasks, M, sched, stream);
    case 2: return launch_tg<2>(descs, count, total_tasks, M, sched, stream);
    case 3: return launch_tg<3>(descs, count, total_tasks, M, sched, stream);
    case 4: return launch_tg<4>(descs, count, total_tasks, M, sched, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int TG>
static hipError_t launch_single_tg(const ql_gemv_desc& d, int M, hipStream_t stream) {
  constexpr int W = gemv_waves(TG);
  const int64_t nslabs = ((int64_t)d.N + kSlab - 1) / kSlab;
  const int slots = device_cu_count() * kWgPerCu;
  const int64_t wg_needed = (nslabs + W - 1) / W;
  const int grid = (int)(wg_needed < slots ? wg_needed : slots);
  hipLaunchKernelGGL(gemv_kernel<TG>, dim3(grid), dim3(W * 64), 0, stream, d, 1, nslabs, M);
  return hipGetLastError();
}

hipError_t launch_gemv(const MatArgs& a, int M, hipStream_t stream) {
  const ql_gemv_desc d{a.packed, a.pscales, a.blk_grid, a.blk_off, a.x, a.y, a.N, a.K, a.grid, 0, 1, 0, 0};
  switch ((M + 3) / 4) {
    case 1: return launch_single_tg<1>(d, M, stream);
    case 2: return launch_single_tg<2>(d, M, stream);
    case 3: return launch_single_tg<3>(d, M, stream);
    case 4: return launch_single_tg<4>(d, M, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ql
