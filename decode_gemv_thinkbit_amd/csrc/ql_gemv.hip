// Decode-time batch-1 GEMV over ThinkBit-packed weights on gfx950 (the drivers
// are templated on the token count; only M = 1 is instantiated).
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
#include "ql_internal.hpp"
#include "ql_stream.hpp"
#include "ql_luts.hpp"

namespace ql {

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

typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

// {high half of lo, low half of hi} of two uniform words, as a two-lane 16-bit
// vector so that it lowers to s_pack_ll_b32_b16 on the scalar unit.
__device__ __forceinline__ uint32_t pack_hi_lo(uint32_t lo, uint32_t hi) {
  const u16x2_t v = {(uint16_t)(lo >> 16), (uint16_t)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// (x_k, x_{k+1}) as a bf16 pair; odd k is re-aligned on the scalar unit.
template <int K0, bool GUARD>
__device__ __forceinline__ uint32_t xpair(cu32p xb, int kleft) {
  if constexpr ((K0 & 1) == 0) {
    return xdw<GUARD>(xb, K0 >> 1, kleft);
  } else {
    return pack_hi_lo(xdw<GUARD>(xb, (K0 - 1) >> 1, kleft), xdw<GUARD>(xb, (K0 + 1) >> 1, kleft));
  }
}

// ---------------------------------------------------------------- per-slab drivers
//
// Software pipeline.  A slab row is consumed in units (M = 1: 8 bytes per lane).
// Issuing a unit starts its LDS table reads and its scalar x loads; the unit
// before it is then multiplied (dot2) and a single lgkmcnt(0) wait closes the
// step.  Scalar loads may return out of order, so a wait on a partial count is
// impossible while they are in flight; ordering "issue next, compute current,
// wait" overlaps both latencies with the current unit's arithmetic instead.
// Code chunks stream through a ring of 128-bit registers (ternary: 4 chunks;
// 2-bit: 2 groups = 4 chunks; 3-bit: 2 groups = 6 chunks), each slot reloaded
// as soon as its last byte has been turned into table addresses.

template <int M>
struct SlabCtx {
  const uint8_t* codes;      // slab base
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

// pair (x_k, x_k+1) from a dword window whose first element is input KK = 0
template <int KK, int XD>
__device__ __forceinline__ uint32_t wpair(const uint32_t (&x)[XD]) {
  if constexpr ((KK & 1) == 0) {
    return x[KK >> 1];
  } else {
    return pack_hi_lo(x[(KK - 1) >> 1], x[(KK + 1) >> 1]);
  }
}

// ---------------------------------------------------------------- ternary units
// The table entry of a stored byte holds its digits as bf16 codes in digit
// order: (d0,d1), (d2,d3), (d4,0), (0,d4).  With the layout's digit order, a
// byte pair covering inputs k..k+9 (k = 10q) multiplies
//   even byte: .x (x_k, x_k+1)  .y (x_k+2, x_k+3)  .z (x_k+4, x_k+5)
//   odd byte:  .x (x_k+6, x_k+7)  .y (x_k+8, x_k+9)  .w (x_k+4, x_k+5)
// so every activation operand is an aligned dword straight from the scalar
// loads, and no dword straddles a 128-input group edge (the edges are even).
//
// Activations come through scalar buffer loads whose range is the x row:
// dwords past K read as zero, so the last, partial period runs through the
// same pipelined loop (its codes past K meet zero activations).


constexpr int kTUnit = 8;                   // bytes per pipeline unit (4 byte pairs)
constexpr int kTUnits = 128 / kTUnit;       // units per period
constexpr int kTUnitXd = 5 * kTUnit / 2;    // x dwords per unit (20)

struct TEnt {
  u32x4_t e[kTUnit];
};
struct TWin {
  uint32_t r[kTUnitXd];
};

// LDS table reads of unit U (the addresses come from the chunk ring).
template <int U, int R>
__device__ __forceinline__ void t_lds(TEnt& b, const uint4 (&d)[R], uint32_t lane_off, const uint8_t* lut) {
  sfor<kTUnit>([&](auto bi) __attribute__((always_inline)) {
    constexpr int j = U * kTUnit + decltype(bi)::value;  // byte within the period
    const uint32_t w = word_of(d[(j >> 4) % R], (j & 15) >> 2);
    const uint32_t addr = __builtin_amdgcn_perm(w, lane_off, 0x0C0C0000u | ((4u + (j & 3)) << 8));
    b.e[decltype(bi)::value] = lds_b128(lut + kTLut + addr);
  });
}

// Scalar loads of unit U's x window (x_off: byte offset of the period in x).
template <int U>
__device__ __forceinline__ void t_x(TWin& w, i32x4_t xrs, int x_off) {
  // two scalar loads (16 + 4 dwords) rather than five of 4: fewer instructions
  // for the scalar unit to issue per step
  static_assert(kTUnitXd == 20, "one 16-dword and one 4-dword load per window");
  const i32x16_t v = ql_sbuf_load_x16(xrs, x_off + 4 * (kTUnitXd * U), 0);
  const i32x4_t t = ql_sbuf_load_x4(xrs, x_off + 4 * (kTUnitXd * U + 16), 0);
  sfor<16>([&](auto i) __attribute__((always_inline)) { w.r[decltype(i)::value] = (uint32_t)v[decltype(i)::value]; });
  w.r[16] = (uint32_t)t.x;
  w.r[17] = (uint32_t)t.y;
  w.r[18] = (uint32_t)t.z;
  w.r[19] = (uint32_t)t.w;
}

template <int U>
__device__ __forceinline__ void t_compute(const TEnt& b, const TWin& w, float (&acc)[5]) {
  sfor<kTUnit / 2>([&](auto qi) __attribute__((always_inline)) {
    constexpr int q = decltype(qi)::value;
    constexpr int k = 5 * kTUnit * U + 10 * q;  // first input of the byte pair, within the period
    const u32x4_t A = b.e[2 * q], B = b.e[2 * q + 1];
    acc[k / 128] = dot2(A.x, w.r[5 * q + 0], acc[k / 128]);
    acc[(k + 2) / 128] = dot2(A.y, w.r[5 * q + 1], acc[(k + 2) / 128]);
    acc[(k + 4) / 128] = dot2(A.z, w.r[5 * q + 2], acc[(k + 4) / 128]);
    acc[(k + 4) / 128] = dot2(B.w, w.r[5 * q + 2], acc[(k + 4) / 128]);
    acc[(k + 6) / 128] = dot2(B.x, w.r[5 * q + 3], acc[(k + 6) / 128]);
    acc[(k + 8) / 128] = dot2(B.y, w.r[5 * q + 4], acc[(k + 8) / 128]);
  });
}

// y += scale(g) * acc[g - 5p] over the period's groups, in group order; the
// period starts at position S0 of its first scale block (sa), later groups sit
// in the next block (sb).  Groups at or past G contribute nothing.
template <int S0>
__device__ __forceinline__ void t_scale(const u32x4_t& sa, const u32x2_t& sb, int g_left, const float (&acc)[5],
                                        float& y) {
  sfor<5>([&](auto gl_) __attribute__((always_inline)) {
    constexpr int gl = decltype(gl_)::value, q = S0 + gl;
    const uint32_t w = q < 8 ? sa[q >> 1] : sb[(q - 8) >> 1];
    const float v = scale_of_pair<q & 1>(w);
    y = fmaf(gl < g_left ? v : 0.0f, acc[gl], y);
  });
}

#ifndef QL_T_RING
#define QL_T_RING 4  // 16-byte chunks in flight per lane (ternary)
#endif

// Batch 1 only.  Periods p0..p1-1 of the slab (the last may be partial).
template <int M>
__device__ void run_t(const SlabCtx<M>& c, int p0, int p1, float (&y)[M]) {
  static_assert(M == 1, "the ternary GEMV runs batch 1");
  if (p0 >= p1) return;
  const int nchunks = (c.K + 79) / 80;
  // the row's chunks end in the first half of its last period (p1 - 1)
  const bool last_half = nchunks - 8 * (p1 - 1) <= 4;
  uint32_t lane_off = (uint32_t)(c.lane & 15) << 4;
  // chunks of the slab up to period p1; later ones (the ring's look-ahead past
  // the end of the row or of a split part) read as zero without memory traffic
  const ChunkSrc src(c.codes, nchunks < 8 * p1 ? nchunks : 8 * p1, c.lane);
  const i32x4_t xrs = scalar_rsrc(c.x, (uint32_t)c.K * 2u);
  // ring of R: chunk ch of a period lives in slot ch % R; once a chunk's last
  // byte is addressed its slot takes the chunk R positions later
  constexpr int R = QL_T_RING;
  static_assert(8 % R == 0, "the ring must divide a period's 8 chunks");
  uint4 d[R];
  sfor<R>([&](auto ch) __attribute__((always_inline)) { d[decltype(ch)::value] = src.load(8 * p0 + decltype(ch)::value); });
  // Per step U: table reads and x window of unit U+1, dot2 of unit U, one
  // lgkmcnt(0) wait.  Unit u uses entry buffer and window u & 1.
  TEnt A, B;
  TWin W0, W1;
  float acc[5];
  t_lds<0, R>(A, d, lane_off, c.lut);
  t_x<0>(W0, xrs, 2 * kPeriodK * p0);
  lgkm_wait0();
  const int G8 = (c.G + 7) >> 3;
  for (int p = p0; p < p1; ++p) {
    // Scales of the period's groups 5p .. 5p+4: the lane's 8-group block holding
    // group 5p and, when the period runs past it, the next block (if stored).
    // Whole-block loads touch each cache line once; per-group loads touched a
    // line per lane.
    const int blk = (5 * p) >> 3, s0 = (5 * p) & 7;
    // A period reaches at most 4 groups into the next block, so only that half
    // is read.  Both loads are unconditional (the second clamped to the last
    // stored block, whose values are then never used) and every loaded dword
    // stays live to the period's end: the chunk waits in between then count
    // these loads as in flight instead of waiting for them.
    const u32x4_t sa = ld_scale_blk(c.scales, blk, c.lane);
    const u32x2_t sb = ld_scale_blk_lo(c.scales, blk + 1 < G8 ? blk + 1 : blk, c.lane);
    const int g_left = c.G - 5 * p;  // groups of the period below G (at least 1)
#pragma unroll
    for (int gl = 0; gl < 5; ++gl) acc[gl] = 0.0f;
    const bool more = p + 1 < p1;
    int x_off = 2 * kPeriodK * p;
    auto step = [&](auto u) __attribute__((always_inline)) {
      constexpr int U = decltype(u)::value;
      constexpr bool odd = (U & 1) != 0;
      auto& cur = odd ? B : A;
      auto& nxt = odd ? A : B;
      auto& wc = odd ? W1 : W0;
      auto& wn = odd ? W0 : W1;
      // issue the next unit's reads at raised wave priority, so that a wave
      // with its operands ready hands the table reads to LDS before the SIMD
      // turns to other waves' arithmetic
      __builtin_amdgcn_s_setprio(1);
      if constexpr (U + 1 < kTUnits) {
        t_lds<U + 1, R>(nxt, d, lane_off, c.lut);
        t_x<U + 1>(wn, xrs, x_off);
        constexpr int last_byte = (U + 1) * kTUnit + kTUnit - 1;
        if constexpr ((last_byte & 15) == 15) {
          constexpr int ch = last_byte >> 4;
          d[ch % R] = src.load(ch + R < 8 ? 8 * p + ch + R : 8 * (p + 1) + ch + R - 8);
        }
      } else {
        if (more) {
          t_lds<0, R>(nxt, d, lane_off, c.lut);
          t_x<0>(wn, xrs, x_off + 2 * kPeriodK);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      sched_fence();
      t_compute<U>(cur, wc, acc);
      after(lane_off, acc);
      sched_fence();
      pin_s(x_off);
      lgkm_wait0();
    };
    // The second half-period of the last period is skipped when the row ends
    // in its first half (all of it would be padding against zero activations).
    sfor<kTUnits / 2>(step);
    if (more || !last_half)
      sfor_from<kTUnits / 2, kTUnits / 2>(step);
    switch (s0) {
      case 0: t_scale<0>(sa, sb, g_left, acc, y[0]); break;
      case 1: t_scale<1>(sa, sb, g_left, acc, y[0]); break;
      case 2: t_scale<2>(sa, sb, g_left, acc, y[0]); break;
      case 3: t_scale<3>(sa, sb, g_left, acc, y[0]); break;
      case 4: t_scale<4>(sa, sb, g_left, acc, y[0]); break;
      case 5: t_scale<5>(sa, sb, g_left, acc, y[0]); break;
      case 6: t_scale<6>(sa, sb, g_left, acc, y[0]); break;
      default: t_scale<7>(sa, sb, g_left, acc, y[0]); break;
    }
  }
}

// ---------------------------------------------------------------- 2-bit units
// unit = UB2 bytes of one group (4 codes per byte); a group is 32 bytes = 2 chunks.
template <int M>
constexpr int i2_ub() { return 8 / M; }

template <int M>
struct I2Buf {
  u32x2_t e[i2_ub<M>()];
  uint32_t x[M][2 * i2_ub<M>()];
};

// ring: 4 chunks = 2 groups; group slot S (0, 1) holds chunks 2S, 2S+1
template <int M, int S, int U>
__device__ __forceinline__ void i2_issue(I2Buf<M>& b, const uint4 (&d)[4], uint32_t lane_off, const uint8_t* lut,
                                         const cu32p (&xb)[M]) {
  constexpr int UB = i2_ub<M>();
  sfor<UB>([&](auto bi) __attribute__((always_inline)) {
    constexpr int j = U * UB + decltype(bi)::value;  // byte within the group (0..31)
    const uint32_t w = word_of(d[2 * S + (j >> 4)], (j & 15) >> 2);
    const uint32_t bv = (w >> (8 * (j & 3))) & 0xFFu;
    b.e[decltype(bi)::value] = lds_b64(lut + kI2Lut + ((bv << 5) | lane_off));
  });
#pragma unroll
  for (int m = 0; m < M; ++m)
    sfor<2 * UB>([&](auto i) __attribute__((always_inline)) {
      b.x[m][decltype(i)::value] = xb[m][2 * U * UB + decltype(i)::value];
    });
}

template <int M>
__device__ __forceinline__ void i2_compute(const I2Buf<M>& b, float (&acc)[M]) {
  constexpr int UB = i2_ub<M>();
  sfor<UB>([&](auto bi) __attribute__((always_inline)) {
    constexpr int q = decltype(bi)::value;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      acc[m] = dot2(b.e[q].x, b.x[m][2 * q], acc[m]);
      acc[m] = dot2(b.e[q].y, b.x[m][2 * q + 1], acc[m]);
    }
  });
}

template <int M>
__device__ void run_i2(const SlabCtx<M>& c, int g0, int g1, float (&y)[M]) {
  constexpr int NU = 32 / i2_ub<M>();  // units per group
  if (g0 >= g1) return;
  uint32_t lane_off = (uint32_t)(c.lane & 3) << 3;
  const ChunkSrc src(c.codes, 2 * g1, c.lane);
  uint4 d[4];
  sfor<4>([&](auto q) __attribute__((always_inline)) { d[decltype(q)::value] = src.load(2 * g0 + decltype(q)::value); });
  I2Buf<M> A, B;
  cu32p xb[M];
  set_xb(xb, c, kGroup * g0);
  i2_issue<M, 0, 0>(A, d, lane_off, c.lut, xb);
  lgkm_wait0();
  for (int gb = g0; gb < g1; gb += 2) {
    sfor<2>([&](auto s_) __attribute__((always_inline)) {
      constexpr int S = decltype(s_)::value;
      const int g = gb + S;
      if (g < g1) {
        const float sc = ld_scale(c.scales, g, c.lane);
        float acc[M];
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = 0.0f;
        cu32p xn[M];
        set_xb(xn, c, kGroup * (g + 1));
        const bool more = g + 1 < g1;
        sfor<NU>([&](auto u) __attribute__((always_inline)) {
          constexpr int U = decltype(u)::value;
          constexpr bool even = ((S * NU + U) & 1) == 0;  // buffer of this unit
          if constexpr (U + 1 < NU) {
            if constexpr (even)
              i2_issue<M, S, U + 1>(B, d, lane_off, c.lut, xb);
            else
              i2_issue<M, S, U + 1>(A, d, lane_off, c.lut, xb);
          } else {
            if (more) {
              if constexpr (even)
                i2_issue<M, S ^ 1, 0>(B, d, lane_off, c.lut, xn);
              else
                i2_issue<M, S ^ 1, 0>(A, d, lane_off, c.lut, xn);
            }
            // every byte of this group is addressed: its slot takes group g + 2
            d[2 * S] = src.load(2 * (g + 2));
            d[2 * S + 1] = src.load(2 * (g + 2) + 1);
          }
          sched_fence();
          if constexpr (even)
            i2_compute<M>(A, acc);
          else
            i2_compute<M>(B, acc);
          after(lane_off, acc);
          sched_fence();
          pin_s(xb);
          pin_s(xn);
          lgkm_wait0();
        });
#pragma unroll
        for (int m = 0; m < M; ++m) y[m] = fmaf(sc, acc[m], y[m]);
#pragma unroll
        for (int m = 0; m < M; ++m) xb[m] = xn[m];
      }
    });
  }
}

// ---------------------------------------------------------------- 3-bit units
// unit = NP 6-bit fields (pairs) of one 96-bit triple; a group is 4 triples = 3 chunks.
template <int M>
constexpr int i3_np() { return 16 / M; }

template <int M>
struct I3Buf {
  uint32_t e[i3_np<M>()];
  uint32_t x[M][i3_np<M>()];
};

// triple T (0..3) of group slot S: words 3T..3T+2 of the slot's 3 chunks (12 words)
template <int M, int S, int U>
__device__ __forceinline__ void i3_issue(I3Buf<M>& b, const uint4 (&d)[6], const uint8_t* lut, const cu32p (&xb)[M],
                                         uint32_t tok, uint32_t lane_off) {
  constexpr int NP = i3_np<M>();
  constexpr int T = (U * NP) / 16;   // triple within the group
  constexpr int P0 = (U * NP) % 16;  // first pair within the triple
  constexpr int wb = 3 * T;          // first word of the triple within the group
  uint32_t w0 = word_of(d[3 * S + (wb >> 2)], wb & 3);
  uint32_t w1 = word_of(d[3 * S + ((wb + 1) >> 2)], (wb + 1) & 3);
  uint32_t w2 = word_of(d[3 * S + ((wb + 2) >> 2)], (wb + 2) & 3);
  asm volatile("" : "+v"(w0), "+v"(w1), "+v"(w2) : "v"(tok));  // table reads stay in this step
  sfor<NP>([&](auto pi) __attribute__((always_inline)) {
    constexpr int P = P0 + decltype(pi)::value;
    b.e[decltype(pi)::value] = lds_b32(lut + kI3Lut + i3_addr<P>(w0, w1, w2, lane_off));
  });
#pragma unroll
  for (int m = 0; m < M; ++m)
    sfor<NP>([&](auto i) __attribute__((always_inline)) {
      b.x[m][decltype(i)::value] = xb[m][16 * T + P0 + decltype(i)::value];
    });
}

template <int M>
__device__ __forceinline__ void i3_compute(const I3Buf<M>& b, float (&acc)[M]) {
  sfor<i3_np<M>()>([&](auto pi) __attribute__((always_inline)) {
    constexpr int q = decltype(pi)::value;
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = dot2(b.e[q], b.x[m][q], acc[m]);
  });
}

template <int M>
__device__ void run_i3(const SlabCtx<M>& c, int g0, int g1, float (&y)[M]) {
  constexpr int NU = 64 / i3_np<M>();  // units per group (4 triples x 16 pairs)
  if (g0 >= g1) return;
  const ChunkSrc src(c.codes, 3 * g1, c.lane);
  uint4 d[6];
  sfor<6>([&](auto q) __attribute__((always_inline)) { d[decltype(q)::value] = src.load(3 * g0 + decltype(q)::value); });
  I3Buf<M> A, B;
  cu32p xb[M];
  set_xb(xb, c, kGroup * g0);
  const uint32_t lane_off = i3_lane_off(c.lane);
  uint32_t tok = 0;  // step token: rewritten (as far as the compiler knows) after each step's arithmetic
  i3_issue<M, 0, 0>(A, d, c.lut, xb, tok, lane_off);
  lgkm_wait0();
  for (int gb = g0; gb < g1; gb += 2) {
    sfor<2>([&](auto s_) __attribute__((always_inline)) {
      constexpr int S = decltype(s_)::value;
      const int g = gb + S;
      if (g < g1) {
        const float sc = ld_scale(c.scales, g, c.lane);
        float acc[M];
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = 0.0f;
        cu32p xn[M];
        set_xb(xn, c, kGroup * (g + 1));
        const bool more = g + 1 < g1;
        sfor<NU>([&](auto u) __attribute__((always_inline)) {
          constexpr int U = decltype(u)::value;
          constexpr bool even = ((S * NU + U) & 1) == 0;
          __builtin_amdgcn_s_setprio(1);  // the next unit's reads at raised priority, as in the ternary step
          if constexpr (U + 1 < NU) {
            if constexpr (even)
              i3_issue<M, S, U + 1>(B, d, c.lut, xb, tok, lane_off);
            else
              i3_issue<M, S, U + 1>(A, d, c.lut, xb, tok, lane_off);
          } else {
            if (more) {
              if constexpr (even)
                i3_issue<M, S ^ 1, 0>(B, d, c.lut, xn, tok, lane_off);
              else
                i3_issue<M, S ^ 1, 0>(A, d, c.lut, xn, tok, lane_off);
            }
#pragma unroll
            for (int q = 0; q < 3; ++q) d[3 * S + q] = src.load(3 * (g + 2) + q);
          }
          __builtin_amdgcn_s_setprio(0);
          sched_fence();
          if constexpr (even)
            i3_compute<M>(A, acc);
          else
            i3_compute<M>(B, acc);
          after(tok, acc);
          sched_fence();
          pin_s(xb);
          pin_s(xn);
          lgkm_wait0();
        });
#pragma unroll
        for (int m = 0; m < M; ++m) y[m] = fmaf(sc, acc[m], y[m]);
#pragma unroll
        for (int m = 0; m < M; ++m) xb[m] = xn[m];
      }
    });
  }
}

// A slab's share of the input: periods [p0, p1) on ternary slabs, group
// pairs [k0, k1) (groups 2 k0 .. min(2 k1, G) - 1) on 2- and 3-bit slabs.
template <int M>
__device__ __forceinline__ void run_slab(int gr, const SlabCtx<M>& c, int p0, int p1, int k0, int k1, float (&y)[M]) {
  const int g0 = 2 * k0, g1 = (2 * k1 < c.G) ? 2 * k1 : c.G;
  if (gr == QL_GRID_T)
    run_t<M>(c, p0, p1, y);
  else if (gr == QL_GRID_I2)
    run_i2<M>(c, g0, g1, y);
  else
    run_i3<M>(c, g0, g1, y);
}

// ---------------------------------------------------------------- kernels
#ifndef QL_WAVES
#define QL_WAVES 8
#endif
#ifndef QL_WAVES_PER_EU
#define QL_WAVES_PER_EU 4
#endif
#ifndef QL_WG_PER_CU
#define QL_WG_PER_CU 2
#endif
constexpr int kWaves = QL_WAVES;          // waves per workgroup
constexpr int kWgPerCu = QL_WG_PER_CU;    // resident workgroups per CU (LDS tables: 77 KB each)

// One wave task: one 64-row slab of one descriptor, or one part of its input
// when the entry is split (partial sums then meet in the state buffer).
// Descriptor fields are re-read per task, which keeps their live ranges short
// (the kernels stay free of register spills).
template <int M>
__device__ __forceinline__ void gemv_task(const ql_gemv_desc* __restrict__ descs, const TaskLoc& loc, int64_t t,
                                          int Mact, const uint8_t* lut, int lane, uint32_t* state) {
  static_assert(M == 1, "split partial sums hold one value per lane");
  const ql_gemv_desc& d = descs[loc.di];
  if (!task_in_entry(d, t)) return;
  const SplitTask st(d, t);
  const int K = d.K, G = K / kGroup, G8 = (G + 7) / 8;
  float y[M];
#pragma unroll
  for (int m = 0; m < M; ++m) y[m] = 0.0f;
  SlabCtx<M> c{static_cast<const uint8_t*>(d.packed) + loc.off, d.pscales + st.slab * (int64_t)G8 * kSlab * 8, d.x,
               K, G, Mact, lane, lut};
  run_slab<M>(loc.gr, c, st.p0(K), st.p1(K), st.k0(K), st.k1(K), y);
  if (st.split()) {
    float* sl = st.slots(d, state);
    st.put(sl, lane, y[0]);
    if (!st.arrive(st.counter(d, state), lane)) return;
    st.totals<1, 8>(sl, y, lane);
  }
  const int64_t row = (int64_t)st.slab * kSlab + lane;
  if (row < d.N) d.y[row] = y[0];
}

// A single matrix: all slabs cost the same, so waves stride over them.  The
// descriptor travels in the kernel arguments; `count` (always 1) is a runtime
// value so its reads stay inside the task loop instead of being hoisted and
// kept live across it.
template <int M>
__global__ void __launch_bounds__(kWaves * 64, QL_WAVES_PER_EU) gemv_kernel(ql_gemv_desc desc, int count, int64_t total, int Mact) {
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLutBytes];
  build_luts<kWaves * 64>(lut);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  for (int64_t t = (int64_t)blockIdx.x * kWaves + wave; t < total; t += (int64_t)gridDim.x * kWaves)
    gemv_task<M>(&desc, locate_task(&desc, count, t), t, Mact, lut, lane, nullptr);
}

// Many independent matrices in one persistent launch.  Slab costs differ
// (row length, grid), so after its first task a wave keeps drawing tasks from
// the task queues: list scheduling over tasks that the host numbered
// longest-first.  The next task is drawn when the current one starts and read
// when it ends, so the atomic's round trip is hidden behind the task instead
// of stalling the wave between tasks; a wave then holds at most one task
// ahead, which costs little balance because the last tasks are the shortest.
template <int M>
__global__ void __launch_bounds__(kWaves * 64, QL_WAVES_PER_EU) gemv_grouped_kernel(const ql_gemv_desc* __restrict__ descs,
                                                                      int count, int64_t total, int Mact,
                                                                      uint32_t* __restrict__ sched) {
  __shared__ __attribute__((aligned(16))) uint8_t lut[kLutBytes];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int64_t t = (int64_t)blockIdx.x * kWaves + wave;
  // the first task's descriptor loads are in flight while the tables are built
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
    gemv_task<M>(descs, loc, t, Mact, lut, lane, sched);
    t = tq.resolve(claim, lane);
    if (t >= 0) loc = locate_task(descs, count, t);
  }
  tq.checkout(lane);
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

// Only the batch-1 instantiation exists: the pipelined template for
// 2 <= M <= 8 spilled thousands of registers and faulted the GPU in its first
// test, so it is not built; M >= 2 runs on the MFMA path instead.
hipError_t launch_gemv(const MatArgs& a, int M, hipStream_t stream) {
  if (M != 1) return hipErrorInvalidValue;
  const int64_t nslabs = ((int64_t)a.N + kSlab - 1) / kSlab;
  const ql_gemv_desc d{a.packed, a.pscales, a.blk_grid, a.blk_off, a.x, a.y, a.N, a.K, a.grid, 0, 1, 0, 0};
  const int slots = device_cu_count() * kWgPerCu;
  const int64_t wg_needed = (nslabs + kWaves - 1) / kWaves;
  const int grid = (int)(wg_needed < slots ? wg_needed : slots);
  hipLaunchKernelGGL(gemv_kernel<1>, dim3(grid), dim3(kWaves * 64), 0, stream, d, 1, nslabs, 1);
  return hipGetLastError();
}

int64_t grouped_wave_slots(int M) {
  if (M == 1) return (int64_t)device_cu_count() * kWgPerCu * kWaves;
  return b4_wave_slots(M);
}

hipError_t launch_grouped_for(const ql_gemv_desc* descs, int32_t count, int64_t total_tasks, int M, uint32_t* sched,
                              hipStream_t stream) {
  if (M == 1) return launch_gemv_grouped(descs, count, total_tasks, M, sched, stream);
  return launch_gemv_b4_grouped(descs, count, total_tasks, M, sched, stream);
}

hipError_t launch_gemv_grouped(const ql_gemv_desc* descs, int32_t count, int64_t total_tasks, int M, uint32_t* sched,
                               hipStream_t stream) {
  if (M != 1) return hipErrorInvalidValue;
  const int slots = device_cu_count() * kWgPerCu;
  const int64_t wg_needed = (total_tasks + kWaves - 1) / kWaves;
  const int grid = (int)(wg_needed < slots ? wg_needed : slots);
  hipLaunchKernelGGL(gemv_grouped_kernel<1>, dim3(grid), dim3(kWaves * 64), 0, stream, descs, count, total_tasks, 1,
                     sched);
  return hipGetLastError();
}

}  // namespace ql
