// Streaming helpers shared by the decode kernels (gfx950): 128-bit buffer
// loads of slab chunks, scalar buffer loads of activations, LDS table reads,
// v_dot2_f32_bf16, compile-time loops, zero-instruction step boundaries for the
// software pipelines, and the grouped launches' task location, split-K and
// task queues.
#pragma once

#include <utility>

#include "ql_device.hpp"

namespace ql {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef const __attribute__((address_space(4))) uint32_t* cu32p;  // scalar-loaded x

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <class F, int... I>
__device__ __forceinline__ void sfor_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void sfor(F&& f) {
  sfor_impl(f, std::make_integer_sequence<int, N>{});
}
// f(B), f(B+1), ..., f(B+N-1) with compile-time arguments
template <int B, class F, int... I>
__device__ __forceinline__ void sfor_from_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, B + I>{}), ...);
}
template <int B, int N, class F>
__device__ __forceinline__ void sfor_from(F&& f) {
  sfor_from_impl<B>(f, std::make_integer_sequence<int, N>{});
}

// s_waitcnt lgkmcnt(0), leaving vmcnt/expcnt alone.
__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Compiler-only step boundaries (empty asm, no instruction).  pin_v/pin_s
// claim to rewrite a value, so address arithmetic that reads it (and the loads
// it feeds) stays below this point.  `after` also reads the step's
// accumulators, so the step's arithmetic stays above it.  Together they keep
// one unit of operands in flight: without them the compiler sinks arithmetic
// below later loads and keeps several units live (and spills).
__device__ __forceinline__ void pin_v(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin_s(int& v) { asm volatile("" : "+s"(v)); }
template <int M>
__device__ __forceinline__ void pin_s(cu32p (&p)[M]) {
#pragma unroll
  for (int m = 0; m < M; ++m) asm volatile("" : "+s"(p[m]));
}
template <int N>
__device__ __forceinline__ void after(uint32_t& v, const float (&acc)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v) : "v"(acc[i]));
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef const __attribute__((address_space(1))) u32x4_t* gu32x4p;  // global memory
typedef const __attribute__((address_space(3))) u32x4_t* lu32x4p;  // LDS
typedef const __attribute__((address_space(3))) u32x2_t* lu32x2p;
typedef const __attribute__((address_space(3))) uint32_t* lu32p;

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// A pointer the compiler must treat as wave-uniform (it is: every slab
// pointer is derived from wave-uniform task indices), so resources built from
// it live in SGPRs and need no per-lane waterfall.
__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (void*)(((uint64_t)hi << 32) | lo);
}

// Code chunks of one slab, read through a buffer resource: a chunk past the
// wave's range reads as zero without a memory access, so the prefetch ring
// needs no branches.  Non-temporal: each weight byte is used once per pass.
struct ChunkSrc {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t lane_off;  // lane * 16
  __device__ __forceinline__ ChunkSrc(const uint8_t* slab, int nchunks, int lane)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(uniform_ptr(slab), (short)0,
                                               __builtin_amdgcn_readfirstlane(nchunks * kSlabChunkBytes), 0x00020000)),
        lane_off((uint32_t)lane * kChunkBytes) {}
  __device__ __forceinline__ uint4 load(int chunk) const {
    const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, lane_off + (uint32_t)chunk * kSlabChunkBytes, 0, 2);
    return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
  }
};

// Table reads from LDS.  The ternary read keeps all 16 bytes (volatile stops
// the compiler from narrowing it to ds_read_b96, which the probe measured at
// less than half the throughput of ds_read_b128 on replicated tables).
__device__ __forceinline__ u32x4_t lds_b128(const uint8_t* p) {
  return *(const volatile __attribute__((address_space(3))) u32x4_t*)(p);
}
__device__ __forceinline__ u32x2_t lds_b64(const uint8_t* p) { return *(lu32x2p)(p); }
__device__ __forceinline__ uint32_t lds_b32(const uint8_t* p) { return *(lu32p)(p); }

typedef const __attribute__((address_space(1))) uint16_t* gu16p;

// The aligned dword holding the scales of groups g & ~1 (low half) and g | 1
// (high half) of slab row `lane`; read as a whole so no zero-extension ties
// the value to the load's completion before it is used.
__device__ __forceinline__ uint32_t ld_scale_pair(const uint16_t* __restrict__ ss, int g, int lane) {
  typedef const __attribute__((address_space(1))) uint32_t* gu32p;
  return ((gu32p)ss)[(((g >> 3) * kSlab + lane) * 8 + (g & 7)) >> 1];
}
// fp32 value of half H of a scale pair
template <int H>
__device__ __forceinline__ float scale_of_pair(uint32_t p) {
  return __uint_as_float(H ? (p & 0xFFFF0000u) : (p << 16));
}
// The 16 bytes holding the scales of groups 8 blk .. 8 blk + 7 of slab row `lane`
// (one coalesced kilobyte per wave); blk must be below ceil(G / 8).
__device__ __forceinline__ u32x4_t ld_scale_blk(const uint16_t* __restrict__ ss, int blk, int lane) {
  return ((gu32x4p)ss)[blk * kSlab + lane];
}
// The first half of that block (groups 8 blk .. 8 blk + 3).
__device__ __forceinline__ u32x2_t ld_scale_blk_lo(const uint16_t* __restrict__ ss, int blk, int lane) {
  typedef const __attribute__((address_space(1))) u32x2_t* gu32x2p;
  return ((gu32x2p)ss)[(blk * kSlab + lane) * 2];
}
__device__ __forceinline__ float ld_scale(const uint16_t* __restrict__ ss, int g, int lane) {
  return bf16_bits_to_f32(((gu16p)ss)[((g >> 3) * kSlab + lane) * 8 + (g & 7)]);
}

__device__ __forceinline__ uint32_t word_of(const uint4& d, int w) {
  return w == 0 ? d.x : (w == 1 ? d.y : (w == 2 ? d.z : d.w));
}

__device__ i32x4_t ql_sbuf_load_x4(i32x4_t rsrc, int offset, int cachepolicy) __asm("llvm.amdgcn.s.buffer.load.v4i32");

// Buffer resource over n_bytes of uniform memory at p (raw, stride 0).
__device__ __forceinline__ i32x4_t scalar_rsrc(const void* p, uint32_t n_bytes) {
  const uint64_t v = (uint64_t)p;
  return i32x4_t{(int)__builtin_amdgcn_readfirstlane((uint32_t)v),
                 (int)(__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) & 0xFFFFu),
                 (int)__builtin_amdgcn_readfirstlane(n_bytes), 0x00020000};
}

}  // namespace ql

namespace ql {

// Index of the descriptor holding grouped task (slab) t: the last entry whose
// slab_begin <= t (entries are in slab_begin order).
__device__ __forceinline__ int find_desc(const ql_gemv_desc* __restrict__ descs, int count, int64_t t) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (descs[mid].slab_begin <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// True when task t lies inside descriptor d's own tasks.  A task total larger
// than the one prepare returned would map its extra tasks onto the last entry
// with slab indices past its rows; such tasks are dropped instead of reading
// past the entry's packed and scale buffers.
__device__ __forceinline__ bool task_in_entry(const ql_gemv_desc& d, int64_t t) {
  const int64_t nslabs = ((int64_t)d.N + kSlab - 1) / kSlab;
  const int64_t parts = d.kparts > 1 ? d.kparts : 1;
  return t - (int64_t)d.slab_begin < nslabs * parts;
}

// ---------------------------------------------------------------- split-K
// qlinear_grouped_prepare_split may cut the input of every slab of an entry
// into kparts parts, each a task of its own: whole 640-input periods on
// ternary slabs, whole pairs of 128-input groups on 2- and 3-bit slabs
// (kparts never exceeds the periods, so no part is empty).  The
// entry's split state starts at word ws_begin of the launch's state buffer:
// one counter per slab (each in its own 128-byte line), then kPartWords
// partial sums per (slab, part).  A part stores its partial sums and counts
// itself in; the wave that counts last sums the parts in part order, so the
// result is the same bits whichever wave finishes last, and resets the counter
// for the next launch.
//
// Partial sums travel as device-scope atomic stores and loads, which the
// hardware keeps coherent across the XCDs' separate L2 caches by themselves
// (they write through to, and read from, the device's coherence point).  The
// counter increment is issued only once those stores are complete, and the
// last wave's loads only once its increment has returned, so no device-scope
// fence is needed: such a fence writes back (release) or invalidates (acquire)
// a whole L2, and with one per task those cache operations serialized the
// launch (measured: a 2688-task launch took 2.6x as long as its unsplit form).
struct SplitTask {
  uint32_t slab, part, parts;  // task indices stay below 2^31

  __device__ __forceinline__ SplitTask(const ql_gemv_desc& d, int64_t t) {
    parts = d.kparts > 1 ? (uint32_t)d.kparts : 1u;
    const uint32_t local = (uint32_t)(t - d.slab_begin);
    slab = local / parts;
    part = local - slab * parts;
  }
  // ternary: periods [p0, p1) of the row
  __device__ __forceinline__ int p0(int K) const { return (int)(part * (uint32_t)((K + kPeriodK - 1) / kPeriodK) / parts); }
  __device__ __forceinline__ int p1(int K) const {
    return (int)((part + 1) * (uint32_t)((K + kPeriodK - 1) / kPeriodK) / parts);
  }
  // 2- and 3-bit: group pairs [k0, k1) (groups 2 k0 .. min(2 k1, G) - 1), so
  // that each part starts on an even group: the scale pairs and ring slots of
  // the 2- and 3-bit drivers then have compile-time parity
  __device__ __forceinline__ int k0(int K) const { return (int)(part * (uint32_t)((K / kGroup + 1) / 2) / parts); }
  __device__ __forceinline__ int k1(int K) const {
    return (int)((part + 1) * (uint32_t)((K / kGroup + 1) / 2) / parts);
  }
  __device__ __forceinline__ bool split() const { return __builtin_expect(parts > 1u, 0); }
  // the slab's counter and partial sums (part q at q * kPartWords)
  __device__ __forceinline__ uint32_t* counter(const ql_gemv_desc& d, uint32_t* state) const {
    return state + d.ws_begin + (int64_t)slab * kCounterWords;
  }
  __device__ __forceinline__ float* slots(const ql_gemv_desc& d, uint32_t* state) const {
    const int64_t nslabs = ((int64_t)d.N + kSlab - 1) / kSlab;
    return reinterpret_cast<float*>(state + d.ws_begin + nslabs * kCounterWords) + (int64_t)slab * parts * kPartWords;
  }
  // partial-sum word w of this part
  __device__ __forceinline__ void put(float* sl, int w, float v) const {
    __hip_atomic_store(sl + part * kPartWords + w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // After this part's put()s: count the part in.  True (wave-uniform) in the
  // wave whose part completes the slab.
  __device__ __forceinline__ bool arrive(uint32_t* cnt, int lane) const {
    // this wave's stores complete before the increment is issued (the memory
    // clobber also keeps the compiler from moving them past it)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != parts - 1u) return false;
    asm volatile("" ::: "memory");  // the loads of totals() stay below the increment
    if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  // Last wave only: acc[j] = sum over the parts, in part order, of partial-sum
  // word 64 j + lane.  The loads of B parts are issued together, so the sum
  // costs about parts / B memory round trips.
  template <int NW, int B>
  __device__ __forceinline__ void totals(const float* sl, float (&acc)[NW], int lane) const {
    for (int q0 = 0; q0 < (int)parts; q0 += B) {
      float v[B][NW];
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int j = 0; j < NW; ++j)
          v[b][j] = q0 + b < (int)parts
                        ? __hip_atomic_load(sl + (q0 + b) * kPartWords + 64 * j + lane, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT)
                        : 0.0f;
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int j = 0; j < NW; ++j)
          if (q0 + b < (int)parts) acc[j] = q0 + b == 0 ? v[b][j] : acc[j] + v[b][j];
    }
  }
};

// Where task t lives: its descriptor, its slab's byte offset and grid.  Split
// from the task so that a wave's first task can be located (two or three
// dependent scalar loads) while the workgroup builds its LDS tables.
struct TaskLoc {
  int di;       // descriptor index
  int gr;       // grid of the slab
  int64_t off;  // byte offset of the slab in the packed matrix
};

__device__ __forceinline__ TaskLoc locate_task(const ql_gemv_desc* __restrict__ descs, int count, int64_t t) {
  TaskLoc l;
  l.di = find_desc(descs, count, t);
  const ql_gemv_desc& d = descs[l.di];
  const SplitTask st(d, t);
  l.off = task_in_entry(d, t) ? slab_offset(st.slab, d.K, d.grid, d.blk_grid, d.blk_off, &l.gr) : 0;
  return l;
}

// ---------------------------------------------------------------- task queues
// Persistent grouped launches run tasks 0..total-1, numbered by the host
// longest first.  Wave w of the launch takes task w; the rest, r = t - nwaves,
// are dealt round-robin to kQueues queues (queue q holds r = q, q + kQueues,
// ..., so each queue is longest-first too), each a counter in its own 128-byte
// line of the caller's state buffer.  A wave draws from its home queue (its
// workgroup index mod kQueues) until the queue runs dry; then one 64-lane load
// reads every queue's counter and the wave moves to the first live queue after
// its home.  One shared counter would serialize every draw of the launch on a
// single address, which caps the whole launch at one task per atomic round
// trip.  Counters only grow, so a stale read can only show a dry queue as live;
// the draw that follows then fails and the wave reads again.
constexpr int kQueues = 64;         // one per lane of the scan
constexpr int kQueueStride = 32;    // words between counters (128 bytes)
constexpr int kLineBase = kQueues * kQueueStride;      // check-out counter of home h at kLineBase + h * kQueueStride
constexpr int kSchedDone = 2 * kQueues * kQueueStride;  // check-out word
static_assert(kSchedDone + 1 <= QL_SCHED_WORDS, "scheduler state larger than QL_SCHED_WORDS");

struct TaskQueues {
  uint32_t* sched;
  int64_t nwaves;  // tasks of the first round
  int64_t rest;    // tasks dealt to the queues (total - nwaves, may be <= 0)
  int home;

  __device__ TaskQueues(uint32_t* s, int64_t total, int64_t nw)
      : sched(s), nwaves(nw), rest(total - nw), home((int)(blockIdx.x % kQueues)) {}

  // Every task is some wave's first task (total <= waves): no wave draws from
  // the queues, so the state is never touched and the check-out is skipped
  // (it costs short launches two dependent device-scope atomics per wave).
  __device__ bool single_round() const { return rest <= 0; }

  __device__ uint32_t qcount(int q) const {
    return rest > q ? (uint32_t)((rest - q + kQueues - 1) / kQueues) : 0u;
  }
  // the next task of this wave, or -1 once every queue is dry (wave-uniform)
  __device__ int64_t next(int lane) {
    if (single_round()) return -1;
    for (;;) {
      const uint32_t cnt = qcount(home);
      if (cnt > 0) {
        uint32_t t = 0;
        if (lane == 0) t = __hip_atomic_fetch_add(sched + home * kQueueStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        t = __builtin_amdgcn_readfirstlane(t);
        if (t < cnt) return nwaves + home + (int64_t)t * kQueues;
      }
      const int q = (home + lane) % kQueues;
      const uint32_t c = __hip_atomic_load(sched + q * kQueueStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t live = __ballot(c < qcount(q));
      if (!live) return -1;
      home = (home + (int)__builtin_ctzll(live)) % kQueues;
    }
  }
  // draw from the home queue now; lane 0 holds the result until resolve reads it
  __device__ uint32_t claim(int lane) {
    uint32_t t = 0xFFFFFFFFu;
    if (qcount(home) > 0 && lane == 0)
      t = __hip_atomic_fetch_add(sched + home * kQueueStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return t;
  }
  // the task a claim drew, or -1 if its queue was dry (then next() finds one)
  __device__ int64_t drawn(uint32_t claimed) const {
    const uint32_t t = __builtin_amdgcn_readfirstlane(claimed);
    return t < qcount(home) ? nwaves + home + (int64_t)t * kQueues : -1;
  }
  // the task a claim drew, or the next one found by next() if it drew nothing
  __device__ int64_t resolve(uint32_t claimed, int lane) {
    const int64_t t = drawn(claimed);
    return t >= 0 ? t : next(lane);
  }
  // Every wave checks out once, after its last draw; the last one zeroes the
  // state for the next launch.  Check-out is two-level so that no address takes
  // one atomic per wave (thousands of them, serialized at the end of the
  // launch): a wave counts itself in on the check-out line of its workgroup's
  // first home queue (one 128-byte line per home, apart from the queue lines);
  // the wave completing a line counts the line in on the check-out word, and
  // the wave completing that resets every counter.
  __device__ void checkout(int lane) {
    if (single_round()) return;
    const int h = (int)(blockIdx.x % kQueues);
    const int wgs = (int)gridDim.x;
    const uint32_t line_waves = (uint32_t)(((wgs - 1 - h) / kQueues + 1) * (nwaves / wgs));
    const uint32_t lines = (uint32_t)(wgs < kQueues ? wgs : kQueues);
    uint32_t c = 0;
    if (lane == 0) c = __hip_atomic_fetch_add(sched + kLineBase + h * kQueueStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    c = __builtin_amdgcn_readfirstlane(c);
    if (c != line_waves - 1) return;
    uint32_t done = 0;
    if (lane == 0) done = __hip_atomic_fetch_add(sched + kSchedDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    done = __builtin_amdgcn_readfirstlane(done);
    if (done == lines - 1) {
      __hip_atomic_store(sched + lane * kQueueStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(sched + kLineBase + lane * kQueueStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0) __hip_atomic_store(sched + kSchedDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
};

}  // namespace ql
