// Streaming helpers shared by the batch-1 GEMV kernels (gfx950): 128-bit
// buffer loads of slab chunks, scalar buffer loads of activations, LDS table
// reads, v_dot2_f32_bf16, compile-time loops and zero-instruction step
// boundaries for the software pipelines.
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
constexpr int kSchedDone = kQueues * kQueueStride;  // check-out word
static_assert(kSchedDone + 1 <= QL_SCHED_WORDS, "scheduler state larger than QL_SCHED_WORDS");

struct TaskQueues {
  uint32_t* sched;
  int64_t nwaves;  // tasks of the first round
  int64_t rest;    // tasks dealt to the queues (total - nwaves, may be <= 0)
  int home;

  __device__ TaskQueues(uint32_t* s, int64_t total, int64_t nw)
      : sched(s), nwaves(nw), rest(total - nw), home((int)(blockIdx.x % kQueues)) {}

  __device__ uint32_t qcount(int q) const {
    return rest > q ? (uint32_t)((rest - q + kQueues - 1) / kQueues) : 0u;
  }
  // the next task of this wave, or -1 once every queue is dry (wave-uniform)
  __device__ int64_t next(int lane) {
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
  // the task a claim drew, or the next one found by next() if it drew nothing
  __device__ int64_t resolve(uint32_t claimed, int lane) {
    const uint32_t t = __builtin_amdgcn_readfirstlane(claimed);
    if (t < qcount(home)) return nwaves + home + (int64_t)t * kQueues;
    return next(lane);
  }
  // every wave checks out once; the last one zeroes the state for the next launch
  __device__ void checkout(int lane) {
    uint32_t done = 0;
    if (lane == 0) done = __hip_atomic_fetch_add(sched + kSchedDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    done = __builtin_amdgcn_readfirstlane(done);
    if (done == (uint32_t)(nwaves - 1)) {
      __hip_atomic_store(sched + lane * kQueueStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0) __hip_atomic_store(sched + kSchedDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
};

}  // namespace ql
