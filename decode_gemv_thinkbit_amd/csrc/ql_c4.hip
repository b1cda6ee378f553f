// Batch-1 GEMV over 4-bit containers: the baseline the native kernels are
// measured against.
//
// The summary page (onedev.kr/papers/1416, section "Premises & limits") notes
// that the published checkpoints keep their 1.6/2/3-bit codewords in 4-bit
// containers, so a decode step streams about twice the bytes.  This kernel
// reads that format with the same machinery as the native GEMV -- 64-row slab
// tasks (lane = row), 128-bit buffer loads of the same slab-interleaved
// layout, activations through scalar buffer loads, exact bf16 code pairs from
// an LDS table, v_dot2_f32_bf16 with fp32 sums per 128-input group and one
// scale multiply per group -- so the comparison isolates bits per weight.
//
// Decode: one byte holds two codes (inputs 2i, 2i+1), so one table entry per
// byte value is the bf16 pair (c_lo, c_hi), which multiplies the activation
// dword (x_2i, x_2i+1) directly.  The table has 64 replicas, 256 B per byte
// value, so lane l reads replica l and the 64 lanes of a ds_read_b32 always
// fall on distinct banks; the address is one v_perm (byte << 8 | lane * 4).
#include "ql_internal.hpp"
#include "ql_stream.hpp"

namespace ql {

namespace {

constexpr int kC4Rep = 64;                      // table replicas (one per lane)
constexpr int kC4LutBytes = 256 * kC4Rep * 4;   // 64 KB
constexpr int kC4Ring = 8;                      // 16-byte chunks in flight per lane
constexpr int kC4Waves = 8;                     // waves per workgroup
constexpr int kC4WgPerCu = 2;                   // resident workgroups per CU (64 KB tables each)
constexpr int kC4ChunkK = 32;                   // inputs per 16-byte chunk

__device__ void build_c4_lut(uint8_t* lut) {
  for (int e = threadIdx.x; e < 256 * kC4Rep; e += blockDim.x) {
    const int b = e / kC4Rep;  // byte value; e % kC4Rep is the replica
    const int lo = (b & 15) - ((b & 8) << 1), hi = (b >> 4) - ((b & 128) >> 3);
    *reinterpret_cast<uint32_t*>(lut + 4 * e) = code_bf16(lo) | (code_bf16(hi) << 16);
  }
}

// One pipeline unit = one 16-byte chunk of a row (32 inputs).
struct C4Unit {
  uint32_t e[16];  // table entries: bf16 code pairs
  uint32_t x[16];  // activation dwords (scalar)
};

// Issue unit from ring slot SLOT: 16 table reads and 4 scalar x loads
// (x_off: byte offset of the chunk's first activation).
template <int SLOT>
__device__ __forceinline__ void c4_issue(C4Unit& u, const uint4 (&d)[kC4Ring], uint32_t lane_off, const uint8_t* lut,
                                         i32x4_t xrs, int x_off) {
  sfor<16>([&](auto bi) __attribute__((always_inline)) {
    constexpr int j = decltype(bi)::value;
    const uint32_t w = word_of(d[SLOT], j >> 2);
    const uint32_t addr = __builtin_amdgcn_perm(w, lane_off, 0x0C0C0000u | ((4u + (j & 3)) << 8));
    u.e[j] = lds_b32(lut + addr);
  });
  sfor<4>([&](auto qi) __attribute__((always_inline)) {
    constexpr int q = decltype(qi)::value;
    const i32x4_t v = ql_sbuf_load_x4(xrs, x_off + 16 * q, 0);
    u.x[4 * q + 0] = (uint32_t)v.x;
    u.x[4 * q + 1] = (uint32_t)v.y;
    u.x[4 * q + 2] = (uint32_t)v.z;
    u.x[4 * q + 3] = (uint32_t)v.w;
  });
}

__device__ __forceinline__ void c4_compute(const C4Unit& u, float (&acc)[1]) {
  sfor<16>([&](auto bi) __attribute__((always_inline)) {
    constexpr int j = decltype(bi)::value;
    acc[0] = dot2(u.e[j], u.x[j], acc[0]);
  });
}

// Row `lane` of one slab: y = sum_g s_g * sum_{k in g} c_k x_k.  Units run
// "issue next, compute current, wait"; ring slot u % 8 is reloaded with chunk
// u + 8 as soon as unit u's addresses are formed.  Chunks past the row and
// activations past K read as zero (buffer range checks), so no unit is guarded;
// the unit issued after the last one only reads table row 0.
__device__ float c4_slab(const uint8_t* slab, const uint16_t* scales, const uint16_t* x, int K, int lane,
                         const uint8_t* lut) {
  const int NC = K / kC4ChunkK, G = K / kGroup;
  const ChunkSrc src(slab, NC, lane);
  const i32x4_t xrs = scalar_rsrc(x, (uint32_t)K * 2);
  uint32_t lane_off = (uint32_t)lane * 4;
  // Scales run one group ahead, each as the dword of its group pair, converted
  // only where used, so waiting for a scale never drains the chunk ring.
  uint32_t sc[2];  // sc[g & 1]: scale pair holding group g
  sc[0] = ld_scale_pair(scales, 0, lane);
  uint4 d[kC4Ring];
  sfor<kC4Ring>([&](auto q) __attribute__((always_inline)) { d[decltype(q)::value] = src.load(decltype(q)::value); });
  C4Unit A, B;
  c4_issue<0>(A, d, lane_off, lut, xrs, 0);
  lgkm_wait0();
  float y = 0.0f;
  for (int g0 = 0; g0 < G; g0 += 2) {  // two groups (8 units) per iteration: ring slots are static
    // With G odd the last iteration's second group is g = G: its chunks and
    // activations read as zero, so it adds s * 0 and needs no guard.
    sfor<2>([&](auto s_) __attribute__((always_inline)) {
      constexpr int S = decltype(s_)::value;
      const int g = g0 + S;
      {
        // (clamped for the group after the last, whose contribution is s * 0)
        sc[S ^ 1] = ld_scale_pair(scales, g + 1 < G ? g + 1 : G - 1, lane);
        float acc[1] = {0.0f};
        sfor<4>([&](auto q_) __attribute__((always_inline)) {
          constexpr int U = 4 * S + decltype(q_)::value;  // ring slot of this unit
          const int u = 4 * g + decltype(q_)::value;      // chunk index
          int x_next = (u + 1) * (kC4ChunkK * 2);
          pin_s(x_next);
          // past the last chunk this reads zeros (in-range table rows, no memory access)
          if constexpr ((U & 1) == 0)
            c4_issue<(U + 1) % kC4Ring>(B, d, lane_off, lut, xrs, x_next);
          else
            c4_issue<(U + 1) % kC4Ring>(A, d, lane_off, lut, xrs, x_next);
          d[U] = src.load(u + kC4Ring);
          sched_fence();
          if constexpr ((U & 1) == 0)
            c4_compute(A, acc);
          else
            c4_compute(B, acc);
          after(lane_off, acc);
          sched_fence();
          lgkm_wait0();
        });
        pin_v(sc[S]);
        y = fmaf(scale_of_pair<S>(sc[S]), acc[0], y);  // g & 1 == S: g0 is even
      }
    });
  }
  return y;
}

__device__ __forceinline__ void c4_task(const ql_gemv_desc* __restrict__ descs, int count, int64_t t,
                                        const uint8_t* lut, int lane) {
  const ql_gemv_desc& d = descs[find_desc(descs, count, t)];
  if (d.grid != QL_GRID_C4) return;  // not a container: nothing of it is read
  if (!task_in_entry(d, t)) return;
  const int64_t slab = t - d.slab_begin;
  const int K = d.K, G8 = (K / kGroup + 7) / 8;
  const uint8_t* codes = static_cast<const uint8_t*>(d.packed) + slab * (int64_t)kSlab * (K / 2);
  const float y = c4_slab(codes, d.pscales + slab * (int64_t)G8 * kSlab * 8, d.x, K, lane, lut);
  const int64_t row = slab * kSlab + lane;
  // a global store (a flat one would also hold up the next task's lgkmcnt waits)
  if (row < d.N) ((__attribute__((address_space(1))) float*)d.y)[row] = y;
}

__global__ void __launch_bounds__(kC4Waves * 64, 4) c4_gemv_kernel(ql_gemv_desc desc, int count, int64_t total) {
  __shared__ __attribute__((aligned(16))) uint8_t lut[kC4LutBytes];
  build_c4_lut(lut);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  for (int64_t t = (int64_t)blockIdx.x * kC4Waves + wave; t < total; t += (int64_t)gridDim.x * kC4Waves)
    c4_task(&desc, count, t, lut, lane);
}

// Persistent launch over many containers, scheduled exactly as the native
// grouped GEMV: first task by wave index, then draws from the task queues, each
// made when the previous task starts.
__global__ void __launch_bounds__(kC4Waves * 64, 4) c4_gemv_grouped_kernel(const ql_gemv_desc* __restrict__ descs,
                                                                          int count, int64_t total,
                                                                          uint32_t* __restrict__ sched) {
  __shared__ __attribute__((aligned(16))) uint8_t lut[kC4LutBytes];
  build_c4_lut(lut);
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  TaskQueues tq(sched, total, (int64_t)gridDim.x * kC4Waves);
  int64_t t = (int64_t)blockIdx.x * kC4Waves + wave;
  if (t >= total) t = tq.next(lane);
  while (t >= 0) {
    const uint32_t claim = tq.claim(lane);
    c4_task(descs, count, t, lut, lane);
    t = tq.resolve(claim, lane);
  }
  tq.checkout(lane);
}

int c4_grid_size(int64_t tasks) {
  const int slots = device_cu_count() * kC4WgPerCu;
  const int64_t wg_needed = (tasks + kC4Waves - 1) / kC4Waves;
  return (int)(wg_needed < slots ? wg_needed : slots);
}

}  // namespace

hipError_t launch_c4_gemv(const MatArgs& a, hipStream_t stream) {
  const int64_t nslabs = ((int64_t)a.N + kSlab - 1) / kSlab;
  const ql_gemv_desc d{a.packed, a.pscales, nullptr, nullptr, a.x, a.y, a.N, a.K, QL_GRID_C4, 0, 1, 0, 0};
  hipLaunchKernelGGL(c4_gemv_kernel, dim3(c4_grid_size(nslabs)), dim3(kC4Waves * 64), 0, stream, d, 1, nslabs);
  return hipGetLastError();
}

hipError_t launch_c4_gemv_grouped(const ql_gemv_desc* descs, int32_t count, int64_t total_slabs, uint32_t* sched,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(c4_gemv_grouped_kernel, dim3(c4_grid_size(total_slabs)), dim3(kC4Waves * 64), 0, stream, descs,
                     count, total_slabs, sched);
  return hipGetLastError();
}

}  // namespace ql
