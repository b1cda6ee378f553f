// Pure HBM read probe: the bandwidth reference the decode kernels are judged
// against beside the nominal peak.  Waves sweep the buffer in 1 KB blocks
// (block b read by wave b mod nwaves, four blocks in flight per wave, one
// workgroup of 8 waves per CU), with the same 128-bit non-temporal buffer
// loads as the GEMV's code stream.  Of the access patterns measured on this
// device (per-wave contiguous streams, dynamically handed-out tasks, this
// interleaved sweep at 8 / 16 / 32 waves per CU), this one read fastest.
// Every byte is folded into an XOR so that the loads are not dead code and the
// result can be checked.
#include "ql_internal.hpp"

namespace ql {

namespace {

constexpr int kProbeWaves = 8;
constexpr int kProbeInFlight = 4;

typedef int i32x4p_t __attribute__((ext_vector_type(4)));

// p as a wave-uniform value.  Both halves go through uint32_t: readfirstlane
// returns int, and an int low half would sign-extend into the high word.
__device__ __forceinline__ void* probe_uniform(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (void*)(((uint64_t)hi << 32) | lo);
}

__global__ void __launch_bounds__(kProbeWaves * 64) read_probe_kernel(const uint8_t* buf, int64_t nblk, uint32_t* out) {
  __shared__ uint32_t part[kProbeWaves][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nwaves = (int64_t)gridDim.x * kProbeWaves;
  const int64_t w = (int64_t)blockIdx.x * kProbeWaves + wave;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      probe_uniform(buf), (short)0, __builtin_amdgcn_readfirstlane((int)(uint32_t)(nblk * 1024)), 0x00020000);
  i32x4p_t acc = {0, 0, 0, 0};
  int64_t b = w;
  for (; b + (kProbeInFlight - 1) * nwaves < nblk; b += kProbeInFlight * nwaves) {
    i32x4p_t v[kProbeInFlight];
#pragma unroll
    for (int r = 0; r < kProbeInFlight; ++r)
      v[r] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (uint32_t)((b + r * nwaves) * 1024) + lane * 16u, 0, 2);
#pragma unroll
    for (int r = 0; r < kProbeInFlight; ++r) acc ^= v[r];
  }
  for (; b < nblk; b += nwaves) acc ^= __builtin_amdgcn_raw_buffer_load_b128(rsrc, (uint32_t)(b * 1024) + lane * 16u, 0, 2);
#pragma unroll
  for (int j = 0; j < 4; ++j) part[wave][lane][j] = (uint32_t)acc[j];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t x = 0;
#pragma unroll
      for (int q = 0; q < kProbeWaves; ++q) x ^= part[q][lane][j];
      __hip_atomic_fetch_xor(out + 4 * lane + j, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* out, hipStream_t stream) {
  const int64_t nblk = bytes / 1024;
  const int64_t want = (nblk + kProbeWaves - 1) / kProbeWaves;
  const int grid = (int)(want < device_cu_count() ? want : device_cu_count());
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kProbeWaves * 64), 0, stream,
                     static_cast<const uint8_t*>(buf), nblk, out);
  return hipGetLastError();
}

}  // namespace ql
