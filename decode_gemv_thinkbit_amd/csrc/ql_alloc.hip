// Grid allocation: rounding noise per grid on the GPU, and the multiple-choice
// knapsack over grids on the host.
//
// ThinkBit summary page (onedev.kr/papers/1416), section "How it differs",
// stage 1 (Allocate): a layer's sensitivity S -- the product of the squared
// norms of its input activations and of its output gradients -- times the
// rounding noise of a grid approximates the loss increase of storing the
// layer on that grid; ternary / 2-bit / 3-bit are then chosen per layer under
// one bit budget for the whole decoder, a multiple-choice knapsack solved by
// Lagrangian relaxation.  The units here are whatever the caller groups
// (a linear, or a 128-row block, the granularity the packed layout stores).
#include <algorithm>
#include <vector>

#include "ql_internal.hpp"

namespace ql {

// ---------------------------------------------------------------- rounding noise
// One workgroup per (128-row block, grid); each wave takes (row, group) items
// in a fixed order, 64 lanes x 2 weights, and quantizes them exactly as
// quantize_kernel does.  Squared errors are summed in fp64: per lane, then a
// fixed shuffle tree per item, then per wave in item order, then the four
// waves in order, so the result is deterministic.
__global__ void __launch_bounds__(256) rtn_noise_kernel(int64_t N, int64_t K, const float* __restrict__ W,
                                                        double* __restrict__ noise) {
  const int64_t b = blockIdx.x;
  const int gr = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cmin = grid_cmin(gr), cmax = grid_cmax(gr);
  const int64_t G = K / kGroup, r0 = b * kBlock;
  const int64_t rows = (N - r0) < kBlock ? (N - r0) : kBlock;
  double wsum = 0.0;
  for (int64_t it = wave; it < rows * G; it += 4) {
    const int64_t n = r0 + it / G, g = it % G;
    const float2 v = reinterpret_cast<const float2*>(W + n * K + g * kGroup)[lane];
    float a = fmaxf(fabsf(v.x), fabsf(v.y));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
    const double s = (double)bf16_bits_to_f32(f32_to_bf16_bits(a / (float)(-cmin)));
    double c0 = 0.0, c1 = 0.0;
    if (s != 0.0) {
      c0 = fmin(fmax(rint((double)v.x / s), (double)cmin), (double)cmax);
      c1 = fmin(fmax(rint((double)v.y / s), (double)cmin), (double)cmax);
    }
    const double e0 = (double)v.x - c0 * s, e1 = (double)v.y - c1 * s;
    double e = e0 * e0 + e1 * e1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) e += __shfl_xor(e, off, 64);
    wsum += e;  // identical in every lane
  }
  __shared__ double part[4];
  if (lane == 0) part[wave] = wsum;
  __syncthreads();
  if (threadIdx.x == 0) noise[b * 3 + gr] = ((part[0] + part[1]) + part[2]) + part[3];
}

hipError_t launch_rtn_noise(int64_t N, int64_t K, const float* W, double* noise, hipStream_t stream) {
  const int64_t nb = (N + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(rtn_noise_kernel, dim3((unsigned)nb, 3), dim3(256), 0, stream, N, K, W, noise);
  return hipGetLastError();
}

// ---------------------------------------------------------------- sensitivity
// S of every 128-row block of a linear: ||x||^2 times the block's sum of
// squared output gradients.  Each square is exact in fp64 (a bf16 or fp32
// value squared), and both sums run in ascending index order in one lane, so
// the result does not depend on the launch shape.  Offline work: one
// workgroup per block, the x norm recomputed by each (K is a row length).
__global__ void __launch_bounds__(64) block_sensitivity_kernel(int64_t N, int64_t K, const uint16_t* __restrict__ x,
                                                               const float* __restrict__ grad,
                                                               double* __restrict__ S) {
  if (threadIdx.x != 0) return;
  const int64_t b = blockIdx.x;
  double xs = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    const double v = (double)bf16_bits_to_f32(x[k]);
    xs += v * v;
  }
  double gs = 0.0;
  const int64_t n1 = (b + 1) * kBlock < N ? (b + 1) * kBlock : N;
  for (int64_t n = b * kBlock; n < n1; ++n) {
    const double g = (double)grad[n];
    gs += g * g;
  }
  S[b] = xs * gs;
}

hipError_t launch_block_sensitivity(int64_t N, int64_t K, const uint16_t* x, const float* grad, double* S,
                                    hipStream_t stream) {
  const int64_t nb = (N + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(block_sensitivity_kernel, dim3((unsigned)nb), dim3(64), 0, stream, N, K, x, grad, S);
  return hipGetLastError();
}

// ---------------------------------------------------------------- knapsack (host)
namespace {

struct Alloc {
  const ql_alloc_unit* u;
  int64_t count;
  const double* bits;
  int order[3];  // grids by increasing bits (ties by id)

  // allowed grid of unit i minimising S*E[g] + lam*(n*bits[g]); the first
  // minimum in increasing bits wins, so ties go to fewer bits
  int pick(int64_t i, double lam) const {
    int best = -1;
    double bc = 0.0;
    for (int t = 0; t < 3; ++t) {
      const int g = order[t];
      if (!(u[i].allowed >> g & 1u)) continue;
      const double c = u[i].sensitivity * u[i].noise[g] + lam * ((double)u[i].weights * bits[g]);
      if (best < 0 || c < bc) {
        best = g;
        bc = c;
      }
    }
    return best;
  }
  double used(double lam) const {
    double s = 0.0;
    for (int64_t i = 0; i < count; ++i) s += (double)u[i].weights * bits[pick(i, lam)];
    return s;
  }
};

}  // namespace

// Bits used fall as the multiplier grows, and a unit's choice changes only
// where two of its costs cross, so assignments are constant between
// consecutive crossings.  Each interval is represented by an interior point
// (0, the midpoints, twice the last crossing), where no cost comparison sits
// on a rounding tie; the first point whose bits fit is found by binary search.
int allocate_grids(const ql_alloc_unit* units, int64_t count, double budget, const double* bits, int8_t* out,
                   double* lam_out) {
  Alloc a{units, count, bits, {0, 1, 2}};
  std::sort(a.order, a.order + 3, [&](int x, int y) { return bits[x] < bits[y] || (bits[x] == bits[y] && x < y); });
  double total_n = 0.0;
  for (int64_t i = 0; i < count; ++i) total_n += (double)units[i].weights;
  const double cap = budget * total_n;
  std::vector<double> cand{0.0};
  cand.reserve(1 + 3 * (size_t)count);
  for (int64_t i = 0; i < count; ++i)
    for (int x = 0; x < 3; ++x)
      for (int y = 0; y < 3; ++y) {
        if (!(units[i].allowed >> x & 1u) || !(units[i].allowed >> y & 1u) || !(bits[x] < bits[y])) continue;
        const double S = units[i].sensitivity;
        const double lam = (S * units[i].noise[x] - S * units[i].noise[y]) / ((double)units[i].weights * (bits[y] - bits[x]));
        if (lam > 0.0) cand.push_back(lam);
      }
  std::sort(cand.begin(), cand.end());
  cand.erase(std::unique(cand.begin(), cand.end()), cand.end());
  std::vector<double> pts{0.0};
  if (cand.size() > 1) pts.push_back(0.5 * cand[1]);
  for (size_t j = 1; j < cand.size(); ++j)
    pts.push_back(j + 1 < cand.size() ? 0.5 * (cand[j] + cand[j + 1]) : 2.0 * cand[j]);
  if (a.used(pts.back()) > cap) return -2;
  size_t lo = 0, hi = pts.size() - 1;  // used(pts[hi]) <= cap
  while (lo < hi) {
    const size_t mid = (lo + hi) / 2;
    if (a.used(pts[mid]) <= cap) hi = mid; else lo = mid + 1;
  }
  for (int64_t i = 0; i < count; ++i) out[i] = (int8_t)a.pick(i, pts[lo]);
  if (lam_out) *lam_out = pts[lo];
  return 0;
}

}  // namespace ql
