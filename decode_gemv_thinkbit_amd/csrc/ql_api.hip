// C ABI of the qlinear library: argument checks, then dispatch to the launchers.
// Every check happens before anything is enqueued.
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cmath>
#include <cstring>

#include "ql_internal.hpp"

namespace {

thread_local char g_err[512] = "";

ql_status fail(ql_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

ql_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return QL_OK;
  return fail(QL_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool grid_valid(int g) { return g == QL_GRID_T || g == QL_GRID_I2 || g == QL_GRID_I3; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kMaxGroupedK = (int64_t)1 << 26;  // 2 * 16 tokens * K bytes of x stay below 2^31

ql_status check_shape(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return fail(QL_EINVAL, "N and K must be positive (N=%lld, K=%lld)", (long long)N, (long long)K);
  if (K % QL_GROUP) return fail(QL_EINVAL, "K=%lld is not a multiple of %d", (long long)K, QL_GROUP);
  if (N > kMaxDim || K > kMaxDim || N * K > ((int64_t)1 << 40))
    return fail(QL_EINVAL, "shape too large (N=%lld, K=%lld)", (long long)N, (long long)K);
  return QL_OK;
}

ql_status check_grid(int grid, const int8_t* blk_grid, const int64_t* blk_off, bool need_off) {
  if (grid == QL_GRID_MIXED) {
    if (!blk_grid) return fail(QL_EINVAL, "mixed grid needs blk_grid");
    if (need_off && !blk_off) return fail(QL_EINVAL, "mixed grid needs blk_off");
    return QL_OK;
  }
  if (!grid_valid(grid)) return fail(QL_EINVAL, "unknown grid id %d", grid);
  return QL_OK;
}

ql_status check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (!p) return fail(QL_EINVAL, "null pointer argument");
    if (!aligned16(p)) return fail(QL_EINVAL, "pointer %p is not 16-byte aligned", p);
  }
  return QL_OK;
}

}  // namespace

ql_status ql::set_error(ql_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

namespace {

#define QL_TRY(x)                    \
  do {                               \
    ql_status _s = (x);              \
    if (_s != QL_OK) return _s;      \
  } while (0)

}  // namespace

extern "C" {

int qlinear_version(void) { return QL_LAYOUT_VERSION; }

const char* qlinear_last_error(void) { return g_err; }

int64_t qlinear_row_bytes(int grid, int64_t K) {
  if (!grid_valid(grid) || K <= 0 || K % QL_GROUP || K > kMaxDim) return 0;
  return ql::row_bytes(grid, K);
}

ql_status qlinear_block_offsets(int64_t N, int64_t K, const int8_t* blk_grid, int64_t* off) {
  QL_TRY(check_shape(N, K));
  if (!blk_grid || !off) return fail(QL_EINVAL, "null pointer argument");
  const int64_t S = (N + QL_SLAB - 1) / QL_SLAB, nb = (N + QL_BLOCK - 1) / QL_BLOCK;
  off[0] = 0;
  for (int64_t b = 0; b < nb; ++b) {
    if (!grid_valid(blk_grid[b])) return fail(QL_EINVAL, "blk_grid[%lld] = %d is not a grid", (long long)b, blk_grid[b]);
    const int64_t slabs = (S - 2 * b) < 2 ? (S - 2 * b) : 2;
    off[b + 1] = off[b] + slabs * QL_SLAB * ql::row_bytes(blk_grid[b], K);
  }
  return QL_OK;
}

int64_t qlinear_packed_bytes(int64_t N, int64_t K, int grid) {
  if (check_shape(N, K) != QL_OK || !grid_valid(grid)) return 0;
  return ((N + QL_SLAB - 1) / QL_SLAB) * QL_SLAB * ql::row_bytes(grid, K);
}

int64_t qlinear_packed_scales_len(int64_t N, int64_t K) {
  if (check_shape(N, K) != QL_OK) return 0;
  return ((N + QL_SLAB - 1) / QL_SLAB) * ((K / QL_GROUP + 7) / 8) * QL_SLAB * 8;
}

ql_status qlinear_quantize(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const float* W, int8_t* codes,
                           uint16_t* scales, hipStream_t stream) {
  QL_TRY(check_shape(N, K));
  QL_TRY(check_grid(grid, blk_grid, nullptr, false));
  QL_TRY(check_ptrs({W, codes, scales}));
  return hip_status(ql::launch_quantize(N, K, grid, blk_grid, W, codes, scales, stream), "quantize launch");
}

ql_status qlinear_pack(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                       const int8_t* codes, const uint16_t* scales, void* packed, uint16_t* pscales,
                       hipStream_t stream) {
  QL_TRY(check_shape(N, K));
  QL_TRY(check_grid(grid, blk_grid, blk_off, true));
  QL_TRY(check_ptrs({codes, packed}));
  if ((scales == nullptr) != (pscales == nullptr)) return fail(QL_EINVAL, "scales and pscales: give both or neither");
  if (scales) QL_TRY(check_ptrs({scales, pscales}));
  QL_TRY(hip_status(ql::launch_pack(N, K, grid, blk_grid, blk_off, codes, static_cast<uint8_t*>(packed), stream),
                    "pack launch"));
  if (!scales) return QL_OK;
  return hip_status(ql::launch_scales(N, K, const_cast<uint16_t*>(scales), pscales, 0, stream), "pack scales launch");
}

ql_status qlinear_pack_scales(int64_t N, int64_t K, const uint16_t* scales, uint16_t* pscales, hipStream_t stream) {
  QL_TRY(check_shape(N, K));
  QL_TRY(check_ptrs({scales, pscales}));
  return hip_status(ql::launch_scales(N, K, const_cast<uint16_t*>(scales), pscales, 0, stream), "pack_scales launch");
}

ql_status qlinear_unpack(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                         const void* packed, int8_t* codes, hipStream_t stream) {
  QL_TRY(check_shape(N, K));
  QL_TRY(check_grid(grid, blk_grid, blk_off, true));
  QL_TRY(check_ptrs({packed, codes}));
  return hip_status(ql::launch_unpack(N, K, grid, blk_grid, blk_off, static_cast<const uint8_t*>(packed), nullptr, 0,
                                      codes, stream),
                    "unpack launch");
}

ql_status qlinear_unpack_scales(int64_t N, int64_t K, const uint16_t* pscales, uint16_t* scales, hipStream_t stream) {
  QL_TRY(check_shape(N, K));
  QL_TRY(check_ptrs({pscales, scales}));
  return hip_status(ql::launch_scales(N, K, scales, const_cast<uint16_t*>(pscales), 1, stream),
                    "unpack_scales launch");
}

ql_status qlinear_dequant(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                          const void* packed, const uint16_t* pscales, int out_bf16, void* out, hipStream_t stream) {
  QL_TRY(check_shape(N, K));
  QL_TRY(check_grid(grid, blk_grid, blk_off, true));
  QL_TRY(check_ptrs({packed, pscales, out}));
  return hip_status(ql::launch_unpack(N, K, grid, blk_grid, blk_off, static_cast<const uint8_t*>(packed), pscales,
                                      out_bf16 ? 2 : 1, out, stream),
                    "dequant launch");
}

ql_status qlinear_validate_codes(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int8_t* codes,
                                 uint32_t* counts, hipStream_t stream) {
  QL_TRY(check_shape(N, K));
  QL_TRY(check_grid(grid, blk_grid, nullptr, false));
  QL_TRY(check_ptrs({codes, counts}));
  return hip_status(ql::launch_validate_codes(N, K, grid, blk_grid, codes, counts, stream), "validate_codes launch");
}

ql_status qlinear_validate_packed(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                                  const void* packed, uint32_t* counts, hipStream_t stream) {
  QL_TRY(check_shape(N, K));
  QL_TRY(check_grid(grid, blk_grid, blk_off, true));
  QL_TRY(check_ptrs({packed, counts}));
  return hip_status(ql::launch_validate_packed(N, K, grid, blk_grid, blk_off, static_cast<const uint8_t*>(packed),
                                               counts, stream),
                    "validate_packed launch");
}

static ql_status mat_args(int64_t M, int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                          const void* packed, const uint16_t* pscales, const uint16_t* x, float* y, ql::MatArgs* a) {
  QL_TRY(check_shape(N, K));
  QL_TRY(check_grid(grid, blk_grid, blk_off, true));
  QL_TRY(check_ptrs({packed, pscales, x, y}));
  if (N >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31)) return fail(QL_EINVAL, "N and K must be below 2^31");
  *a = ql::MatArgs{static_cast<const uint8_t*>(packed), pscales, blk_grid, blk_off, x, y, (int32_t)N, (int32_t)K, grid};
  (void)M;
  return QL_OK;
}

ql_status qlinear_gemv(int64_t M, int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                       const void* packed, const uint16_t* pscales, const uint16_t* x, float* y, hipStream_t stream) {
  if (M < 1 || M > 16) return fail(QL_EINVAL, "gemv needs 1 <= M <= 16 (M=%lld)", (long long)M);
  ql::MatArgs a;
  QL_TRY(mat_args(M, N, K, grid, blk_grid, blk_off, packed, pscales, x, y, &a));
  if (K > ((int64_t)1 << 26)) return fail(QL_EINVAL, "gemv needs K <= 2^26 (K=%lld)", (long long)K);
  return hip_status(ql::launch_gemv(a, (int)M, stream), "gemv launch");
}

int64_t qlinear_grouped_prepare_split(ql_gemv_desc* descs, int32_t count, int64_t min_tasks, int64_t* state_words) {
  if (!descs || count <= 0) return fail(QL_EINVAL, "empty descriptor list"), -1;
  const bool containers = descs[0].grid == QL_GRID_C4;
  int64_t slabs = 0;
  for (int32_t i = 0; i < count; ++i) {
    const ql_gemv_desc& d = descs[i];
    if (check_shape(d.N, d.K) != QL_OK) return -1;
    if ((d.grid == QL_GRID_C4) != containers)
      return fail(QL_EINVAL, "descriptor %d: a list must not mix 4-bit containers and native grids", i), -1;
    if (!containers && check_grid(d.grid, d.blk_grid, d.blk_off, true) != QL_OK) return -1;
    if (check_ptrs({d.packed, d.pscales, d.x, d.y}) != QL_OK) return -1;
    // the GEMV kernel addresses up to 16 tokens' activations through one 32-bit buffer range
    if (d.K > kMaxGroupedK)
      return fail(QL_EINVAL, "descriptor %d: K=%d above the grouped launch's limit %lld", i, d.K,
                  (long long)kMaxGroupedK), -1;
    if (d.kparts < 0) return fail(QL_EINVAL, "descriptor %d: kparts must be >= 0", i), -1;
    if (containers && d.kparts > 1) return fail(QL_EINVAL, "descriptor %d: containers are not split", i), -1;
    slabs += (d.N + QL_SLAB - 1) / QL_SLAB;
  }
  // parts per slab: forced, or enough for min_tasks where the rows have periods for it
  const int64_t need = (!containers && min_tasks > slabs) ? (min_tasks + slabs - 1) / slabs : 1;
  for (int32_t i = 0; i < count; ++i) {
    ql_gemv_desc& d = descs[i];
    const int64_t periods = (d.K + ql::kPeriodK - 1) / ql::kPeriodK;
    const int64_t want = std::min<int64_t>(d.kparts > 0 ? d.kparts : need, QL_MAX_KPARTS);
    d.kparts = (int32_t)std::min(want, periods);
    d.reserved = 0;
  }
  // longest tasks first: the tail of the launch is then made of short tasks
  std::stable_sort(descs, descs + count, [](const ql_gemv_desc& a, const ql_gemv_desc& b) {
    return (int64_t)a.K * b.kparts > (int64_t)b.K * a.kparts;
  });
  int64_t total = 0, words = QL_SCHED_WORDS;
  words = (words + 63) / 64 * 64;
  bool split = false;
  for (int32_t i = 0; i < count; ++i) {
    ql_gemv_desc& d = descs[i];
    const int64_t ns = (d.N + QL_SLAB - 1) / QL_SLAB;
    if (total + ns * d.kparts >= ((int64_t)1 << 31)) return fail(QL_EINVAL, "too many tasks"), -1;
    d.slab_begin = (int32_t)total;
    total += ns * d.kparts;
    d.ws_begin = 0;
    if (d.kparts > 1) {
      d.ws_begin = words;
      words += ns * ql::kCounterWords + ns * d.kparts * ql::kPartWords;
      split = true;
    }
  }
  if (state_words) *state_words = split ? words : QL_SCHED_WORDS;
  return total;
}

int64_t qlinear_grouped_prepare(ql_gemv_desc* descs, int32_t count) {
  if (!descs || count <= 0) return fail(QL_EINVAL, "empty descriptor list"), -1;
  for (int32_t i = 0; i < count; ++i) descs[i].kparts = 1;
  return qlinear_grouped_prepare_split(descs, count, 0, nullptr);
}

int64_t qlinear_grouped_wave_slots(int32_t M) {
  if (M < 1 || M > 16) return fail(QL_EINVAL, "wave slots: M=%d outside 1..16", M), -1;
  return ql::grouped_wave_slots(M);
}

ql_status qlinear_gemv_grouped(const ql_gemv_desc* descs, int32_t count, int64_t total_tasks, int32_t M,
                               uint32_t* sched, hipStream_t stream) {
  if (M < 1 || M > 16) return fail(QL_EINVAL, "grouped gemv needs 1 <= M <= 16 (M=%d)", M);
  if (count <= 0 || total_tasks <= 0 || total_tasks >= ((int64_t)1 << 31))
    return fail(QL_EINVAL, "bad count (%d) or task total (%lld)", count, (long long)total_tasks);
  QL_TRY(check_ptrs({descs, sched}));
  return hip_status(ql::launch_gemv_grouped(descs, count, total_tasks, M, sched, stream), "grouped gemv launch");
}

size_t qlinear_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) { return ql::gemm_workspace_bytes(M, N, K); }

// ---------------------------------------------------------------- grid allocation
ql_status qlinear_rtn_noise(int64_t N, int64_t K, const float* W, double* noise, hipStream_t stream) {
  QL_TRY(check_shape(N, K));
  QL_TRY(check_ptrs({W, noise}));
  return hip_status(ql::launch_rtn_noise(N, K, W, noise, stream), "rtn_noise launch");
}

ql_status qlinear_block_sensitivity(int64_t N, int64_t K, const uint16_t* x, const float* grad, double* S,
                                     hipStream_t stream) {
  if (N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim)
    return fail(QL_EINVAL, "block sensitivity needs positive N and K (N=%lld, K=%lld)", (long long)N, (long long)K);
  QL_TRY(check_ptrs({x, grad, S}));
  return hip_status(ql::launch_block_sensitivity(N, K, x, grad, S, stream), "block_sensitivity launch");
}

ql_status qlinear_allocate(const ql_alloc_unit* units, int64_t count, double budget_bits, const double* grid_bits,
                           int8_t* grid_out, double* lambda_out) {
  if (!units || !grid_out || count <= 0) return fail(QL_EINVAL, "allocate needs units, an output and count > 0");
  static const double kDefaultBits[3] = {1.584962500721156 + 0.125, 2.125, 3.125};  // log2(3) + 1/8, ...
  const double* bits = grid_bits ? grid_bits : kDefaultBits;
  for (int g = 0; g < 3; ++g)
    if (!(bits[g] > 0.0) || !std::isfinite(bits[g])) return fail(QL_EINVAL, "grid_bits[%d] must be positive", g);
  if (!(budget_bits > 0.0) || !std::isfinite(budget_bits)) return fail(QL_EINVAL, "budget must be positive");
  for (int64_t i = 0; i < count; ++i) {
    const ql_alloc_unit& u = units[i];
    bool ok = u.weights > 0 && u.sensitivity >= 0.0 && std::isfinite(u.sensitivity) && (u.allowed & 7u) &&
              !(u.allowed & ~7u);
    for (int g = 0; g < 3; ++g) ok = ok && u.noise[g] >= 0.0 && std::isfinite(u.noise[g]);
    if (!ok) return fail(QL_EINVAL, "unit %lld: bad weights, sensitivity, noise or allowed mask", (long long)i);
  }
  if (ql::allocate_grids(units, count, budget_bits, bits, grid_out, lambda_out) != 0)
    return fail(QL_EINVAL, "budget %.4f bits per weight is below the cheapest allowed grids", budget_bits);
  return QL_OK;
}

// ---------------------------------------------------------------- LittleBit
static bool lb_shape_ok(int64_t d_out, int64_t d_in, int64_t rank) {
  return d_out > 0 && d_in > 0 && rank > 0 && d_in % 128 == 0 && d_out <= kMaxDim && d_in <= kMaxDim &&
         rank <= d_out + d_in && rank <= kMaxDim;
}

double qlinear_lb_bpw(int64_t d_out, int64_t d_in, int64_t rank) {
  if (d_out <= 0 || d_in <= 0 || rank < 0) return 0.0;
  return ((2.0 * rank + 32.0) * (double)(d_out + d_in) + 32.0 * rank) / ((double)d_out * (double)d_in);
}

int64_t qlinear_lb_rank(int64_t d_out, int64_t d_in, double bpw) {
  if (d_out <= 0 || d_in <= 0 || !(bpw > 0.0)) return 0;
  // b(r) is linear in r: solve, then step to the largest r with b(r) <= bpw
  const double per = (2.0 * (double)(d_out + d_in) + 32.0) / ((double)d_out * (double)d_in);
  int64_t r = (int64_t)std::floor((bpw - qlinear_lb_bpw(d_out, d_in, 0)) / per);
  if (r < 0) r = 0;
  while (r > 0 && qlinear_lb_bpw(d_out, d_in, r) > bpw) --r;
  while (qlinear_lb_bpw(d_out, d_in, r + 1) <= bpw) ++r;
  return r;
}

int64_t qlinear_lb_u_bytes(int64_t d_out, int64_t rank) {
  if (d_out <= 0 || rank <= 0 || d_out > kMaxDim || rank > kMaxDim) return 0;
  return (d_out + QL_SLAB - 1) / QL_SLAB * QL_SLAB * ql::lb_u_row_bytes(rank);
}

int64_t qlinear_lb_v_bytes(int64_t d_in, int64_t rank) {
  if (d_in <= 0 || d_in % 128 || rank <= 0 || d_in > kMaxDim || rank > kMaxDim) return 0;
  return 2 * ql::lb_latent_rows(rank) * (d_in / 8);
}

ql_status qlinear_lb_pack(int64_t d_out, int64_t d_in, int64_t rank, const int8_t* u_signs, const int8_t* v_signs,
                          void* u_bits, void* v_bits, hipStream_t stream) {
  if (!lb_shape_ok(d_out, d_in, rank))
    return fail(QL_EINVAL, "bad LittleBit shape (d_out=%lld, d_in=%lld, rank=%lld; d_in %% 128 == 0)",
                (long long)d_out, (long long)d_in, (long long)rank);
  QL_TRY(check_ptrs({u_signs, v_signs, u_bits, v_bits}));
  return hip_status(ql::launch_lb_pack(d_out, d_in, rank, u_signs, v_signs, static_cast<uint8_t*>(u_bits),
                                       static_cast<uint8_t*>(v_bits), stream),
                    "lb_pack launch");
}

size_t qlinear_lb_workspace_bytes(int64_t d_out, int64_t d_in, int64_t rank) {
  if (!lb_shape_ok(d_out, d_in, rank)) return 0;
  return ql::lb_workspace_bytes(d_out, d_in, rank);
}

ql_status qlinear_lb_gemv(const ql_littlebit* w, const uint16_t* x, float* y, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (!w) return fail(QL_EINVAL, "null LittleBit weight");
  if (!lb_shape_ok(w->d_out, w->d_in, w->rank))
    return fail(QL_EINVAL, "bad LittleBit shape (d_out=%d, d_in=%d, rank=%d; d_in %% 128 == 0)", w->d_out, w->d_in,
                w->rank);
  QL_TRY(check_ptrs({w->u_bits, w->v_bits, w->g, w->l, w->h, x, y, workspace}));
  const size_t need = ql::lb_workspace_bytes(w->d_out, w->d_in, w->rank);
  if (workspace_bytes < need) return fail(QL_EINVAL, "workspace too small (%zu < %zu)", workspace_bytes, need);
  return hip_status(ql::launch_lb_gemv(*w, x, y, workspace, stream), "lb_gemv launch");
}

// ---------------------------------------------------------------- 4-bit container baseline
int64_t qlinear_c4_bytes(int64_t N, int64_t K) {
  if (check_shape(N, K) != QL_OK) return 0;
  return ((N + QL_SLAB - 1) / QL_SLAB) * QL_SLAB * (K / 2);
}

ql_status qlinear_c4_pack(int64_t N, int64_t K, const int8_t* codes, void* c4, hipStream_t stream) {
  QL_TRY(check_shape(N, K));
  QL_TRY(check_ptrs({codes, c4}));
  return hip_status(ql::launch_c4_pack(N, K, codes, static_cast<uint8_t*>(c4), stream), "c4_pack launch");
}

ql_status qlinear_c4_unpack(int64_t N, int64_t K, const void* c4, int8_t* codes, hipStream_t stream) {
  QL_TRY(check_shape(N, K));
  QL_TRY(check_ptrs({c4, codes}));
  return hip_status(ql::launch_c4_unpack(N, K, static_cast<const uint8_t*>(c4), codes, stream), "c4_unpack launch");
}

ql_status qlinear_c4_to_packed(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                               const void* c4, void* packed, hipStream_t stream) {
  QL_TRY(check_shape(N, K));
  QL_TRY(check_grid(grid, blk_grid, blk_off, true));
  QL_TRY(check_ptrs({c4, packed}));
  return hip_status(ql::launch_c4_to_packed(N, K, grid, blk_grid, blk_off, static_cast<const uint8_t*>(c4),
                                            static_cast<uint8_t*>(packed), stream),
                    "c4_to_packed launch");
}

ql_status qlinear_c4_gemv(int64_t M, int64_t N, int64_t K, const void* c4, const uint16_t* pscales, const uint16_t* x,
                          float* y, hipStream_t stream) {
  if (M != 1) return fail(QL_EUNSUPPORTED, "the container GEMV runs batch 1 only (M=%lld)", (long long)M);
  QL_TRY(check_shape(N, K));
  QL_TRY(check_ptrs({c4, pscales, x, y}));
  if (N >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31)) return fail(QL_EINVAL, "N and K must be below 2^31");
  const ql::MatArgs a{static_cast<const uint8_t*>(c4), pscales, nullptr, nullptr, x, y, (int32_t)N, (int32_t)K,
                      QL_GRID_C4};
  return hip_status(ql::launch_c4_gemv(a, stream), "c4_gemv launch");
}

ql_status qlinear_c4_gemv_grouped(const ql_gemv_desc* descs, int32_t count, int64_t total_slabs, int32_t M,
                                  uint32_t* sched, hipStream_t stream) {
  if (M != 1) return fail(QL_EUNSUPPORTED, "the container GEMV runs batch 1 only (M=%d)", M);
  if (count <= 0 || total_slabs <= 0 || total_slabs >= ((int64_t)1 << 31))
    return fail(QL_EINVAL, "bad count (%d) or slab total (%lld)", count, (long long)total_slabs);
  QL_TRY(check_ptrs({descs, sched}));
  return hip_status(ql::launch_c4_gemv_grouped(descs, count, total_slabs, sched, stream), "c4 grouped gemv launch");
}

ql_status qlinear_gemm(int64_t M, int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                       const void* packed, const uint16_t* pscales, const uint16_t* x, float* y, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (M < 1 || M >= ((int64_t)1 << 24)) return fail(QL_EINVAL, "gemm needs 1 <= M < 2^24 (M=%lld)", (long long)M);
  ql::MatArgs a;
  QL_TRY(mat_args(M, N, K, grid, blk_grid, blk_off, packed, pscales, x, y, &a));
  if (workspace_bytes < ql::gemm_workspace_bytes(M, N, K))
    return fail(QL_EINVAL, "workspace too small (%zu < %zu)", workspace_bytes, ql::gemm_workspace_bytes(M, N, K));
  return hip_status(ql::launch_gemm(a, (int)M, workspace, workspace_bytes, stream), "gemm launch");
}

int64_t qlinear_gemm_grouped_prepare(ql_gemv_desc* descs, int32_t count, int64_t M, int64_t* workspace_bytes) {
  if (!descs || count <= 0 || count > 65535) return fail(QL_EINVAL, "grouped gemm needs 1..65535 descriptors"), -1;
  if (M < 16 || M >= ((int64_t)1 << 24))
    return fail(QL_EINVAL, "grouped gemm needs 16 <= M < 2^24 (M=%lld)", (long long)M), -1;
  int64_t tasks = 0;
  for (int32_t i = 0; i < count; ++i) {
    const ql_gemv_desc& d = descs[i];
    if (check_shape(d.N, d.K) != QL_OK) return -1;
    if (d.grid == QL_GRID_C4) return fail(QL_EINVAL, "descriptor %d: the grouped gemm takes native grids", i), -1;
    if (check_grid(d.grid, d.blk_grid, d.blk_off, true) != QL_OK) return -1;
    if (check_ptrs({d.packed, d.pscales, d.x, d.y}) != QL_OK) return -1;
    tasks += ((d.N + 255) / 256) * ((M + 63) / 64) * 16;
    if (tasks >= ((int64_t)1 << 31)) return fail(QL_EINVAL, "too many tasks"), -1;
  }
  int64_t ws = 0;
  const int64_t total = ql::gemm_grouped_plan(descs, count, M, &ws);
  if (workspace_bytes) *workspace_bytes = ws * (int64_t)sizeof(float);
  return total;
}

ql_status qlinear_gemm_grouped(const ql_gemv_desc* descs, int32_t count, int64_t total_tasks, int64_t M,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!descs || count <= 0 || count > 65535) return fail(QL_EINVAL, "grouped gemm needs 1..65535 descriptors");
  if (M < 16 || M >= ((int64_t)1 << 24))
    return fail(QL_EINVAL, "grouped gemm needs 16 <= M < 2^24 (M=%lld)", (long long)M);
  if (total_tasks <= 0 || total_tasks >= ((int64_t)1 << 31)) return fail(QL_EINVAL, "bad task count");
  if (workspace_bytes && !workspace) return fail(QL_EINVAL, "workspace_bytes without a workspace");
  if (workspace) QL_TRY(check_ptrs({workspace}));
  QL_TRY(check_ptrs({descs}));
  return hip_status(ql::launch_gemm_grouped(descs, count, total_tasks, (int)M, static_cast<float*>(workspace),
                                            (int64_t)(workspace_bytes / sizeof(float)), stream),
                    "grouped gemm launch");
}

ql_status qlinear_read_probe(const void* buf, int64_t bytes, uint32_t* out, hipStream_t stream) {
  if (bytes <= 0 || bytes % 1024 || bytes >= ((int64_t)1 << 32))
    return fail(QL_EINVAL, "read probe needs 0 < bytes < 2^32, a multiple of 1024 (bytes=%lld)", (long long)bytes);
  QL_TRY(check_ptrs({buf, out}));
  return hip_status(ql::launch_read_probe(buf, bytes, out, stream), "read probe launch");
}

}  // extern "C"
