// Internal launcher declarations of the qlinear library (not part of the C ABI).
#pragma once

#include "ql_device.hpp"

namespace ql {

// Records the message qlinear_last_error() returns on this thread; returns st.
ql_status set_error(ql_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

hipError_t launch_quantize(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const float* W, int8_t* codes,
                           uint16_t* scales, hipStream_t stream);
hipError_t launch_pack(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                       const int8_t* codes, uint8_t* packed, hipStream_t stream);
hipError_t launch_c4_to_packed(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                               const uint8_t* c4, uint8_t* packed, hipStream_t stream);
hipError_t launch_c4_pack(int64_t N, int64_t K, const int8_t* codes, uint8_t* c4, hipStream_t stream);
hipError_t launch_c4_unpack(int64_t N, int64_t K, const uint8_t* c4, int8_t* codes, hipStream_t stream);
// mode 0: int8 codes, 1: fp32 c*s, 2: bf16 bits of c*s
hipError_t launch_unpack(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                         const uint8_t* packed, const uint16_t* pscales, int mode, void* out, hipStream_t stream);
// dir 0: pack, 1: unpack
hipError_t launch_scales(int64_t N, int64_t K, uint16_t* scales, uint16_t* ps, int dir, hipStream_t stream);

// One matrix of a GEMV / GEMM.
struct MatArgs {
  const uint8_t* packed;
  const uint16_t* pscales;
  const int8_t* blk_grid;
  const int64_t* blk_off;
  const uint16_t* x;
  float* y;
  int32_t N, K, grid;
};

// The decode GEMV (ql_gemv.hip): one lane per weight row, LDS decode tables, products on
// 4x4x4 MFMA; 1 <= M <= 16 tokens.  A single matrix (static slab striding) or a grouped
// descriptor list (task queues and split-K state in `sched`).
hipError_t launch_gemv(const MatArgs& a, int M, hipStream_t stream);
hipError_t launch_gemv_grouped(const ql_gemv_desc* descs, int32_t count, int64_t total_tasks, int M, uint32_t* sched,
                               hipStream_t stream);
hipError_t launch_c4_gemv(const MatArgs& a, hipStream_t stream);
hipError_t launch_c4_gemv_grouped(const ql_gemv_desc* descs, int32_t count, int64_t total_slabs, uint32_t* sched,
                                  hipStream_t stream);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(const MatArgs& a, int M, void* workspace, size_t ws_bytes, hipStream_t stream);
// Grouped large-tile GEMM (M >= 16): the host plan sorts and splits the entries (slab_begin =
// first task, kparts = K splits, ws_begin = first partial-sum float) and returns the task
// count; the launch runs every entry's tiles and then the reduction of the split ones.
int64_t gemm_grouped_plan(ql_gemv_desc* descs, int32_t count, int64_t M, int64_t* ws_floats);
hipError_t launch_gemm_grouped(const ql_gemv_desc* descs, int32_t count, int64_t total, int M, float* ws,
                               int64_t ws_floats, hipStream_t stream);
// large: the large-tile kernel (bf16 c*s operands), else the small-batch exact kernel
hipError_t launch_gemm_as(const MatArgs& a, int M, void* workspace, size_t ws_bytes, bool large, hipStream_t stream);

hipError_t launch_validate_codes(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int8_t* codes,
                                 uint32_t* counts, hipStream_t stream);
hipError_t launch_validate_packed(int64_t N, int64_t K, int grid, const int8_t* blk_grid, const int64_t* blk_off,
                                  const uint8_t* packed, uint32_t* counts, hipStream_t stream);
hipError_t launch_rtn_noise(int64_t N, int64_t K, const float* W, double* noise, hipStream_t stream);
hipError_t launch_block_sensitivity(int64_t N, int64_t K, const uint16_t* x, const float* grad, double* S,
                                    hipStream_t stream);
// 0, -2 when the cheapest allowed grids exceed the budget
int allocate_grids(const ql_alloc_unit* units, int64_t count, double budget, const double* bits, int8_t* out,
                   double* lam_out);

int64_t lb_latent_rows(int64_t r);
int64_t lb_u_row_bytes(int64_t r);
size_t lb_workspace_bytes(int64_t d_out, int64_t d_in, int64_t r);
hipError_t launch_lb_pack(int64_t d_out, int64_t d_in, int64_t r, const int8_t* u_signs, const int8_t* v_signs,
                          uint8_t* u_bits, uint8_t* v_bits, hipStream_t stream);
hipError_t launch_lb_gemv(const ql_littlebit& w, const uint16_t* x, float* y, void* ws, hipStream_t stream);

int device_cu_count();
// read-bandwidth probe over `bytes` (a multiple of 1024) of device memory; out ^= XOR of the data
hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* out, hipStream_t stream);
// waves of a persistent grouped launch at batch size M
int64_t grouped_wave_slots(int M);

}  // namespace ql
