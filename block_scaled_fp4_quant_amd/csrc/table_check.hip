// table_check.hip -- the optional device-side validation of a grouped call's routing tables
// (enabled with fp4moe_set_debug_checks).  The GEMM kernels never need it for memory safety (they
// clamp offsets and turn bad rows into NaN); it exists so that a caller can learn that its tables
// break the contract of the CSR layout [CHECK: f16g grouped GEMM, the offsets array of rows packed
// per expert] instead of reading NaN rows or silently clamped segments.
#include "kernels.h"

namespace fp4moe {

namespace {

constexpr int kThreads = 1024;

// One workgroup walks the tables with plain strided loads and keeps, per condition, the smallest
// index that violates it (LDS atomics only).  status[i] = that index, or -1 when none does:
//   0: offsets[0] != 0 (index 0)
//   1: offsets[e + 1] < offsets[e] (index e)
//   2: offsets[E] != total_rows (index E)
//   3: row_ids[p] outside [0, a_rows) (index p; only when row_ids is given)
//   4: kinds[e] outside 0..3 (index e)
__global__ __launch_bounds__(kThreads) void table_check_kernel(const int32_t* __restrict__ offsets, int32_t num_experts,
                                                                 int32_t total_rows, const int32_t* __restrict__ row_ids,
                                                                 int32_t a_rows, const int32_t* __restrict__ kinds,
                                                                 int32_t* __restrict__ status) {
  __shared__ int first[kTableCheckWords];
  const int tid = threadIdx.x;
  if (tid < kTableCheckWords) first[tid] = INT32_MAX;
  __syncthreads();
  if (tid == 0) {
    if (offsets[0] != 0) atomicMin(&first[0], 0);
    if (offsets[num_experts] != total_rows) atomicMin(&first[2], num_experts);
  }
  for (int e = tid; e < num_experts; e += kThreads) {
    if (offsets[e + 1] < offsets[e]) atomicMin(&first[1], e);
    const int kd = kinds[e];
    if (kd < 0 || kd > 3) atomicMin(&first[4], e);
  }
  if (row_ids) {
    for (int p = tid; p < total_rows; p += kThreads) {
      const int r = row_ids[p];
      if (r < 0 || r >= a_rows) atomicMin(&first[3], p);
    }
  }
  __syncthreads();
  if (tid < kTableCheckWords) status[tid] = first[tid] == INT32_MAX ? -1 : first[tid];
}

}  // namespace

hipError_t launch_table_check(const int32_t* offsets, int32_t num_experts, int32_t total_rows, const int32_t* row_ids,
                              int32_t a_rows, const int32_t* kinds, int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(table_check_kernel, dim3(1), dim3(kThreads), 0, stream, offsets, num_experts, total_rows, row_ids,
                     a_rows, kinds, status);
  return hipGetLastError();
}

}  // namespace fp4moe
