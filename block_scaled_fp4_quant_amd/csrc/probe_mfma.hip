// probe_mfma.hip -- the GPU's sustained dense f16 matrix-core rate and core clock, measured with a
// register-only MFMA loop.  A measurement aid for the roofline denominators (built into its own
// library, libfp4moe_probe.so, and called by the benchmark's peaks workload); not part of the method.
//
// Each wavefront issues `iters` rounds of four independent v_mfma_f32_32x32x16_f16 (4 x 32,768
// flops) on register operands: no memory traffic inside the loop.  With toggle != 0 the operands'
// mantissa bits change every round (a new pattern each round), so the multipliers see changing
// data as in a real GEMM; with toggle == 0 they multiply the same operands every round.  Lane 0 of
// each workgroup records s_memtime (core clock cycles) and s_memrealtime (a fixed 100 MHz counter)
// before and after its loop, so clocks[4 b .. 4 b + 3] = {cycles start, cycles end, 100 MHz start,
// 100 MHz end} give workgroup b's average core clock under this load.
//
// C ABI (plain pointers; sink and clocks are device memory owned by the caller):
//   int fp4moe_probe_mfma_loop(int32_t iters, int32_t toggle, int32_t nblocks, float* sink,
//                              uint64_t* clocks, hipStream_t stream);
//   sink: f32 [nblocks * 256] (one value per thread keeps the accumulators live); clocks: u64
//   [nblocks * 4].  Returns 0, 1 for invalid arguments (iters or nblocks <= 0, a null pointer),
//   2 for a launch error.  Enqueues one kernel of nblocks workgroups of 256 threads on `stream`.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t xorshift(uint32_t& x) {
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  return x;
}

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, int toggle, float* sink, uint64_t* clocks) {
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  // f16 operands in [0.5, 1) with random signs and mantissas: finite, and the sums stay far from
  // overflow over any loop length used here
  uint32_t x = gid * 2654435761u + 12345u;
  u32x4 ua, ub;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ua[i] = 0x38003800u | (xorshift(x) & 0x83FF83FFu);
    ub[i] = 0x38003800u | (xorshift(x) & 0x83FF83FFu);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  uint64_t t0 = 0, r0 = 0;
  if (threadIdx.x == 0) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  uint32_t m = toggle ? (x & 0x03FF03FFu) : 0u;
  for (int it = 0; it < iters; ++it) {
    const h16x8 a = __builtin_bit_cast(h16x8, ua), b = __builtin_bit_cast(h16x8, ub);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, b, c3, 0, 0, 0);
    // mantissa bits only: the operands stay in [0.5, 1) up to sign
    ua ^= m;
    ub ^= (m >> 1) & 0x03FF03FFu;
    m = toggle ? (m * 1664525u + 1013904223u) & 0x03FF03FFu : 0u;
  }
  if (threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    uint64_t* c = clocks + (size_t)blockIdx.x * 4;
    c[0] = t0;
    c[1] = t1;
    c[2] = r0;
    c[3] = r1;
  }
  float s = 0.0f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
  sink[gid] = s;
}

}  // namespace

extern "C" __attribute__((visibility("default"))) int fp4moe_probe_mfma_loop(int32_t iters, int32_t toggle,
                                                                            int32_t nblocks, float* sink,
                                                                            uint64_t* clocks, hipStream_t stream) {
  if (iters <= 0 || nblocks <= 0 || !sink || !clocks) return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)nblocks), dim3(256), 0, stream, iters, toggle, sink, clocks);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
