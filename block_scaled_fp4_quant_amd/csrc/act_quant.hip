// act_quant.hip -- FP8 E4M3 activation quantization, one power-of-two scale per row per 128
// columns (memra-engine 0.98.0 dsv4_native_gemm_gate.rs page, `quant_rows`).
//
// The [rows, k] input is a flat sequence of 128-float groups (k is a multiple of 128), and so are
// the code and scale outputs, so the kernel walks groups without caring about rows.  A half
// wavefront (32 lanes) owns one group: each lane loads one 16-byte float4, the group amax is a
// DPP/swizzle maximum over the 32 lanes, and each lane stores its four codes as one dword.  A block
// of 8 half waves handles 32 groups per iteration (four independent 16-byte loads per lane in
// flight, each load instruction covering 1 KB of contiguous input per wavefront); blocks stride
// over the group sequence.  HBM-bound: 4 bytes read and 1 + 4/128 bytes written per element.
#include "device_common.h"
#include "kernels.h"

namespace fp4moe {

namespace {
constexpr int kAqThreads = 256;
constexpr int kAqUnroll = 4;                             // groups per half wave per iteration
constexpr int kAqGroupsPerBlock = (kAqThreads / 32) * kAqUnroll;

__global__ __launch_bounds__(kAqThreads) void act_quant_kernel(const float* __restrict__ x,
                                                               uint8_t* __restrict__ codes,
                                                               float* __restrict__ scales,
                                                               int64_t ngroups) {
  const int lane = threadIdx.x & 31;
  const int hw = threadIdx.x >> 5;
  const float inv448 = u2f(0x3B124925u);                 // 1/448 rounded once to f32
  for (int64_t base = (int64_t)blockIdx.x * kAqGroupsPerBlock; base < ngroups;
       base += (int64_t)gridDim.x * kAqGroupsPerBlock) {
    f32x4 v[kAqUnroll];
#pragma unroll
    for (int u = 0; u < kAqUnroll; ++u) {
      const int64_t grp = base + u * (kAqThreads / 32) + hw;
      v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (grp < ngroups)
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + grp * 128) + lane);
    }
#pragma unroll
    for (int u = 0; u < kAqUnroll; ++u) {
      const int64_t grp = base + u * (kAqThreads / 32) + hw;
      float m = fmaxf(fmaxf(fabsf(v[u][0]), fabsf(v[u][1])), fmaxf(fabsf(v[u][2]), fabsf(v[u][3])));
      m = halfwave_max(m);
      m = fmaxf(m, 1e-4f);
      const float s = pow2_ceil_pos(m * inv448);
      const float r = pow2_recip(s);                   // x * r == x / s exactly (s = 2^e)
      const float a0 = fminf(fmaxf(v[u][0] * r, -448.f), 448.f);
      const float a1 = fminf(fmaxf(v[u][1] * r, -448.f), 448.f);
      const float a2 = fminf(fmaxf(v[u][2] * r, -448.f), 448.f);
      const float a3 = fminf(fmaxf(v[u][3] * r, -448.f), 448.f);
      int packed = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
      packed = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, packed, true);
      if (grp < ngroups) {
        reinterpret_cast<uint32_t*>(codes + grp * 128)[lane] = (uint32_t)packed;
        if (lane == 0) scales[grp] = s;
      }
    }
  }
}
}  // namespace

hipError_t launch_act_quant(const float* x, uint8_t* codes, float* scales, int64_t ngroups,
                            hipStream_t stream) {
  const int64_t want = (ngroups + kAqGroupsPerBlock - 1) / kAqGroupsPerBlock;
  const int blocks = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(act_quant_kernel, dim3(blocks), dim3(kAqThreads), 0, stream, x, codes, scales,
                     ngroups);
  return hipGetLastError();
}

}  // namespace fp4moe
