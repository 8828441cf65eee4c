// swiglu_quant.hip -- the expert activation between the gate/up and the down projection, fused with
// the FP8 activation quantization of its result (memra-engine 0.98.0 dsv4_native_gemm_gate.rs page:
// the swiglu_limit saturation cell's clamp math and its swiglu call, then `quant_rows` on h).
//
//   h[r, i] = silu(min(g, limit)) * clamp(u, -limit, limit) * w[r],  silu(t) = t / (1 + exp(-t))
//   g = gu[r, i], u = gu[r, inter + i]   (gu: the fused gate/up GEMM output, gate columns first)
//
// followed by the same per-128-column E4M3 quantization as act_quant_fp8, so that the codes and
// scales feed the down-projection GEMM directly.  h itself is written only when asked for.
//
// Layout and work split follow act_quant.hip: h is a flat sequence of 128-wide groups; a half
// wavefront owns one group, each lane four consecutive elements (one 16-byte load of gate values
// and one of up values); blocks of 8 half waves take 32 groups per iteration.  HBM-bound: 8 bytes
// read and 1 + 4/128 bytes written per element (+ 4 with h).
//
// Arithmetic is f32 in the page's order: min/clamp, expf, one correctly rounded division, then
// gate * sigmoid * up * weight.
#include "device_common.h"
#include "kernels.h"

namespace fp4moe {

namespace {
constexpr int kSqThreads = 256;
constexpr int kSqUnroll = 4;                             // groups per half wave per iteration
constexpr int kSqGroupsPerBlock = (kSqThreads / 32) * kSqUnroll;

__global__ __launch_bounds__(kSqThreads) void swiglu_quant_kernel(const float* __restrict__ gu,
                                                                  const float* __restrict__ weights,
                                                                  float limit, uint8_t* __restrict__ codes,
                                                                  float* __restrict__ scales,
                                                                  float* __restrict__ h_out, int64_t ngroups,
                                                                  int32_t groups_per_row) {
  const int lane = threadIdx.x & 31;
  const int hw = threadIdx.x >> 5;
  const float inv448 = u2f(0x3B124925u);                 // 1/448 rounded once to f32
  const int64_t inter = (int64_t)groups_per_row * 128;
  for (int64_t base = (int64_t)blockIdx.x * kSqGroupsPerBlock; base < ngroups;
       base += (int64_t)gridDim.x * kSqGroupsPerBlock) {
    f32x4 g[kSqUnroll], u[kSqUnroll];
    float w[kSqUnroll];
#pragma unroll
    for (int j = 0; j < kSqUnroll; ++j) {
      const int64_t grp = base + j * (kSqThreads / 32) + hw;
      g[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      u[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      w[j] = 1.0f;
      if (grp < ngroups) {
        const int64_t r = grp / groups_per_row, q = grp - r * groups_per_row;
        const float* row = gu + r * 2 * inter + q * 128;
        g[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row) + lane);
        u[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + inter) + lane);
        if (weights) w[j] = weights[r];
      }
    }
#pragma unroll
    for (int j = 0; j < kSqUnroll; ++j) {
      const int64_t grp = base + j * (kSqThreads / 32) + hw;
      f32x4 h;
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = swiglu_one(g[j][e], u[j][e], limit, w[j]);
      float m = fmaxf(fmaxf(fabsf(h[0]), fabsf(h[1])), fmaxf(fabsf(h[2]), fabsf(h[3])));
      m = halfwave_max(m);
      m = fmaxf(m, 1e-4f);
      const float s = pow2_ceil_pos(m * inv448);
      const float rcp = pow2_recip(s);                 // h * rcp == h / s exactly (s = 2^e)
      const float a0 = fminf(fmaxf(h[0] * rcp, -448.f), 448.f);
      const float a1 = fminf(fmaxf(h[1] * rcp, -448.f), 448.f);
      const float a2 = fminf(fmaxf(h[2] * rcp, -448.f), 448.f);
      const float a3 = fminf(fmaxf(h[3] * rcp, -448.f), 448.f);
      int packed = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
      packed = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, packed, true);
      if (grp < ngroups) {
        reinterpret_cast<uint32_t*>(codes + grp * 128)[lane] = (uint32_t)packed;
        if (lane == 0) scales[grp] = s;
        if (h_out) reinterpret_cast<f32x4*>(h_out + grp * 128)[lane] = h;
      }
    }
  }
}
}  // namespace

hipError_t launch_swiglu_quant(const float* gu, const float* weights, float limit, uint8_t* codes,
                               float* scales, float* h_out, int64_t rows, int32_t inter,
                               hipStream_t stream) {
  const int32_t gpr = inter / 128;
  const int64_t ngroups = rows * gpr;
  const int64_t want = (ngroups + kSqGroupsPerBlock - 1) / kSqGroupsPerBlock;
  const int blocks = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(swiglu_quant_kernel, dim3(blocks), dim3(kSqThreads), 0, stream, gu, weights, limit,
                     codes, scales, h_out, ngroups, gpr);
  return hipGetLastError();
}

}  // namespace fp4moe
