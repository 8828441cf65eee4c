// rung.hip -- the bf16-dequant rung: a reference route for the quantized expert GEMM on exact
// weights and unquantized activations (memra-engine 0.98.0 dsv4_native_gemm_gate.rs page,
// comparison 3: the f32 activations converted to bf16, the expert weights dequantized to bf16, a
// bf16 GEMM with f32 output).  The native path's difference from it is the numeric-class shift of
// quantizing the activations to E4M3.
//
//   cvt_bf16:          f32 -> bf16, round to nearest even; NaN stays NaN (sign and top payload bits
//                      kept, quiet bit set).
//   dequant_bf16:      w[c, k] = bf16(f32(E2M1(nibble) * ws[c, k / gs])), ws = f32(E4M3(S) * scale2)
//                      for NVFP4, 2^(S - 127) for MXFP4 -- the weight scale of the GEMM; a NaN
//                      scale gives the canonical bf16 NaN 0x7FC0.
//   gemm_bf16:         out[r, c] = sum_k a[r, k] * w[c, k], bf16 operands, f32 accumulation.
//
// None of this is on the hot path: the kernels are plain.  The GEMM gives each wavefront one 32 x 32
// output tile and feeds the 32x32x16 bf16 MFMA straight from global memory.
#include "device_common.h"
#include "kernels.h"

namespace fp4moe {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = f2u(x);
  if (__builtin_isnan(x)) return (u >> 16) | 0x0040u;
  const uint32_t lower = u & 0xFFFFu, upper = u >> 16;
  return (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) ? upper + 1u : upper;
}

constexpr int kRungThreads = 256;

__global__ __launch_bounds__(kRungThreads) void cvt_bf16_kernel(const float* __restrict__ x,
                                                                uint16_t* __restrict__ out, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * kRungThreads + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * kRungThreads)
    out[i] = (uint16_t)bf16_bits(x[i]);
}

// One thread: 8 consecutive weights of one column (4 nibble bytes) -> 16 bytes of bf16.
__global__ __launch_bounds__(kRungThreads) void dequant_bf16_kernel(const uint8_t* __restrict__ w,
                                                                    const uint8_t* __restrict__ s,
                                                                    float scale2, int32_t kind, int32_t n,
                                                                    int32_t k, uint16_t* __restrict__ out) {
  const int gs = kind == 0 ? 16 : 32;
  const int64_t per_col = k / 8;
  const int64_t total = (int64_t)n * per_col;
  for (int64_t i = (int64_t)blockIdx.x * kRungThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kRungThreads) {
    const int64_t c = i / per_col;
    const int32_t k0 = (int32_t)(i - c * per_col) * 8;
    const uint8_t sb = s[c * (k / gs) + k0 / gs];
    float ws;
    if (kind == 0) {
      ws = __builtin_amdgcn_cvt_f32_fp8((int)sb, 0) * scale2;
    } else {
      ws = sb == 255 ? __builtin_nanf("") : (sb == 0 ? u2f(0x00400000u) : u2f((uint32_t)sb << 23));
    }
    const uint32_t nib = *reinterpret_cast<const uint32_t*>(w + c * (k / 2) + k0 / 2);
    uint32_t packed[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t h[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t code = (nib >> (4 * (2 * q + e))) & 0xFu;
        // E2M1: exponent field bits 2..1, mantissa bit 0; 0.5 * m when the exponent field is 0
        const uint32_t ef = (code >> 1) & 3u, m = code & 1u;
        const float mag = ef == 0 ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * (float)(1u << (ef - 1));
        const float v = ((code & 8u) ? -mag : mag) * ws;
        h[e] = __builtin_isnan(v) ? 0x7FC0u : bf16_bits(v);
      }
      packed[q] = h[0] | (h[1] << 16);
    }
    *reinterpret_cast<u32x4*>(out + c * k + k0) = u32x4{packed[0], packed[1], packed[2], packed[3]};
  }
}

// out = a * w^T.  Wavefront (tm, tn) of the grid computes rows 32 tm .. +32 and columns 32 tn .. +32.
// 32x32x16 bf16 MFMA operand layout: lane l supplies row (column) l % 32 and k = 8 (l / 32) .. +8;
// the result holds column l % 32 and rows 8 (v / 4) + 4 (l / 32) + v % 4, v = 0 .. 15.
__global__ __launch_bounds__(kRungThreads) void gemm_bf16_kernel(const uint16_t* __restrict__ a,
                                                                 const uint16_t* __restrict__ w,
                                                                 float* __restrict__ out, int32_t m, int32_t n,
                                                                 int32_t k, int32_t tiles_n) {
  const int lane = threadIdx.x & 63;
  const int64_t tile = (int64_t)blockIdx.x * (kRungThreads / 64) + (threadIdx.x >> 6);
  const int32_t tm = (int32_t)(tile / tiles_n), tn = (int32_t)(tile % tiles_n);
  if ((int64_t)tm * 32 >= m) return;                 // uniform per wavefront
  const rsrc_t ra = make_rsrc(a, (uint32_t)m * (uint32_t)k * 2u);
  const rsrc_t rw = make_rsrc(w, (uint32_t)n * (uint32_t)k * 2u);
  const int row = tm * 32 + (lane & 31), col = tn * 32 + (lane & 31);
  const uint32_t oa = row < m ? ((uint32_t)row * (uint32_t)k + 8u * (lane >> 5)) * 2u : kOffNone;
  const uint32_t ow = col < n ? ((uint32_t)col * (uint32_t)k + 8u * (lane >> 5)) * 2u : kOffNone;
  f32x16 acc = {};
  for (int32_t k0 = 0; k0 < k; k0 += 16) {
    const uint32_t d = (uint32_t)k0 * 2u;
    const bf16x8 av = __builtin_bit_cast(bf16x8, buf_load_x4(ra, oa == kOffNone ? kOffNone : oa + d));
    const bf16x8 wv = __builtin_bit_cast(bf16x8, buf_load_x4(rw, ow == kOffNone ? kOffNone : ow + d));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, wv, acc, 0, 0, 0);
  }
  const int c = tn * 32 + (lane & 31);
  if (c >= n) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int r = tm * 32 + 8 * (v / 4) + 4 * (lane >> 5) + v % 4;
    if (r < m) out[(int64_t)r * n + c] = acc[v];
  }
}

int grid_for(int64_t items) {
  const int64_t want = (items + kRungThreads - 1) / kRungThreads;
  return (int)(want < 16384 ? (want > 0 ? want : 1) : 16384);
}

}  // namespace

hipError_t launch_cvt_bf16(const float* x, uint16_t* out, int64_t count, hipStream_t stream) {
  hipLaunchKernelGGL(cvt_bf16_kernel, dim3(grid_for(count)), dim3(kRungThreads), 0, stream, x, out, count);
  return hipGetLastError();
}

hipError_t launch_dequant_bf16(const uint8_t* w, const uint8_t* s, float scale2, int32_t kind, int32_t n,
                               int32_t k, uint16_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(dequant_bf16_kernel, dim3(grid_for((int64_t)n * (k / 8))), dim3(kRungThreads), 0, stream, w,
                     s, scale2, kind, n, k, out);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const uint16_t* a, const uint16_t* w, float* out, int32_t m, int32_t n, int32_t k,
                            hipStream_t stream) {
  const int32_t tiles_n = (n + 31) / 32;
  const int64_t tiles = (int64_t)((m + 31) / 32) * tiles_n;
  const int64_t blocks = (tiles + kRungThreads / 64 - 1) / (kRungThreads / 64);
  hipLaunchKernelGGL(gemm_bf16_kernel, dim3((uint32_t)blocks), dim3(kRungThreads), 0, stream, a, w, out, m, n, k,
                     tiles_n);
  return hipGetLastError();
}

}  // namespace fp4moe
