// w4a4.hip -- the W4A4 NVFP4 variant: E2M1 activations with a two-level scale, the loudest-channel
// side path, and the FP4 x FP4 GEMM (memra-engine 0.71.0 kernel_check.rs page, the NVFP4 MMQ W4A4
// arms: a per-token row scale from the row amax, a UE4M3 micro-scale of amax_sub / 6 per 16-element
// sub-block, E2M1 codes; the sub-block-only quantizer it replaced; the k loudest channels kept out of
// the E2M1 path and added back exactly).  Lossy by design: E2M1 has 8 magnitudes.
//
// Quantizer, per row (f32, each step one IEEE operation):
//   rs = amax_row / 2688 (6 x 448, so the loudest sub-block gets micro-scale 448), 1 without the row
//   level or for an all-zero row;  micro = E4M3(clamp((amax_sub / rs) / 6, 2^-9, 448)) rounded to
//   nearest even, 0 for an all-zero sub-block;  code = E2M1((x / rs) / micro), nearest grid point,
//   ties to the even code, magnitude capped at 6, 0 when micro is 0.  Kept-out channels count as 0.
// GEMM: out[r, c] = rs[r] * scale2 * sum_k (E2M1(a) * micro) * (E2M1(w) * E4M3(ws)) + sum over kept
//   channels j of x[r, j] * (E2M1(w[c, j]) * f32(E4M3(ws) * scale2)).  The first term runs on the
//   tiled matrix-core kernel of the FP8 path (gemm_prefill.hip) with W4A4 activation staging: both
//   products E2M1 x E4M3 have at most 5 significant bits, so its f16 operands are exact, and the row
//   and tensor scales multiply the f32 sum (exact for power-of-two scale2).  The kept channels are
//   added by w4a4_residual_kernel.
//
// Layouts: codes u8 [rows, k/2] (even k in the low nibble), micro u8 [rows, k/16], rs f32 [rows].
// The quantizer takes one block per row with the row in registers (k <= 8192; one wavefront per row
// and two passes above that); the channel selection one block.
#include "device_common.h"
#include "kernels.h"

namespace fp4moe {
namespace {

constexpr int kW4Threads = 256;
constexpr int kMaxSkip = 64;

// E2M1 code of a finite f32: the comparisons against the midpoints of the grid
// {0, .5, 1, 1.5, 2, 3, 4, 6}, each tie going to the even code.
__device__ __forceinline__ uint32_t e2m1_encode(float q) {
  const float a = fabsf(q);
  const uint32_t m = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
  return m | ((f2u(q) >> 28) & 8u);
}

__device__ __forceinline__ float e2m1_value(uint32_t code) {
  const uint32_t ef = (code >> 1) & 3u, m = code & 1u;
  const float mag = ef == 0 ? 0.5f * (float)m : (1.0f + 0.5f * (float)m) * (float)(1u << (ef - 1));
  return (code & 8u) ? -mag : mag;
}

__device__ __forceinline__ float e4m3_value(uint32_t byte) { return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0); }

__device__ __forceinline__ uint32_t e4m3_encode_pos(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0x7Fu;
}

// Maximum over each aligned group of 4 lanes.
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  return fmaxf(v, dpp_f32<kDppQuadXor2>(v));
}

__device__ __forceinline__ float wave_max(float v) {
  v = halfwave_max(v);
  return fmaxf(u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(v), 0)),
               u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(v), 32)));
}

// One wavefront per row; 256 elements per step (4 per lane, a 16-element sub-block per 4 lanes).
__global__ __launch_bounds__(kW4Threads) void act_quant_fp4_kernel(const float* __restrict__ x,
                                                                   const int32_t* __restrict__ skip, int32_t n_skip,
                                                                   int32_t rows, int32_t k, int32_t two_level,
                                                                   uint8_t* __restrict__ codes,
                                                                   uint8_t* __restrict__ micro,
                                                                   float* __restrict__ row_scale) {
  __shared__ int32_t s_skip[kMaxSkip];
  for (int i = threadIdx.x; i < n_skip; i += kW4Threads) s_skip[i] = skip[i];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (kW4Threads / 64) + (threadIdx.x >> 6);
  if (r >= rows) return;                             // uniform per wavefront
  const float* xr = x + r * k;
  auto load4 = [&](int c0) {
    f32x4 v = *reinterpret_cast<const f32x4*>(xr + c0);
    for (int i = 0; i < n_skip; ++i) {
      const int d = s_skip[i] - c0;
      if (d >= 0 && d < 4) v[d] = 0.0f;
    }
    return v;
  };
  float amax = 0.0f;
  for (int c0 = 4 * lane; c0 < k; c0 += 256) {
    const f32x4 v = load4(c0);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  }
  amax = wave_max(amax);
  const float rs = (two_level && amax > 0.0f) ? amax / 2688.0f : 1.0f;
  if (lane == 0) row_scale[r] = rs;
  for (int c0 = 4 * lane; c0 < k; c0 += 256) {
    const f32x4 v = load4(c0);
    const float asub = quad_max(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    const float want = (asub / rs) / 6.0f;
    const uint32_t mb = want > 0.0f ? e4m3_encode_pos(fminf(fmaxf(want, 0x1p-9f), 448.0f)) : 0u;
    const float dec = e4m3_value(mb);
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t c = dec > 0.0f ? e2m1_encode((v[e] / rs) / dec) : 0u;
      packed |= c << (4 * e);
    }
    reinterpret_cast<uint16_t*>(codes + r * (k / 2))[c0 / 4] = (uint16_t)packed;
    if ((lane & 3) == 0) micro[r * (k / 16) + c0 / 16] = (uint8_t)mb;
  }
}

// One block per row with the row held in registers (k <= 8192): thread t owns the 16-byte pieces
// t + 256 j of the row, so every quad of threads owns one 16-element sub-block.  One read of x.
constexpr int kRowPieces = 8;                        // 16-byte pieces per thread: k <= 256 x 8 x 4

template <int NP>
__global__ __launch_bounds__(kW4Threads) void act_quant_fp4_row_kernel(const float* __restrict__ x,
                                                                       const int32_t* __restrict__ skip,
                                                                       int32_t n_skip, int32_t rows, int32_t k,
                                                                       int32_t two_level, uint8_t* __restrict__ codes,
                                                                       uint8_t* __restrict__ micro,
                                                                       float* __restrict__ row_scale) {
  __shared__ int32_t s_skip[kMaxSkip];
  __shared__ float s_max[kW4Threads / 64];
  for (int i = threadIdx.x; i < n_skip; i += kW4Threads) s_skip[i] = skip[i];
  __syncthreads();
  const int64_t r = blockIdx.x;
  const float* xr = x + r * k;
  const int npieces = k / 4;
  f32x4 v[NP];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int piece = threadIdx.x + kW4Threads * j;
    v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (piece < npieces) {
      v[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(xr) + piece);
      for (int i = 0; i < n_skip; ++i) {
        const int d = s_skip[i] - 4 * piece;
        if (d >= 0 && d < 4) v[j][d] = 0.0f;
      }
    }
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3]))));
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float rs = (two_level && amax > 0.0f) ? amax / 2688.0f : 1.0f;
  if (threadIdx.x == 0) row_scale[r] = rs;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int piece = threadIdx.x + kW4Threads * j;
    // uniform per quad: a sub-block is 4 pieces and npieces is a multiple of 4
    const float asub = quad_max(fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3]))));
    if (piece >= npieces) continue;
    const float want = (asub / rs) / 6.0f;
    const uint32_t mb = want > 0.0f ? e4m3_encode_pos(fminf(fmaxf(want, 0x1p-9f), 448.0f)) : 0u;
    const float dec = e4m3_value(mb);
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t c = dec > 0.0f ? e2m1_encode((v[j][e] / rs) / dec) : 0u;
      packed |= c << (4 * e);
    }
    reinterpret_cast<uint16_t*>(codes + r * (k / 2))[piece] = (uint16_t)packed;
    if ((threadIdx.x & 3) == 0) micro[r * (k / 16) + piece / 4] = (uint8_t)mb;
  }
}

// One block: the k_res channels with the largest max |x| over rows, ties to the lower index.  Each
// thread keeps the keys of channels tid + 1024 i (i < 8): high word the order-preserving bits of the
// (non-negative) column max, low word ~channel.
constexpr int kLoudThreads = 1024;
constexpr int kLoudPer = 8;

__global__ __launch_bounds__(kLoudThreads) void loud_channels_kernel(const float* __restrict__ x, int32_t rows,
                                                                     int32_t k, int32_t k_res,
                                                                     int32_t* __restrict__ idx) {
  __shared__ uint64_t s_best[kLoudThreads / 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint64_t key[kLoudPer];
#pragma unroll
  for (int i = 0; i < kLoudPer; ++i) {
    const int c = threadIdx.x + kLoudThreads * i;
    float m = 0.0f;
    if (c < k)
      for (int32_t r = 0; r < rows; ++r) m = fmaxf(m, fabsf(x[(int64_t)r * k + c]));
    key[i] = c < k ? (((uint64_t)f2u(m) << 32) | (uint32_t)~c) : 0ull;
  }
  for (int j = 0; j < k_res; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < kLoudPer; ++i) best = best > key[i] ? best : key[i];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint64_t o = __shfl_xor(best, d, 64);
      best = best > o ? best : o;
    }
    if (lane == 0) s_best[wv] = best;
    __syncthreads();
    best = s_best[0];
    for (int w = 1; w < kLoudThreads / 64; ++w) best = best > s_best[w] ? best : s_best[w];
    __syncthreads();
    const int c = (int)~(uint32_t)best;
#pragma unroll
    for (int i = 0; i < kLoudPer; ++i)
      if (c == (int)threadIdx.x + kLoudThreads * i) key[i] = 0ull;
    if (threadIdx.x == 0) idx[j] = c;
  }
}

// The kept channels, added to the W4A4 GEMM's output: out[r, c] += sum_j x[r, j] * W(c, j) over the
// channel list, W = E2M1 x f32(E4M3(ws) x scale2), one f32 FMA per term in list order.  One thread
// per output; channel indices outside [0, k) add nothing.
__global__ __launch_bounds__(kW4Threads) void w4a4_residual_kernel(const float* __restrict__ x,
                                                                   const int32_t* __restrict__ res_idx,
                                                                   int32_t k_res, const uint8_t* __restrict__ w,
                                                                   const uint8_t* __restrict__ s, float scale2,
                                                                   float* __restrict__ out, int32_t g, int32_t n,
                                                                   int32_t k) {
  const int64_t i = (int64_t)blockIdx.x * kW4Threads + threadIdx.x;
  if (i >= (int64_t)g * n) return;
  const int64_t r = i / n, col = i - r * n;
  float o = out[i];
  for (int j = 0; j < k_res; ++j) {
    const int32_t c = res_idx[j];
    if (c < 0 || c >= k) continue;
    const uint32_t byte = w[col * (k / 2) + c / 2];
    const float wv = e2m1_value((c & 1) ? (byte >> 4) : (byte & 0xFu)) *
                     (e4m3_value(s[col * (k / 16) + c / 16]) * scale2);
    o = fmaf(x[r * k + c], wv, o);
  }
  out[i] = o;
}

}  // namespace

hipError_t launch_act_quant_fp4(const float* x, const int32_t* skip, int32_t n_skip, int32_t rows, int32_t k,
                                int32_t two_level, uint8_t* codes, uint8_t* micro, float* row_scale,
                                hipStream_t stream) {
  const int per_thread = (k / 4 + kW4Threads - 1) / kW4Threads;
  if (per_thread <= kRowPieces) {
#define FP4MOE_AQ4(NP)                                                                                        \
  hipLaunchKernelGGL(act_quant_fp4_row_kernel<NP>, dim3(rows), dim3(kW4Threads), 0, stream, x, skip, n_skip, rows, \
                     k, two_level, codes, micro, row_scale)
    if (per_thread <= 1) FP4MOE_AQ4(1);
    else if (per_thread <= 2) FP4MOE_AQ4(2);
    else if (per_thread <= 4) FP4MOE_AQ4(4);
    else FP4MOE_AQ4(8);
#undef FP4MOE_AQ4
    return hipGetLastError();
  }
  const int blocks = (rows + kW4Threads / 64 - 1) / (kW4Threads / 64);
  hipLaunchKernelGGL(act_quant_fp4_kernel, dim3(blocks), dim3(kW4Threads), 0, stream, x, skip, n_skip, rows, k,
                     two_level, codes, micro, row_scale);
  return hipGetLastError();
}

hipError_t launch_loud_channels(const float* x, int32_t rows, int32_t k, int32_t k_res, int32_t* idx,
                                hipStream_t stream) {
  hipLaunchKernelGGL(loud_channels_kernel, dim3(1), dim3(kLoudThreads), 0, stream, x, rows, k, k_res, idx);
  return hipGetLastError();
}

hipError_t launch_w4a4_residual(const float* x, const int32_t* res_idx, int32_t k_res, const uint8_t* w,
                                const uint8_t* s, float scale2, float* out, int32_t g, int32_t n, int32_t k,
                                hipStream_t stream) {
  const int64_t items = (int64_t)g * n;
  hipLaunchKernelGGL(w4a4_residual_kernel, dim3((uint32_t)((items + kW4Threads - 1) / kW4Threads)), dim3(kW4Threads),
                     0, stream, x, res_idx, k_res, w, s, scale2, out, g, n, k);
  return hipGetLastError();
}

}  // namespace fp4moe
