// swizzle.hip -- load-time reordering of one expert's FP4 planes into the order the GEMM kernels'
// matrix-core lanes consume them (the values are the memra-engine 0.98.0 dsv4_native_gemm_gate.rs
// page's `ExpertRaw` planes, unchanged).
//
// In the plain layout a lane of the 16x16x32 MFMA operand holds 32 k of one column, so a 64-lane
// weight load touches 16 column rows (16 half cache lines, k/2 bytes apart).  The swizzled layout
// stores, for each group of 16 columns and each 128-wide k block, the 64 lane pieces of 16 bytes in
// lane order: [column group t][block b][k piece p][column j][16 bytes].  One 64-lane load then reads
// 1 KB of consecutive bytes.  The scale planes are grouped per 4 blocks the same way,
// [t][4-block chunk q][p][j][the piece's scale bytes of blocks 4q..4q+3], so a lane reads the scales
// of its pieces for 4 blocks with one 8-byte (NVFP4) or 4-byte (MXFP4) load.
#include "kernels.h"

namespace fp4moe {
namespace {

constexpr int kThreads = 256;

// One thread per 16-byte lane piece of the nibble plane.
__global__ void swizzle_w_kernel(const uint8_t* __restrict__ w, uint8_t* __restrict__ out, int32_t n, int32_t k,
                                 int64_t pieces) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= pieces) return;
  const int nblk = k >> 7;
  const int j = (int)(i & 15), p = (int)((i >> 4) & 3);
  const int64_t tb = i >> 6;                         // t * nblk + b
  const int b = (int)(tb % nblk);
  const int64_t c = (tb / nblk) * 16 + j;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (c < n) v = *reinterpret_cast<const uint4*>(w + c * (int64_t)(k / 2) + 64 * b + 16 * p);
  *reinterpret_cast<uint4*>(out + i * 16) = v;
}

// One thread per lane piece of a 4-block chunk of the scale plane: 8 bytes (NVFP4: 2 scales per
// block) or 4 bytes (MXFP4: 1 scale per block).
__global__ void swizzle_s_kernel(const uint8_t* __restrict__ s, uint8_t* __restrict__ out, int32_t kind,
                                 int32_t n, int32_t k, int64_t pieces) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= pieces) return;
  const int nblk = k >> 7, nq = (nblk + 3) >> 2;
  const int j = (int)(i & 15), p = (int)((i >> 4) & 3);
  const int64_t tq = i >> 6;                         // t * nq + q
  const int q = (int)(tq % nq);
  const int64_t c = (tq / nq) * 16 + j;
  if (kind == 0) {
    const int64_t row = c * (int64_t)(k / 16);
    uint32_t lo = 0u, hi = 0u;
    for (int m = 0; m < 4; ++m) {
      const int b = 4 * q + m;
      uint32_t pair = 0u;
      if (c < n && b < nblk) pair = (uint32_t)s[row + 8 * b + 2 * p] | ((uint32_t)s[row + 8 * b + 2 * p + 1] << 8);
      if (m < 2) lo |= pair << (16 * m);
      else hi |= pair << (16 * (m - 2));
    }
    *reinterpret_cast<uint2*>(out + i * 8) = make_uint2(lo, hi);
  } else {
    const int64_t row = c * (int64_t)(k / 32);
    uint32_t v = 0u;
    for (int m = 0; m < 4; ++m) {
      const int b = 4 * q + m;
      if (c < n && b < nblk) v |= (uint32_t)s[row + 4 * b + p] << (8 * m);
    }
    *reinterpret_cast<uint32_t*>(out + i * 4) = v;
  }
}

}  // namespace

int64_t swizzled_weight_bytes(int32_t n, int32_t k) {
  return (int64_t)((n + 15) / 16) * 16 * (k / 2);
}

int64_t swizzled_scale_bytes(int32_t kind, int32_t n, int32_t k) {
  const int64_t nq = ((k / 128) + 3) / 4;
  return (int64_t)((n + 15) / 16) * nq * 64 * (kind == 0 ? 8 : 4);
}

hipError_t launch_weight_swizzle(const uint8_t* w, const uint8_t* s, int32_t kind, int32_t n, int32_t k,
                                 uint8_t* w_out, uint8_t* s_out, hipStream_t stream) {
  const int64_t wp = swizzled_weight_bytes(n, k) / 16;
  const int64_t sp = swizzled_scale_bytes(kind, n, k) / (kind == 0 ? 8 : 4);
  hipLaunchKernelGGL(swizzle_w_kernel, dim3((unsigned)((wp + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                     w, w_out, n, k, wp);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(swizzle_s_kernel, dim3((unsigned)((sp + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                     s, s_out, kind, n, k, sp);
  return hipGetLastError();
}

}  // namespace fp4moe
