// route.hip -- the routing steps around the grouped expert GEMM: top-k selection over router logits
// with softmax weights, the packing of the routed (token, slot) pairs per expert (CSR offsets, the
// token of each packed row and the packed row of each pair), the gather of quantized rows, and the
// weighted combine of the expert outputs back to token order.
//
// Sources: memra-engine 0.125.0 qwen4exp_gpu_gate.rs page, the device-router arm (softmax top-k over
// the router logits; selected ids and their order exact; ties of duplicates across the cut, all-equal
// rows and underflowing probabilities); memra-engine 0.71.0 kernel_check.rs page, f16g grouped GEMM
// section (routed rows packed per expert behind CSR offsets).
//
// Ranking: a larger logit ranks first; equal logits (+0 equal to -0) rank by the lower expert id; NaN
// ranks below every number.  Each logit becomes a 64-bit key whose unsigned order is that ranking:
// the high word is the float's bits mapped to an order-preserving unsigned integer (NaN -> 1, so it
// sits below -inf), the low word is ~id, so that the lower id wins among equal values.  A key of 0
// marks an expert already taken or past the end.
//
// All of this is tiny next to the GEMM (the prefill router reads 8 MB of logits); the kernels aim at
// few launches and no atomics on global memory, so that every result is deterministic.
#include "device_common.h"
#include "kernels.h"

namespace fp4moe {

namespace {

// ------------------------------------------------------------------------------ wave reductions
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t swz16_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, kSwizzleXor16);
}
__device__ __forceinline__ uint64_t join64(uint32_t lo, uint32_t hi) { return ((uint64_t)hi << 32) | lo; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return join64(dpp_u32<CTRL>((uint32_t)v), dpp_u32<CTRL>((uint32_t)(v >> 32)));
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Largest key over the wavefront; the result is wave-uniform.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, dpp_u64<kDppQuadXor1>(v));
  v = umax64(v, dpp_u64<kDppQuadXor2>(v));
  v = umax64(v, dpp_u64<kDppRowHalfMirror>(v));
  v = umax64(v, dpp_u64<kDppRowMirror>(v));
  v = umax64(v, join64(swz16_u32((uint32_t)v), swz16_u32((uint32_t)(v >> 32))));
  const uint64_t a = join64((uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 0),
                            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 0));
  const uint64_t b = join64((uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 32),
                            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 32));
  return umax64(a, b);
}

// Sum over the wavefront (a fixed tree: quads, 8, 16, 32 lanes, then the two halves); uniform.
__device__ __forceinline__ float wave_sum(float v) {
  v += u2f(dpp_u32<kDppQuadXor1>(f2u(v)));
  v += u2f(dpp_u32<kDppQuadXor2>(f2u(v)));
  v += u2f(dpp_u32<kDppRowHalfMirror>(f2u(v)));
  v += u2f(dpp_u32<kDppRowMirror>(f2u(v)));
  v += u2f(swz16_u32(f2u(v)));
  return u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(v), 0)) +
         u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(v), 32));
}

// ------------------------------------------------------------------------------------ ranking keys
__device__ __forceinline__ uint32_t order_key(float x) {
  if (__builtin_isnan(x)) return 1u;
  uint32_t b = f2u(x);
  if (b == 0x80000000u) b = 0u;                       // -0 ranks as +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t key) {
  return u2f((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// -------------------------------------------------------------------------------------- top-k
constexpr int kTopkThreads = 256;                     // four tokens per block, one per wavefront

template <int EPL>
__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(const float* __restrict__ logits,
                                                                  int32_t tokens, int32_t experts,
                                                                  int32_t top_k, int32_t normalize,
                                                                  int32_t* __restrict__ ids,
                                                                  float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (kTopkThreads / 64) + (threadIdx.x >> 6);
  if (t >= tokens) return;                            // uniform per wavefront
  const float* l = logits + t * experts;
  uint64_t key[EPL];
  float v[EPL];
  bool nan_here = false;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    v[i] = 0.0f;
    key[i] = 0;
    if (e < experts) {
      v[i] = __builtin_nontemporal_load(l + e);
      nan_here |= __builtin_isnan(v[i]);
      key[i] = join64(~(uint32_t)e, order_key(v[i]));
    }
  }
  float m = 0.0f, sel_sum = 0.0f, my_x = 0.0f;
  int my_id = 0;
  for (int j = 0; j < top_k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = umax64(best, key[i]);
    best = wave_max_u64(best);
    const int e = (int)~(uint32_t)best;
    const float x = key_value((uint32_t)(best >> 32));
    if (j == 0) m = x;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (e == lane + 64 * i) key[i] = 0;
    if (normalize) sel_sum += expf(x - m);
    if (lane == j) {
      my_id = e;
      my_x = x;
    }
  }
  float denom = sel_sum;
  if (!normalize) {
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + 64 * i < experts) part += expf(v[i] - m);
    denom = wave_sum(part);
  }
  if (__builtin_amdgcn_ballot_w64(nan_here)) denom = __builtin_nanf("");
  if (lane < top_k) {
    ids[t * top_k + lane] = my_id;
    weights[t * top_k + lane] = expf(my_x - m) / denom;
  }
}

// ------------------------------------------------------------------------------------- packing
// Pairs are numbered p = t * top_k + j.  Tokens are cut into slices of 64 (one token per lane);
// counts[e * nslices + s] is the number of pairs of slice s routed to expert e.  An exclusive scan
// of that expert-major array gives, for each (expert, slice), the first packed row of its pairs;
// inside a slice the pairs of one expert are ranked by lane (token) and then by j.
constexpr int kPackThreads = 256;
constexpr int kPackExpertsPerBlock = 64;               // place kernel: experts per block (16 per wave)
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kPackThreads) void route_count_kernel(const int32_t* __restrict__ ids,
                                                                   int32_t tokens, int32_t top_k,
                                                                   int32_t experts,
                                                                   int32_t* __restrict__ counts,
                                                                   int32_t nslices) {
  extern __shared__ int32_t hist[];
  const int s = blockIdx.x;
  for (int e = threadIdx.x; e < experts; e += kPackThreads) hist[e] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)s * 64 * top_k;
  const int64_t p1 = min((int64_t)(s + 1) * 64, (int64_t)tokens) * top_k;
  for (int64_t p = p0 + threadIdx.x; p < p1; p += kPackThreads) {
    const int32_t e = ids[p];
    if (e >= 0 && e < experts) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < experts; e += kPackThreads) counts[(int64_t)e * nslices + s] = hist[e];
}

// One block: exclusive scan of counts in place, offsets[e] = first row of expert e, offsets[E] = the
// number of packed rows.
__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(int32_t* __restrict__ counts, int64_t n,
                                                                  int32_t nslices, int32_t experts,
                                                                  int32_t* __restrict__ offsets) {
  __shared__ int32_t wave_tot[kScanThreads / 64];
  const int tid = threadIdx.x;
  if (n == 0) {
    for (int e = tid; e <= experts; e += kScanThreads) offsets[e] = 0;
    return;
  }
  const int64_t per = (n + kScanThreads - 1) / kScanThreads;
  const int64_t beg = min(n, tid * per), end = min(n, beg + per);
  int32_t local = 0;
  for (int64_t i = beg; i < end; ++i) local += counts[i];
  // inclusive scan inside the wavefront, then across the 16 wavefront totals
  const int lane = tid & 63, wv = tid >> 6;
  int32_t incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t o = __shfl_up(incl, d, 64);
    if (lane >= d) incl += o;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wv; ++w) before += wave_tot[w];
  int32_t run = before + incl - local;
  if (tid == kScanThreads - 1) offsets[experts] = run + local;
  for (int64_t i = beg; i < end; ++i) {
    const int32_t c = counts[i];
    counts[i] = run;
    if (i % nslices == 0) offsets[i / nslices] = run;
    run += c;
  }
}

template <int KMAX>
__global__ __launch_bounds__(kPackThreads) void route_place_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int32_t tokens, int32_t top_k,
    int32_t experts, const int32_t* __restrict__ first_row, int32_t nslices, int32_t* __restrict__ row_ids,
    int32_t* __restrict__ pair_rows, float* __restrict__ row_w) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int s = blockIdx.x;
  const int64_t t = (int64_t)s * 64 + lane;
  const bool live = t < tokens;
  int32_t id[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) id[j] = (live && j < top_k) ? ids[t * top_k + j] : -1;
  if (blockIdx.y == 0 && wv == 0 && live) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < top_k && (id[j] < 0 || id[j] >= experts)) pair_rows[t * top_k + j] = -1;
  }
  const int e_end = min(experts, (int)(blockIdx.y + 1) * kPackExpertsPerBlock);
  for (int e = blockIdx.y * kPackExpertsPerBlock + wv; e < e_end; e += kPackThreads / 64) {
    uint64_t any = 0;
    uint32_t below = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(id[j] == e);
      any |= m;
      below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, below));
    }
    if (any == 0) continue;                          // uniform
    int32_t pos = first_row[(int64_t)e * nslices + s] + (int32_t)below;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (id[j] == e) {
        const int64_t p = t * top_k + j;
        row_ids[pos] = (int32_t)t;
        pair_rows[p] = pos;
        if (row_w) row_w[pos] = w[p];
        ++pos;
      }
    }
  }
}

// --------------------------------------------------------------------------------------- gather
constexpr int kGatherThreads = 256;

__global__ __launch_bounds__(kGatherThreads) void gather_rows_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scales, int32_t a_rows, int32_t k,
    const int32_t* __restrict__ row_ids, int32_t rows, uint8_t* __restrict__ out_codes,
    float* __restrict__ out_scales) {
  const int32_t per_row = k / 16 + k / 128;            // 16-byte code chunks, then scales
  const int64_t total = (int64_t)rows * per_row;
  for (int64_t i = (int64_t)blockIdx.x * kGatherThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kGatherThreads) {
    const int64_t p = i / per_row;
    const int32_t c = (int32_t)(i - p * per_row);
    const int32_t r = row_ids[p];
    const bool ok = r >= 0 && r < a_rows;
    if (c < k / 16) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (ok) v = reinterpret_cast<const u32x4*>(codes + (int64_t)r * k)[c];
      reinterpret_cast<u32x4*>(out_codes + p * k)[c] = v;
    } else {
      const int32_t q = c - k / 16;
      out_scales[p * (k / 128) + q] = ok ? scales[(int64_t)r * (k / 128) + q] : __builtin_nanf("");
    }
  }
}

// -------------------------------------------------------------------------------------- combine
// out[t, c] = sum_j w[t, j] * y[pair_rows[t, j], c], the terms added in j order with one fused
// multiply-add each (a plain add without weights).  One block per (token, 1024 columns); the pair
// table of the token is wave-uniform.
constexpr int kCombineThreads = 256;
constexpr int kCombineCols = kCombineThreads * 4;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ y, int32_t y_rows, int32_t n, const int32_t* __restrict__ pair_rows,
    const float* __restrict__ w, int32_t top_k, int32_t nchunks, bool vec, float* __restrict__ out) {
  const int64_t t = blockIdx.x / nchunks;
  const int32_t chunk = (int32_t)(blockIdx.x - t * nchunks);
  const int32_t c = chunk * kCombineCols + threadIdx.x * 4;
  if (c >= n) return;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  bool bad = false;
  for (int j = 0; j < top_k; ++j) {
    const int32_t r = pair_rows[t * top_k + j];
    if (r < 0) continue;
    if (r >= y_rows) {
      bad = true;
      continue;
    }
    const float* yr = y + (int64_t)r * n + c;
    f32x4 yv;
    if (vec) {
      yv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yr));
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) yv[q] = (c + q < n) ? yr[q] : 0.0f;
    }
    if (w) {
      const float wj = w[t * top_k + j];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fmaf(wj, yv[q], acc[q]);
    } else {
      acc += yv;
    }
  }
  if (bad) acc = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
  float* o = out + t * n + c;
  if (vec) {
    *reinterpret_cast<f32x4*>(o) = acc;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (c + q < n) o[q] = acc[q];
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int32_t tokens, int32_t experts, int32_t top_k,
                             int32_t normalize, int32_t* ids, float* weights, hipStream_t stream) {
  const dim3 grid((tokens + kTopkThreads / 64 - 1) / (kTopkThreads / 64));
  const int epl = (experts + 63) / 64;
#define FP4MOE_TOPK(N)                                                                                  \
  hipLaunchKernelGGL(route_topk_kernel<N>, grid, dim3(kTopkThreads), 0, stream, logits, tokens, experts, \
                     top_k, normalize, ids, weights)
  if (epl <= 1) FP4MOE_TOPK(1);
  else if (epl <= 2) FP4MOE_TOPK(2);
  else if (epl <= 4) FP4MOE_TOPK(4);
  else if (epl <= 8) FP4MOE_TOPK(8);
  else FP4MOE_TOPK(16);
#undef FP4MOE_TOPK
  return hipGetLastError();
}

int64_t route_pack_workspace_elems(int32_t tokens, int32_t experts) {
  return (int64_t)experts * ((tokens + 63) / 64);
}

hipError_t launch_route_pack(const int32_t* ids, const float* w, int32_t tokens, int32_t top_k,
                             int32_t experts, int32_t* offsets, int32_t* row_ids, int32_t* pair_rows,
                             float* row_w, int32_t* workspace, hipStream_t stream) {
  const int32_t nslices = (tokens + 63) / 64;
  const int64_t n = (int64_t)experts * nslices;
  if (nslices > 0) {
    hipLaunchKernelGGL(route_count_kernel, dim3(nslices), dim3(kPackThreads), experts * sizeof(int32_t),
                       stream, ids, tokens, top_k, experts, workspace, nslices);
    if (hipError_t e = hipGetLastError()) return e;
  }
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, workspace, n, nslices,
                     experts, offsets);
  if (hipError_t e = hipGetLastError()) return e;
  if (nslices == 0) return hipSuccess;
  const dim3 grid(nslices, (experts + kPackExpertsPerBlock - 1) / kPackExpertsPerBlock);
#define FP4MOE_PLACE(N)                                                                             \
  hipLaunchKernelGGL(route_place_kernel<N>, grid, dim3(kPackThreads), 0, stream, ids, w, tokens,    \
                     top_k, experts, workspace, nslices, row_ids, pair_rows, row_w)
  if (top_k <= 8) FP4MOE_PLACE(8);
  else if (top_k <= 16) FP4MOE_PLACE(16);
  else if (top_k <= 32) FP4MOE_PLACE(32);
  else FP4MOE_PLACE(64);
#undef FP4MOE_PLACE
  return hipGetLastError();
}

hipError_t launch_gather_rows(const uint8_t* codes, const float* scales, int32_t a_rows, int32_t k,
                              const int32_t* row_ids, int32_t rows, uint8_t* out_codes, float* out_scales,
                              hipStream_t stream) {
  const int64_t total = (int64_t)rows * (k / 16 + k / 128);
  const int64_t want = (total + kGatherThreads - 1) / kGatherThreads;
  const int blocks = (int)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks), dim3(kGatherThreads), 0, stream, codes, scales,
                     a_rows, k, row_ids, rows, out_codes, out_scales);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y, int32_t y_rows, int32_t n, const int32_t* pair_rows,
                          const float* w, int32_t tokens, int32_t top_k, float* out, hipStream_t stream) {
  const int32_t nchunks = (n + kCombineCols - 1) / kCombineCols;
  // 16-byte row accesses when every row starts 16-byte aligned
  const bool vec = (n % 4) == 0 && ((reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
  hipLaunchKernelGGL(combine_kernel, dim3((uint32_t)((int64_t)tokens * nchunks)), dim3(kCombineThreads), 0,
                     stream, y, y_rows, n, pair_rows, w, top_k, nchunks, vec, out);
  return hipGetLastError();
}

}  // namespace fp4moe
