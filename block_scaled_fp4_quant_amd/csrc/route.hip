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

// Largest key over each group of LPT lanes (LPT = 16: a DPP row; 64: the wavefront); every lane
// of the group receives it (wave-uniform for LPT = 64).
template <int LPT>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  v = umax64(v, dpp_u64<kDppQuadXor1>(v));
  v = umax64(v, dpp_u64<kDppQuadXor2>(v));
  v = umax64(v, dpp_u64<kDppRowHalfMirror>(v));
  v = umax64(v, dpp_u64<kDppRowMirror>(v));
  if constexpr (LPT == 64) {
    v = umax64(v, join64(swz16_u32((uint32_t)v), swz16_u32((uint32_t)(v >> 32))));
    const uint64_t a = join64((uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 0),
                              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 0));
    const uint64_t b = join64((uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 32),
                              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 32));
    v = umax64(a, b);
  }
  return v;
}

// Sum over each group of LPT lanes (a fixed tree: quads, 8, 16 lanes, then for LPT = 64 the 32-lane
// halves and the two halves); every lane of the group receives it.
template <int LPT>
__device__ __forceinline__ float group_sum(float v) {
  v += u2f(dpp_u32<kDppQuadXor1>(f2u(v)));
  v += u2f(dpp_u32<kDppQuadXor2>(f2u(v)));
  v += u2f(dpp_u32<kDppRowHalfMirror>(f2u(v)));
  v += u2f(dpp_u32<kDppRowMirror>(f2u(v)));
  if constexpr (LPT == 64) {
    v += u2f(swz16_u32(f2u(v)));
    v = u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(v), 0)) +
        u2f((uint32_t)__builtin_amdgcn_readlane((int)f2u(v), 32));
  }
  return v;
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
// A token's logits are spread over LPT lanes, EPL per lane (expert e = sub + LPT * i for lane
// sub of the group).  Each of the top_k rounds takes the group maximum of the lanes' best keys and
// clears the winner's key.  With at most 256 experts and top_k <= 16 a token takes 16 lanes (four
// tokens per wavefront, reductions inside a DPP row); otherwise it takes the whole wavefront.  The
// rounds are VALU work, so four tokens per wavefront cut the instructions per token about fourfold.
constexpr int kTopkThreads = 256;

template <int LPT, int EPL>
__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(const float* __restrict__ logits,
                                                                  int32_t tokens, int32_t experts,
                                                                  int32_t top_k, int32_t normalize,
                                                                  int32_t* __restrict__ ids,
                                                                  float* __restrict__ weights) {
  constexpr int kTokPerWave = 64 / LPT;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPT, grp = lane / LPT;
  const int64_t t = ((int64_t)blockIdx.x * (kTopkThreads / 64) + (threadIdx.x >> 6)) * kTokPerWave + grp;
  const bool live = t < tokens;                       // every lane stays for the cross-lane steps
  // bounds-checked loads (zero outside the plane), no branches: the logits plane is < 2^31 bytes
  const rsrc_t rl = make_rsrc(logits, (uint32_t)((int64_t)tokens * experts * 4));
  uint64_t key[EPL];
  float v[EPL];
  uint32_t okm = 0;                                   // bit i: slot i holds an expert of a live token
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = sub + LPT * i;
    const bool ok = live && e < experts;
    okm |= ok ? (1u << i) : 0u;
    v[i] = u2f(buf_load_u32(rl, ok ? (uint32_t)((t * experts + e) * 4) : kOffNone));
  }
  bool nan_here = false;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const bool ok = (okm >> i) & 1u;
    nan_here |= ok && __builtin_isnan(v[i]);
    key[i] = ok ? join64(~(uint32_t)(sub + LPT * i), order_key(v[i])) : 0ull;
  }
  float m = 0.0f, sel_sum = 0.0f, my_x = 0.0f;
  int my_id = 0;
  for (int j = 0; j < top_k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = umax64(best, key[i]);
    best = group_max_u64<LPT>(best);
    const int e = (int)~(uint32_t)best;
    const float x = key_value((uint32_t)(best >> 32));
    m = j == 0 ? x : m;
#pragma unroll
    for (int i = 0; i < EPL; ++i) key[i] = (e == sub + LPT * i) ? 0ull : key[i];
    if (normalize) sel_sum += expf(x - m);
    my_id = sub == j ? e : my_id;
    my_x = sub == j ? x : my_x;
  }
  float denom = sel_sum;
  if (!normalize) {
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const float ex = expf(v[i] - m);
      part += ((okm >> i) & 1u) ? ex : 0.0f;
    }
    denom = group_sum<LPT>(part);
  }
  const uint64_t nan_lanes = __builtin_amdgcn_ballot_w64(nan_here);
  const uint64_t grp_mask = LPT == 64 ? ~0ull : (((1ull << LPT) - 1) << (LPT * grp));
  if (nan_lanes & grp_mask) denom = __builtin_nanf("");
  if (live && sub < top_k) {
    ids[t * top_k + sub] = my_id;
    weights[t * top_k + sub] = expf(my_x - m) / denom;
  }
}

// ------------------------------------------------------------------------------------- packing
// Pairs are numbered p = t * top_k + j.  Tokens are cut into slices of 64 (one token per lane).
//   count:  counts[e * nslices + s] = the number of pairs of slice s routed to expert e;
//   scan:   one wavefront per expert turns its row of counts into exclusive prefixes over the slices
//           and stores the expert's total in totals[e];
//   place:  each block takes the exclusive scan of the totals (the CSR offsets); each wavefront
//           ranks the pairs of its slice inside their experts, by lane (token) and then by j.
// The workspace holds counts (experts x nslices) followed by totals (experts).
constexpr int kPackThreads = 256;
constexpr int kMaxExperts = 1024;

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

// Inclusive prefix sum over the wavefront.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

__global__ __launch_bounds__(kPackThreads) void route_scan_kernel(int32_t* __restrict__ counts,
                                                                  int32_t nslices, int32_t experts,
                                                                  int32_t* __restrict__ totals) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * (kPackThreads / 64) + (threadIdx.x >> 6);
  if (e >= experts) return;                          // uniform per wavefront
  int32_t* row = counts + (int64_t)e * nslices;
  int32_t carry = 0;
  for (int base = 0; base < nslices; base += 64) {
    const int i = base + lane;
    const int32_t c = i < nslices ? row[i] : 0;
    const int32_t incl = wave_incl_scan(c, lane);
    if (i < nslices) row[i] = carry + incl - c;
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) totals[e] = carry;
}

// Place: one wavefront per slice, four slices per block.  Each lane holds its token's ids.  Fast path
// (no token lists an expert twice, as a top-k never does): every pair ORs its lane bit into a
// per-expert token mask in LDS, and a pair's rank inside its expert and slice is the number of
// lower lanes in that mask.  A slice whose tokens repeat an expert (seen as an already-set bit when
// OR-ing) ranks expert by expert instead, pairs of one lane in j order.
template <int KMAX>
__global__ __launch_bounds__(kPackThreads) void route_place_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int32_t tokens, int32_t top_k,
    int32_t experts, const int32_t* __restrict__ first_in_expert, const int32_t* __restrict__ totals,
    int32_t nslices, int32_t* __restrict__ offsets, int32_t* __restrict__ row_ids,
    int32_t* __restrict__ pair_rows, float* __restrict__ row_w) {
  __shared__ int32_t offs[kMaxExperts + 1];
  __shared__ int32_t wave_tot[kPackThreads / 64];
  extern __shared__ uint64_t tok_mask[];             // [kPackThreads / 64][experts]
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  // CSR offsets: exclusive scan of the expert totals, four consecutive experts per thread
  {
    constexpr int kPer = kMaxExperts / kPackThreads;
    int32_t v[kPer], local = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = threadIdx.x * kPer + q;
      v[q] = e < experts ? totals[e] : 0;
      local += v[q];
    }
    const int32_t incl = wave_incl_scan(local, lane);
    if (lane == 63) wave_tot[wv] = incl;
    __syncthreads();
    int32_t run = incl - local;
    for (int q = 0; q < wv; ++q) run += wave_tot[q];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = threadIdx.x * kPer + q;
      if (e < experts) offs[e] = run;
      run += v[q];
    }
    if (threadIdx.x == kPackThreads - 1) offs[experts] = run;   // the grand total
  }
  uint64_t* mask = tok_mask + wv * experts;
  for (int e = lane; e < experts; e += 64) mask[e] = 0;
  __syncthreads();
  if (blockIdx.x == 0)
    for (int e = threadIdx.x; e <= experts; e += kPackThreads) offsets[e] = offs[e];

  const int s = blockIdx.x * (kPackThreads / 64) + wv;   // this wavefront's slice
  const int64_t t = (int64_t)s * 64 + lane;
  const bool live = s < nslices && t < tokens;
  int32_t id[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int32_t e = (live && j < top_k) ? ids[t * top_k + j] : -1;
    id[j] = (e >= 0 && e < experts) ? e : -1;
    if (live && j < top_k && id[j] < 0) pair_rows[t * top_k + j] = -1;
  }
  const uint64_t bit = 1ull << lane;
  bool dup = false;
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (id[j] >= 0) dup |= (atomicOr(&mask[id[j]], bit) & bit) != 0;
  __syncthreads();
  if (__builtin_amdgcn_ballot_w64(dup) == 0) {
    // all loads first (an invalid pair reads element 0, which always exists), then the stores
    int32_t pos[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int32_t e = id[j] < 0 ? 0 : id[j];
      pos[j] = first_in_expert[id[j] < 0 ? 0 : (int64_t)e * nslices + s];
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int32_t e = id[j] < 0 ? 0 : id[j];
      pos[j] += offs[e] + __builtin_popcountll(mask[e] & (bit - 1));
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (id[j] < 0) continue;
      const int64_t p = t * top_k + j;
      row_ids[pos[j]] = (int32_t)t;
      pair_rows[p] = pos[j];
      if (row_w) row_w[pos[j]] = w[p];
    }
    return;
  }
  for (int e = 0; e < experts; ++e) {
    uint64_t any = 0;
    uint32_t below = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(id[j] == e);
      any |= m;
      below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, below));
    }
    if (any == 0) continue;                          // uniform
    int32_t pos = offs[e] + first_in_expert[(int64_t)e * nslices + s] + (int32_t)below;
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
// table of the token is wave-uniform.  Pairs are taken eight at a time: their row indices and rows
// are all loaded before the first addition, so the loads of one token overlap.
constexpr int kCombineThreads = 256;
constexpr int kCombineCols = kCombineThreads * 4;
constexpr int kCombineBatch = 8;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ y, int32_t y_rows, int32_t n, const int32_t* __restrict__ pair_rows,
    const float* __restrict__ w, int32_t top_k, int32_t nchunks, bool vec, float* __restrict__ out) {
  const int64_t t = blockIdx.x / nchunks;
  const int32_t chunk = (int32_t)(blockIdx.x - t * nchunks);
  const int32_t c = chunk * kCombineCols + threadIdx.x * 4;
  if (c >= n) return;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  bool bad = false;
  for (int j0 = 0; j0 < top_k; j0 += kCombineBatch) {
    int32_t r[kCombineBatch];
    f32x4 yv[kCombineBatch];
#pragma unroll
    for (int q = 0; q < kCombineBatch; ++q) r[q] = (j0 + q < top_k) ? pair_rows[t * top_k + j0 + q] : -1;
#pragma unroll
    for (int q = 0; q < kCombineBatch; ++q) {
      yv[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (r[q] >= y_rows) bad = true;
      if (r[q] < 0 || r[q] >= y_rows) continue;
      const float* yr = y + (int64_t)r[q] * n + c;
      if (vec) {
        yv[q] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yr));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) yv[q][e] = (c + e < n) ? yr[e] : 0.0f;
      }
    }
#pragma unroll
    for (int q = 0; q < kCombineBatch; ++q) {
      if (r[q] < 0 || r[q] >= y_rows) continue;
      if (w) {
        const float wj = w[t * top_k + j0 + q];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(wj, yv[q][e], acc[e]);
      } else {
        acc += yv[q];
      }
    }
  }
  if (bad) acc = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
  float* o = out + t * n + c;
  if (vec) {
    *reinterpret_cast<f32x4*>(o) = acc;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (c + e < n) o[e] = acc[e];
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int32_t tokens, int32_t experts, int32_t top_k,
                             int32_t normalize, int32_t* ids, float* weights, hipStream_t stream) {
#define FP4MOE_TOPK(L, N)                                                                                    \
  hipLaunchKernelGGL((route_topk_kernel<L, N>), grid, dim3(kTopkThreads), 0, stream, logits, tokens, experts, \
                     top_k, normalize, ids, weights)
  if (experts <= 256 && top_k <= 16) {
    const int tok_per_block = (kTopkThreads / 64) * 4;
    const dim3 grid((tokens + tok_per_block - 1) / tok_per_block);
    const int epl = (experts + 15) / 16;
    if (epl <= 1) FP4MOE_TOPK(16, 1);
    else if (epl <= 2) FP4MOE_TOPK(16, 2);
    else if (epl <= 4) FP4MOE_TOPK(16, 4);
    else if (epl <= 8) FP4MOE_TOPK(16, 8);
    else FP4MOE_TOPK(16, 16);
  } else {
    const dim3 grid((tokens + kTopkThreads / 64 - 1) / (kTopkThreads / 64));
    const int epl = (experts + 63) / 64;
    if (epl <= 4) FP4MOE_TOPK(64, 4);
    else if (epl <= 8) FP4MOE_TOPK(64, 8);
    else FP4MOE_TOPK(64, 16);
  }
#undef FP4MOE_TOPK
  return hipGetLastError();
}

int64_t route_pack_workspace_elems(int32_t tokens, int32_t experts) {
  return (int64_t)experts * ((tokens + 63) / 64) + experts;
}

hipError_t launch_route_pack(const int32_t* ids, const float* w, int32_t tokens, int32_t top_k,
                             int32_t experts, int32_t* offsets, int32_t* row_ids, int32_t* pair_rows,
                             float* row_w, int32_t* workspace, hipStream_t stream) {
  const int32_t nslices = (tokens + 63) / 64;
  int32_t* counts = workspace;
  int32_t* totals = workspace + (int64_t)experts * nslices;
  if (nslices > 0) {
    hipLaunchKernelGGL(route_count_kernel, dim3(nslices), dim3(kPackThreads), experts * sizeof(int32_t),
                       stream, ids, tokens, top_k, experts, counts, nslices);
    if (hipError_t e = hipGetLastError()) return e;
  }
  hipLaunchKernelGGL(route_scan_kernel, dim3((experts + 3) / 4), dim3(kPackThreads), 0, stream, counts, nslices,
                     experts, totals);
  if (hipError_t e = hipGetLastError()) return e;
  // at least one block, so that the offsets are written even without tokens
  const int per_block = kPackThreads / 64;
  const dim3 grid(nslices > 0 ? (nslices + per_block - 1) / per_block : 1);
  const size_t lds = (size_t)per_block * experts * sizeof(uint64_t);
#define FP4MOE_PLACE(N)                                                                                   \
  hipLaunchKernelGGL(route_place_kernel<N>, grid, dim3(kPackThreads), lds, stream, ids, w, tokens, top_k, \
                     experts, counts, totals, nslices, offsets, row_ids, pair_rows, row_w)
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
