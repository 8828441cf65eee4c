// gemm_skinny.hip -- FP8-activation x block-scaled FP4 GEMM for very few rows: one expert with
// g <= 16 rows, or a grouped launch with at most 128 packed rows (a decode step of a few tokens),
// split over k so that such a launch fills the chip.
//
// What is computed is the same definition as the other two GEMM kernels (memra-engine 0.98.0
// dsv4_native_gemm_gate.rs page, `f64_ref` / `ExpertRaw`):
//   out[r, c] = sum_j ( sum_{k in group j} E4M3(A[r,k]) * E2M1(W[c,k]) ) * ws[c,j] * as[r, k/128]
// accumulated in f32.  A single expert of the decode shapes (n = 2048 or 7168 columns) gives the
// row-streaming kernel only n/256 = 8..28 workgroups, far too few to stream 8 MB of weights; this
// kernel splits each 16-column tile's k over KS wavefronts: wavefront kw takes the 128-wide blocks
// b = kw, kw + KS, kw + 2 KS, ..., so the KS wavefronts of a tile read KS consecutive 1 KB weight
// runs at a time with swizzled planes.  A single-expert launch picks KS from k alone, the smallest
// of 4, 8 and 16 that leaves each wavefront at most kRing blocks (every load of the launch is then
// issued before anything waits); a workgroup holds 8 wavefronts (2 tiles at KS = 4, 1 at KS = 8) or
// 16 (KS = 16).  A grouped launch keeps 8 wavefronts per workgroup and gives a tile KS = 8, 4, 2 or
// 1 wavefronts (the workgroup then owning 8 / KS tiles), so that each wavefront streams a longer run
// of blocks.
//
// Data movement: a wavefront keeps kRing blocks of loads in flight, refilling a slot as soon as it
// has computed on it: per block the lane's 16 weight bytes, its scale bytes and its 32 bytes of
// the activation operand (which hit L2 after the first workgroup).  Only the activation scales go
// through LDS: they are loaded before the weight ring, so storing them waits for them alone, and
// the barrier that publishes them does not wait for the ring.
//
// Arithmetic per block (lane c16 = lane%16 holds column 16t + c16 and activation row c16; lane group
// g = lane/16 holds k = 32g .. +32 of the block), as in the row-streaming kernel: NVFP4 on exact f16
// operands (nibble -> f16 times the E4M3 scale in f16), MXFP4 on exact bf16 operands (the E8M0 scale
// applied by the conversion), four 16x16x32 MFMAs cover one activation-scale group, whose partial
// tile is scaled by as[r, b] with one f32 FMA per output.  The KS wavefronts' f32 tiles of a column
// tile are then summed through LDS in wavefront order (a fixed order for a given KS, n and k: the
// result does not depend on g or on timing), and scale2 multiplies the sum.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace fp4moe {
namespace {

constexpr int kThreads = 512;              // grouped form: 8 wavefronts per workgroup
constexpr int kWaves = 8;
constexpr int kMaxWaves = 16;              // single-expert form: up to 16 wavefronts per workgroup
constexpr int kRing = 4;                    // blocks in flight per wavefront (refilled as they are consumed)
constexpr int kMaxRows = 16;
constexpr int kMaxK = 8192;
// Grouped launches take this kernel automatically when they hold at most kGroupedAutoRows packed
// rows (two tokens at top-8: measured over 256 experts of k = 7168, n = 2048, one token takes 21 us
// here against 44 us in the row-streaming kernel, two tokens 33 against 51, four tokens 58 against
// 56-60, eight 107 against 100), and up to kGroupedMaxRows when the schedule forces it.
constexpr int kGroupedMaxRows = 128;
constexpr int kGroupedAutoRows = 16;
constexpr int kMaxExperts = 1024;
constexpr int kGridCap = 512;                // persistent grid of the grouped form (two per compute unit)
constexpr int kNV = 0;
constexpr int kMX = 1;
constexpr int kSwizzled = 2;

struct Smem {
  float as[(kMaxK / 128) * kMaxRows];        // activation scales [block][row]
  f32x4 red[kMaxWaves][64];                  // per-wavefront result tiles
  int active[kMaxExperts];                   // grouped: the experts with rows, in id order
  int wave_count[kWaves];
};

template <bool SWZ>
__device__ __forceinline__ u32x4 wload(rsrc_t r, uint32_t off) {
  if constexpr (SWZ) return buf_load_x4_nt(r, off);
  else return buf_load_x4(r, off);
}

// One expert's planes and scale2.
struct View {
  const uint8_t* w;
  const uint8_t* s;
  float scale2;
};

// Activation row of packed row `prow`: row_ids[prow] (or prow), -2 when the entry is out of range.
__device__ __forceinline__ int act_row(const GemmArgs& p, int prow) {
  if (!p.row_ids) return prow;
  const int r = p.row_ids[prow];
  return (r >= 0 && r < p.a_rows) ? r : -2;
}

// Packed rows [m0, m0 + mrows) (mrows <= 16) of expert `ex`, column tile group tg: KS wavefronts
// per 16-column tile, so the group holds kWaves / KS tiles, tiles (kWaves / KS) tg + sub, and the
// wavefront kw = wave % KS of a tile takes the blocks b = kw, kw + KS, ...
template <int KIND, bool SWZ, int KS, int WAVES>
__device__ void run(const GemmArgs& p, const View& ex, int tg, int m0, int mrows, Smem& sm) {
  static_assert(KS >= 1 && WAVES % KS == 0 && WAVES <= kMaxWaves, "wavefronts per tile");
  constexpr int kThr = 64 * WAVES;
  const int tid = threadIdx.x, lane = tid & 63, c16 = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = wave / KS, kw = wave % KS;
  const int t = (WAVES / KS) * tg + sub;
  const int k = p.k, nblk = k >> 7, nq = (nblk + 3) >> 2;
  const int col = 16 * t + c16;
  const uint32_t n16 = (uint32_t)(p.n + 15) >> 4;

  rsrc_t rw, rs;
  if constexpr (SWZ) {
    rw = make_rsrc(ex.w, n16 * 16u * (uint32_t)(k / 2));
    rs = make_rsrc(ex.s, n16 * (uint32_t)nq * (KIND == kNV ? 512u : 256u));
  } else {
    rw = make_rsrc(ex.w, (uint32_t)p.n * (uint32_t)(k / 2));
    rs = make_rsrc(ex.s, (uint32_t)p.n * (uint32_t)(k / (KIND == kNV ? 16 : 32)));
  }
  // Block-0 offsets of this lane's weight piece and scale bytes (kOffNone past n).
  const uint32_t piece = (uint32_t)(16 * g + c16);
  uint32_t w0, s0;
  if constexpr (SWZ) {
    w0 = (uint32_t)t * (uint32_t)nblk * 1024u + 16u * piece;
    s0 = ((uint32_t)t * (uint32_t)nq * 64u + piece) * (KIND == kNV ? 8u : 4u);
  } else {
    w0 = (uint32_t)col * (uint32_t)(k / 2) + 16u * g;
    s0 = KIND == kNV ? (uint32_t)col * (uint32_t)(k / 16) + 2u * g : (uint32_t)col * (uint32_t)(k / 32) + g;
  }
  if (col >= p.n) w0 = s0 = kOffNone;
  auto w_off = [&](int b) -> uint32_t {
    if (b >= nblk || w0 == kOffNone) return kOffNone;
    return w0 + (uint32_t)b * (SWZ ? 1024u : 64u);
  };
  // NVFP4: the scale pair of the lane's piece (2 bytes); MXFP4: its scale byte.
  auto s_load = [&](int b) -> uint32_t {
    uint32_t o = kOffNone;
    if (b < nblk && s0 != kOffNone) {
      const uint32_t ub = (uint32_t)b;
      if constexpr (SWZ) o = s0 + (ub >> 2) * (KIND == kNV ? 512u : 256u) + (ub & 3u) * (KIND == kNV ? 2u : 1u);
      else o = s0 + ub * (KIND == kNV ? 8u : 4u);
    }
    if constexpr (KIND == kNV) return buf_load_u16(rs, o);
    else return buf_load_u8(rs, o);
  };

  // Activation operand of block b: packed row m0 + c16, bytes 32g .. +32 of the block (rows past
  // mrows and rows whose row_ids entry is invalid read zero).
  const rsrc_t ra = make_rsrc(p.a_codes, (uint32_t)p.a_rows * (uint32_t)k);
  const int arow = c16 < mrows ? act_row(p, m0 + c16) : -1;
  const uint32_t a0 = arow >= 0 ? (uint32_t)arow * (uint32_t)k + 32u * g : kOffNone;
  auto a_off = [&](int b) -> uint32_t { return (b < nblk && a0 != kOffNone) ? a0 + (uint32_t)b * 128u : kOffNone; };

  const int nbw = (nblk - kw + KS - 1) / KS;
  u32x4 wq[kRing], aq[kRing][2];
  uint32_t sq[kRing];
  // Activation scales [block][row] into LDS, loaded before the weight ring so that storing them waits
  // for these loads only; the barrier after the ring waits for LDS, not for the ring's loads.
  {
    const rsrc_t rsa = make_rsrc(p.a_scales, (uint32_t)p.a_rows * (uint32_t)nblk * 4u);
    constexpr int kPer = kMaxRows * (kMaxK / 128) / kThr;
    float v[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = tid + kThr * j, b = i / kMaxRows, r = i % kMaxRows;
      const int ar = (b < nblk && r < mrows) ? act_row(p, m0 + r) : -1;
      v[j] = u2f(buf_load_u32(rsa, ar >= 0 ? ((uint32_t)ar * (uint32_t)nblk + b) * 4u : kOffNone));
    }
    __builtin_amdgcn_sched_barrier(0);
    // Ring: the wavefront's blocks b = kw + KS i, weights, scale bytes and activation operand of
    // each, all issued before anything waits.

#pragma unroll
  for (int j = 0; j < kRing; ++j) {
    const int b = j < nbw ? kw + KS * j : nblk;
    wq[j] = wload<SWZ>(rw, w_off(b));
    sq[j] = s_load(b);
    aq[j][0] = buf_load_x4(ra, a_off(b));
    aq[j][1] = buf_load_x4(ra, a_off(b) == kOffNone ? kOffNone : a_off(b) + 16u);
  }
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int j = 0; j < kPer; ++j) sm.as[tid + kThr * j] = v[j];
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < nbw; i0 += kRing) {
#pragma unroll
    for (int j = 0; j < kRing; ++j) {
      const int i = i0 + j;
      if (i < nbw) {
        const int b = kw + KS * i;
        f32x4 part = {0.f, 0.f, 0.f, 0.f};
        if constexpr (KIND == kNV) {
          const h16x2 ws = e4m3x2_to_f16<false>(sq[j]);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const u32x4& a = aq[j][m >> 1];
            const h16x8 af = e4m3x8_to_f16(a[2 * (m & 1)], a[2 * (m & 1) + 1]);
            part = mfma16x16x32_f16(af, e2m1x8_scaled_f16(wq[j][m], ws[m >> 1]), part);
          }
        } else {
          const float sv = u2f((sq[j] & 0xFFu) << 23);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const u32x4& a = aq[j][m >> 1];
            const bf16x8 af = e4m3x8_to_bf16(a[2 * (m & 1)], a[2 * (m & 1) + 1]);
            part = mfma16x16x32_bf16(af, e2m1x8_pow2_bf16(wq[j][m], sv), part);
          }
        }
        // the partial tile covers one activation-scale group: result row 4g+v takes as[4g+v, b]
        const f32x4 as = *reinterpret_cast<const f32x4*>(sm.as + b * kMaxRows + 4 * g);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = fmaf(part[v], as[v], acc[v]);
      }
      // refill the slot with the block kRing further on (when the wavefront has more than kRing blocks)
      if (i0 + kRing < nbw) {
        const int inext = i + kRing;
        const int bn = inext < nbw ? kw + KS * inext : nblk;
        wq[j] = wload<SWZ>(rw, w_off(bn));
        sq[j] = s_load(bn);
        aq[j][0] = buf_load_x4(ra, a_off(bn));
        aq[j][1] = buf_load_x4(ra, a_off(bn) == kOffNone ? kOffNone : a_off(bn) + 16u);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Sum the tile's KS wavefront partials in wavefront order, apply scale2, store rows 4g+v of
  // column col.
  sm.red[wave][lane] = acc;
  __syncthreads();
  if (kw == 0) {
    f32x4 sum = sm.red[wave][lane];
#pragma unroll
    for (int w = 1; w < KS; ++w) {
      const f32x4 o = sm.red[wave + w][lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) sum[v] += o[v];
    }
    const float post = KIND == kNV ? ex.scale2 : 1.0f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 4 * g + v;
      if (r < mrows && col < p.n) {
        const bool bad = act_row(p, m0 + r) < 0;
        p.out[(size_t)(m0 + r) * p.n + col] = bad ? __builtin_nanf("") : sum[v] * post;
      }
    }
  }
}

// Packed rows [lo, hi) of expert `ex` for tile group tg, in passes of 16 rows (every pass streams
// the group's weights again; the host sends only launches with few rows per expert here).
template <int KS, int WAVES>
__device__ void run_rows(const GemmArgs& p, const View& ex, int kind, int tg, int lo, int hi, Smem& sm) {
  constexpr int kTilesPerGroup = WAVES / KS;
  constexpr int kThr = 64 * WAVES;
  for (int m0 = lo; m0 < hi; m0 += kMaxRows) {
    const int mrows = min(kMaxRows, hi - m0);
    if (kind == kNV) {
      run<kNV, false, KS, WAVES>(p, ex, tg, m0, mrows, sm);
    } else if (kind == kMX) {
      run<kMX, false, KS, WAVES>(p, ex, tg, m0, mrows, sm);
    } else if (kind == (kNV | kSwizzled)) {
      run<kNV, true, KS, WAVES>(p, ex, tg, m0, mrows, sm);
    } else if (kind == (kMX | kSwizzled)) {
      run<kMX, true, KS, WAVES>(p, ex, tg, m0, mrows, sm);
    } else {
      // a weight format the kernel does not take: NaN rows
      for (int i = threadIdx.x; i < mrows * 16 * kTilesPerGroup; i += kThr) {
        const int col = 16 * kTilesPerGroup * tg + (i % (16 * kTilesPerGroup));
        if (col < p.n) p.out[(size_t)(m0 + i / (16 * kTilesPerGroup)) * p.n + col] = __builtin_nanf("");
      }
    }
    __syncthreads();                         // the next pass reuses the LDS
  }
}

// Rows [lo, hi) of expert e after clamping its offsets to [0, total_rows].
__device__ __forceinline__ int2 expert_rows(const GemmArgs& p, int e) {
  const int lo = min(max(p.offsets[e], 0), p.total_rows);
  const int hi = min(max(p.offsets[e + 1], lo), p.total_rows);
  return make_int2(lo, hi);
}

// Grouped (persistent): every workgroup lists the experts that have rows (a block-wide scan over
// the offsets into LDS), then takes the (active expert, tile group) items blockIdx.x,
// blockIdx.x + gridDim.x, ... -- no workgroup is spent on an empty expert.  The host picks KS so that there are about as many items as workgroups: a wavefront
// then streams one long run of blocks, and its load ring does not drain between short items.
// At most 128 registers (4 wavefronts per SIMD): two workgroups share a compute unit, so one
// computes while the other waits for its loads (one token over 256 experts, 8 wavefronts per tile:
// 26 us, against 30 us with every block of k in flight and one workgroup per compute unit).
template <int KS>
__global__ __launch_bounds__(kThreads, 4) void gemm_skinny_kernel(GemmArgs p, int ngroups) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.num_experts;
  constexpr int kPer = kMaxExperts / kThreads;                 // experts per thread
  int flags[kPer], cnt = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid * kPer + j;
    int2 r = make_int2(0, 0);
    if (e < E) r = expert_rows(p, e);
    flags[j] = r.y > r.x;
    cnt += flags[j];
  }
  int incl = cnt;                                              // inclusive scan inside the wavefront
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) sm.wave_count[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < kWaves; ++w) {
    const int c = sm.wave_count[w];
    if (w < wave) base += c;
    total += c;
  }
  int pos = base + incl - cnt;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (flags[j]) sm.active[pos++] = tid * kPer + j;
  __syncthreads();
  const int items = total * ngroups;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int e = sm.active[it / ngroups], tg = it % ngroups;
    const int2 r = expert_rows(p, e);
    const View ex{reinterpret_cast<const uint8_t*>(p.w_ptrs[e]), reinterpret_cast<const uint8_t*>(p.s_ptrs[e]),
                  p.scale2s[e]};
    run_rows<KS, kWaves>(p, ex, p.kinds[e], tg, r.x, r.y, sm);
  }
}

// Single expert: workgroup tg owns WAVES / KS column tiles of KS wavefronts each, and the host picks
// KS from k alone (so a row gives the same bits alone or in a batch) such that each wavefront
// holds at most kRing blocks: every load of the launch is in flight after one issue round.  The
// arguments are scalars, in the order the kernel first needs them, so that all but the output
// pointer arrive preloaded in SGPRs (no kernel-argument load before the first weight load: 7.3
// against 7.8 us for n = 2048, k = 7168, g = 8, and 6.3 against 7.0 us for n = 7168, k = 2048).
template <int KS, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 4) void gemm_skinny_single_kernel(const float* a_scales, const uint8_t* a_codes,
                                                                          const uint8_t* w, const uint8_t* s, int k, int n,
                                                                          int rows, int kind, float scale2, float* out) {
  __shared__ Smem sm;
  GemmArgs p{};
  p.a_codes = a_codes;
  p.a_scales = a_scales;
  p.a_rows = rows;
  p.total_rows = rows;
  p.num_experts = 1;
  p.w = w;
  p.s = s;
  p.scale2 = scale2;
  p.kind = kind;
  p.out = out;
  p.n = n;
  p.k = k;
  run_rows<KS, WAVES>(p, View{w, s, scale2}, kind, blockIdx.x, 0, rows, sm);
}

template <int KS, int WAVES>
hipError_t launch_single(const GemmArgs& a, int tiles, hipStream_t stream) {
  constexpr int kTilesPerGroup = WAVES / KS;
  const int ngroups = (tiles + kTilesPerGroup - 1) / kTilesPerGroup;
  hipLaunchKernelGGL((gemm_skinny_single_kernel<KS, WAVES>), dim3((unsigned)ngroups), dim3(64 * WAVES), 0, stream,
                     a.a_scales, a.a_codes, a.w, a.s, a.k, a.n, a.total_rows, a.kind, a.scale2, a.out);
  return hipGetLastError();
}

template <int KS>
hipError_t launch_ks(const GemmArgs& a, int tiles, hipStream_t stream) {
  constexpr int kTilesPerGroup = kWaves / KS;
  const int ngroups = (tiles + kTilesPerGroup - 1) / kTilesPerGroup;
  const int64_t grid = a.offsets ? std::min<int64_t>((int64_t)a.num_experts * ngroups, kGridCap) : ngroups;
  hipLaunchKernelGGL(gemm_skinny_kernel<KS>, dim3((unsigned)grid), dim3(kThreads), 0, stream, a, ngroups);
  return hipGetLastError();
}

}  // namespace

bool gemm_skinny_fits(int32_t g, int32_t n, int32_t k) {
  return g >= 1 && g <= kMaxRows && k >= 128 && k <= kMaxK && n >= 1;
}

bool gemm_skinny_grouped_fits(int64_t total_rows, int32_t num_experts, int32_t n, int32_t k, bool forced) {
  const int64_t items = (int64_t)num_experts * ((n + 15) / 16);
  return total_rows >= 1 && total_rows <= (forced ? kGroupedMaxRows : kGroupedAutoRows) && k >= 128 &&
         k <= kMaxK && n >= 1 && num_experts <= kMaxExperts && items < ((int64_t)1 << 31);
}

hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  const int tiles = (a.n + 15) / 16;
  if (!a.offsets) {
    // Single expert: at most kRing blocks per wavefront (k <= 8192: at most 64 blocks).
    const int nblk = a.k / 128;
    if (nblk <= 4 * kRing) return launch_single<4, 8>(a, tiles, stream);
    if (nblk <= 8 * kRing) return launch_single<8, 8>(a, tiles, stream);
    return launch_single<16, 16>(a, tiles, stream);
  }
  // Grouped: at most min(E, rows) experts hold rows.  Take the fewest wavefronts per tile that
  // still give every workgroup of the persistent grid an item (one token at top-8 over n = 2048:
  // 8 experts x 128 tiles -> 4 wavefronts per tile, 512 items).
  const int64_t active = std::min<int64_t>(a.num_experts, a.total_rows);
  for (int ks = 1; ks < kWaves; ks *= 2) {
    const int64_t items = active * ((tiles + kWaves / ks - 1) / (kWaves / ks));
    if (items >= kGridCap) {
      if (ks == 1) return launch_ks<1>(a, tiles, stream);
      if (ks == 2) return launch_ks<2>(a, tiles, stream);
      return launch_ks<4>(a, tiles, stream);
    }
  }
  return launch_ks<kWaves>(a, tiles, stream);
}

}  // namespace fp4moe
