// gemm_decode.hip -- FP8-activation x block-scaled FP4 expert GEMM for few rows per expert.
//
// What is computed (memra-engine 0.98.0 dsv4_native_gemm_gate.rs page, `f64_ref` / `ExpertRaw`):
//   out[r, c] = sum_j ( sum_{k in group j} E4M3(A[r,k]) * E2M1(W[c,k]) ) * ws[c,j] * as[r, k/128]
// accumulated in f32, with NVFP4 (E4M3 scale per 16, times scale2) or MXFP4 (E8M0 scale per 32)
// weights.  Grouped form: rows packed per expert with a CSR offsets array (kernel_check.rs page,
// f16g grouped GEMM section).
//
// Work decomposition.  A workgroup of 4 wavefronts owns 64 output columns of one expert and streams
// that expert's 64 weight rows (k/2 + k/gs bytes each) once per pass of up to 32 activation rows;
// with decode-sized row counts that is one pass, so the weights are read from HBM exactly once.
// The 4 wavefronts split k: wavefront w takes the 128-wide k blocks w, w+4, w+8, ...; each covers
// all 64 columns (4 MFMA column tiles) and all rows of the pass (1 or 2 MFMA row tiles), and the
// 4 partial tiles are added in a fixed order through LDS at the end (deterministic).
//
// Inner step for one 128-wide k block, per lane (c16 = lane%16, g = lane/16):
//   weights: one 16-byte load per column tile = 32 nibbles k0+32g .. +32 of column c16.
//   NVFP4: f16 MFMA 16x16x32.  Nibbles -> f16 with the hardware FP4 conversion, times the E4M3
//     scale in f16 (exact); activation bytes -> f16 (exact).  MFMA i of the block pairs lane
//     group g with k = k0 + 32g + 8i .. +8, so the 128 k of a block are one activation-scale group:
//     the block's four MFMAs accumulate a partial tile that is scaled by as[r, block] in one f32
//     FMA.  scale2 multiplies the final sum (exact for power-of-two scale2; otherwise within one
//     f32 rounding of the per-group scale, inside the accuracy bound).
//   MXFP4: one block-scaled MFMA 16x16x128 per column tile, raw E4M3 activation bytes and raw
//     nibbles, E8M0 weight scales and the activation scale's exponent as the E8M0 row scale: no
//     conversion work at all.
//
// Workgroup order is XCD-aware when there are >= 8 experts: consecutive workgroup ids go to
// different XCDs, so the ids are arranged such that every column tile of one expert lands on the
// same XCD and the expert's activation rows are fetched into one L2 only.
#include "device_common.h"
#include "kernels.h"

namespace fp4moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTileN = 64;
constexpr int kCT = kTileN / 16;
constexpr int kRowsPerPass = 32;
constexpr int kNV = 0;
constexpr int kMX = 1;

struct ExpertView {
  const uint8_t* w;
  const uint8_t* s;
  float scale2;
  int kind;
  int rb, re;          // packed rows [rb, re)
};

// Activation row of packed row `prow`: row_ids[prow] (or prow), -2 when the entry is out of range.
__device__ __forceinline__ int act_row(const GemmArgs& p, int prow) {
  if (!p.row_ids) return prow;
  const int r = p.row_ids[prow];
  return (r >= 0 && r < p.a_rows) ? r : -2;
}

// Buffer descriptors of one pass (uniform per workgroup).
struct PassRsrc {
  rsrc_t w, s, a, as;
};

template <int MT>
struct BlockData {
  u32x4 wq[kCT];          // 32 nibbles of each column tile
  uint32_t sc[kCT];       // NVFP4: 2 E4M3 scale bytes; MXFP4: 1 E8M0 byte
  u32x4 aq[MT][2];        // 32 activation bytes per row tile
  float asa[MT];          // activation scale of this lane's operand row (row l%16) for the block
};

// Per-lane byte offsets of block 0; block b adds b times the per-block strides.
template <int MT>
struct PassOffsets {
  uint32_t w[kCT], s[kCT], a[MT], as[MT];
};

// Loads of block b.  Every load is issued even when b is past the last block: its offset is then
// out of range and the load returns zeros without touching memory, so the number of outstanding
// loads is the same on every path and the compiler's wait counts stay exact.
template <int MT, int KIND>
__device__ __forceinline__ void load_block(const PassRsrc& r, const PassOffsets<MT>& o, int b,
                                           bool valid, BlockData<MT>& d) {
  const uint32_t ub = (uint32_t)b;
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) {
    d.wq[ct] = buf_load_x4(r.w, valid ? o.w[ct] + ub * 64u : kOffNone);
    d.sc[ct] = (KIND == kNV) ? buf_load_u16(r.s, valid ? o.s[ct] + ub * 8u : kOffNone)
                             : buf_load_u8(r.s, valid ? o.s[ct] + ub * 4u : kOffNone);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint32_t ab = valid ? o.a[mt] + ub * 128u : kOffNone;
    d.aq[mt][0] = buf_load_x4(r.a, ab);
    d.aq[mt][1] = buf_load_x4(r.a, ab + (KIND == kNV ? 16u : 64u));
    d.asa[mt] = u2f(buf_load_u32(r.as, valid ? o.as[mt] + ub * 4u : kOffNone));
  }
}

template <int MT>
__device__ __forceinline__ void compute_block_nv(const BlockData<MT>& d, f32x4 (&acc)[MT][kCT]) {
  const int g = (threadIdx.x & 63) >> 4;
  f32x4 part[MT][kCT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) part[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h16x8 af[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      af[mt] = e4m3x8_to_f16(d.aq[mt][i >> 1][2 * (i & 1)], d.aq[mt][i >> 1][2 * (i & 1) + 1]);
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      const h16x2 ws = e4m3x2_to_f16<false>(d.sc[ct]);
      const h16x8 bf = e2m1x8_scaled_f16(d.wq[ct][i], ws[i >> 1]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) part[mt][ct] = mfma16x16x32_f16(af[mt], bf, part[mt][ct]);
    }
  }
  // The partial tile covers exactly one 128-wide activation-scale group: scale its rows.  Result
  // row 4g+v of the tile is operand row 4g+v, whose scale sits in lane 4g+v.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float as[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) as[v] = __shfl(d.asa[mt], 4 * g + v, 64);
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[mt][ct][v] = fmaf(part[mt][ct][v], as[v], acc[mt][ct][v]);
  }
}

template <int MT>
__device__ __forceinline__ void compute_block_mx(const BlockData<MT>& d, f32x4 (&acc)[MT][kCT]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const i32x8 a = {(int)d.aq[mt][0][0], (int)d.aq[mt][0][1], (int)d.aq[mt][0][2], (int)d.aq[mt][0][3],
                     (int)d.aq[mt][1][0], (int)d.aq[mt][1][1], (int)d.aq[mt][1][2], (int)d.aq[mt][1][3]};
    const int sa = (int)((f2u(d.asa[mt]) >> 23) & 0xFFu);   // power-of-two scale -> E8M0
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      const i32x8 bw = {(int)d.wq[ct][0], (int)d.wq[ct][1], (int)d.wq[ct][2], (int)d.wq[ct][3], 0, 0, 0, 0};
      acc[mt][ct] = mfma16x16x128_f8f4(a, bw, acc[mt][ct], sa, (int)d.sc[ct]);
    }
  }
}

template <int MT, int KIND>
__device__ __forceinline__ void compute_block(const BlockData<MT>& d, f32x4 (&acc)[MT][kCT]) {
  if constexpr (KIND == kNV) compute_block_nv<MT>(d, acc);
  else compute_block_mx<MT>(d, acc);
}

// One pass over the packed rows [m0, mend) (at most 32) for the 64 columns starting at n0.
template <int MT, int KIND>
__device__ void run_pass(const GemmArgs& p, const ExpertView& ex, int n0, int m0, int mend,
                         f32x4 (*red)[2][kCT][64]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  const int c16 = lane & 15, g = lane >> 4;
  const int k = p.k, nblk = k >> 7;
  constexpr int GS = (KIND == kNV) ? 16 : 32;

  PassRsrc r;
  r.w = make_rsrc(ex.w, (uint32_t)p.n * (uint32_t)(k / 2));
  r.s = make_rsrc(ex.s, (uint32_t)p.n * (uint32_t)(k / GS));
  r.a = make_rsrc(p.a_codes, (uint32_t)p.a_rows * (uint32_t)k);
  r.as = make_rsrc(p.a_scales, (uint32_t)p.a_rows * (uint32_t)nblk * 4u);
  PassOffsets<MT> o;
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) {
    const int col = n0 + 16 * ct + c16;
    const bool ok = col < p.n;
    o.w[ct] = ok ? (uint32_t)col * (uint32_t)(k / 2) + 16u * g : kOffNone;
    o.s[ct] = ok ? (uint32_t)col * (uint32_t)(k / GS) + (KIND == kNV ? 2u * g : (uint32_t)g) : kOffNone;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int prow = m0 + 16 * mt + c16;
    const int ar = prow < mend ? act_row(p, prow) : -1;
    o.a[mt] = ar >= 0 ? (uint32_t)ar * (uint32_t)k + (KIND == kNV ? 32u * g : 16u * g) : kOffNone;
    o.as[mt] = ar >= 0 ? (uint32_t)ar * (uint32_t)nblk * 4u : kOffNone;
  }

  f32x4 acc[MT][kCT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) acc[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Blocks wave, wave+4, ... through a ring of D register buffers: the loads of the next D-1
  // blocks are in flight while one block is computed (the stream is latency-bound otherwise).
  constexpr int D = (MT == 1) ? 4 : 2;
  BlockData<MT> buf[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const int bj = wave + kWaves * j;
    load_block<MT, KIND>(r, o, bj, bj < nblk, buf[j]);
    // Pin every group of loads where it is written: the machine scheduler would otherwise sink
    // loads toward their first use (the loop latch) or reorder the prologue, and the wait counts
    // at the loop head would then drain the whole ring.
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int b0 = wave; b0 < nblk; b0 += kWaves * D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int bb = b0 + kWaves * j;
      if (bb < nblk) compute_block<MT, KIND>(buf[j], acc);
      const int bn = bb + kWaves * D;
      load_block<MT, KIND>(r, o, bn, bn < nblk, buf[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Fixed-order reduction of the 4 wavefronts' partial tiles.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) red[wave][mt][ct][lane] = acc[mt][ct];
  __syncthreads();
  const float post = (KIND == kNV) ? ex.scale2 : 1.0f;
  for (int t = wave; t < MT * kCT; t += kWaves) {
    const int mt = t / kCT, ct = t % kCT;
    f32x4 sum = red[0][mt][ct][lane];
    sum += red[1][mt][ct][lane];
    sum += red[2][mt][ct][lane];
    sum += red[3][mt][ct][lane];
    const int col = n0 + 16 * ct + c16;
    if (col < p.n) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int crow = m0 + 16 * mt + 4 * g + v;
        if (crow < mend) {
          const int ar = act_row(p, crow);
          p.out[(size_t)crow * p.n + col] = ar >= 0 ? sum[v] * post : __builtin_nanf("");
        }
      }
    }
  }
  __syncthreads();
}

template <int KIND>
__device__ void run_expert(const GemmArgs& p, const ExpertView& ex, int n0, f32x4 (*red)[2][kCT][64]) {
  for (int m0 = ex.rb; m0 < ex.re; m0 += kRowsPerPass) {
    const int mend = min(m0 + kRowsPerPass, ex.re);
    if (mend - m0 > 16) run_pass<2, KIND>(p, ex, n0, m0, mend, red);
    else run_pass<1, KIND>(p, ex, n0, m0, mend, red);
  }
}

__global__ __launch_bounds__(kThreads, 2) void gemm_decode_kernel(GemmArgs p, int ntn, int xcd_map) {
  __shared__ f32x4 red[kWaves][2][kCT][64];
  const int L = blockIdx.x;
  int e, nt;
  if (xcd_map) {
    const int idx = L >> 3;
    e = (idx / ntn) * 8 + (L & 7);
    nt = idx % ntn;
  } else {
    e = L / ntn;
    nt = L % ntn;
  }
  if (e >= p.num_experts) return;
  ExpertView ex;
  if (p.offsets) {
    const int lo = min(max(p.offsets[e], 0), p.total_rows);
    const int hi = min(max(p.offsets[e + 1], lo), p.total_rows);
    ex = ExpertView{reinterpret_cast<const uint8_t*>(p.w_ptrs[e]),
                    reinterpret_cast<const uint8_t*>(p.s_ptrs[e]), p.scale2s[e], p.kinds[e], lo, hi};
  } else {
    ex = ExpertView{p.w, p.s, p.scale2, p.kind, 0, p.total_rows};
  }
  if (ex.rb >= ex.re) return;
  const int n0 = nt * kTileN;
  if (ex.kind == kNV) {
    run_expert<kNV>(p, ex, n0, red);
  } else if (ex.kind == kMX) {
    run_expert<kMX>(p, ex, n0, red);
  } else {
    for (int i = threadIdx.x; i < (ex.re - ex.rb) * kTileN; i += kThreads) {
      const int r = ex.rb + i / kTileN, col = n0 + i % kTileN;
      if (col < p.n) p.out[(size_t)r * p.n + col] = __builtin_nanf("");
    }
  }
}

}  // namespace

hipError_t launch_gemm_decode(const GemmArgs& a, hipStream_t stream) {
  const int ntn = (a.n + kTileN - 1) / kTileN;
  const int xcd_map = a.num_experts >= 8 ? 1 : 0;
  const int64_t eg = xcd_map ? (int64_t)(a.num_experts + 7) / 8 * 8 : a.num_experts;
  const int64_t blocks = eg * ntn;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(gemm_decode_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, ntn,
                     xcd_map);
  return hipGetLastError();
}

}  // namespace fp4moe
