// gemm_prefill.hip -- FP8-activation x block-scaled FP4 expert GEMM for many rows per expert.
//
// Same result as the decode kernel (memra-engine 0.98.0 dsv4_native_gemm_gate.rs page, `f64_ref`):
//   out[r, c] = sum_j ( sum_{k in group j} E4M3(A[r,k]) * E2M1(W[c,k]) ) * ws[c,j] * as[r, k/128]
// accumulated in f32; grouped over experts with a CSR offsets array (kernel_check.rs page, f16g
// grouped GEMM section).  Here the work is a dense contraction, so the kernel is built around the
// matrix cores.
//
// Arithmetic (bf16 MFMA 16x16x32, every operand exact):
//   A: E4M3 activation byte times its power-of-two row scale as[r, block], converted once per
//      workgroup into LDS with the hardware scaled conversion (the scale only moves the exponent,
//      so the bf16 value is exact).  Folding `as` into A removes any per-block partial sums.
//   B: NVFP4 nibble -> f32 (hardware FP4 conversion), times the E4M3 weight scale decoded to f32
//      (<= 6 significant bits: exact), packed to bf16 (exact); MXFP4 nibble -> bf16 with the E8M0
//      scale applied by the hardware conversion (a pure exponent: exact).  scale2 multiplies the
//      final f32 sum (exact for power-of-two scale2, otherwise within one f32 rounding of the
//      per-group weight scale).  Products of these bf16 values are exact in f32.
//
// Tiling.  A workgroup of 4 wavefronts computes a 128-row x 256-column output tile of one expert:
// each wavefront owns 64 columns (4 MFMA column tiles) of all 128 rows (8 row tiles), 128 f32
// accumulators per lane.  Per 128-wide k block, each wavefront streams and dequantizes its own
// weights in registers (one 16-byte load per column tile per lane, a 2-block ring), while the bf16
// activation tile and the block's weight scales sit in a two-stage LDS ring shared by the 4
// wavefronts.  128-row tiles keep the padding of the skewed per-expert row counts small.
//
// Work list.  Tiles are (expert, 128-row slice, 256-column slice).  Each workgroup finds its tile by
// a prefix scan of ceil(rows_e / 128) over the device-side offsets (no workspace, no host read of
// the offsets); the grid is sized for the bound ceil(R / 128) + E row slices and surplus workgroups
// exit.  Consecutive workgroups share the row slice (activation reuse in L2); a column slice stays
// on one XCD across row slices (weight reuse in L2).
#include "device_common.h"
#include "kernels.h"

namespace fp4moe {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBM = 128;                     // rows per tile
constexpr int kMT = kBM / 16;                // 8 MFMA row tiles per wavefront
constexpr int kNT = 4;                       // 4 MFMA column tiles per wavefront
constexpr int kWaveCols = 16 * kNT;          // 64
constexpr int kBN = kWaves * kWaveCols;      // 256 columns per tile
constexpr int kARow = 128 * 2 + 16;          // bf16 activation row of one block, padded (272 B)
constexpr int kNV = 0;
constexpr int kMX = 1;

struct Stage {
  uint8_t a[kBM * kARow];                    // bf16 activations (as folded), [row][128 k]
  uint8_t s[kBN * 8];                        // weight-scale bytes of the block, [column][8 | 4]
};

struct ExpertView {
  const uint8_t* w;
  const uint8_t* s;
  float scale2;
  int kind;
};

__device__ __forceinline__ int act_row(const GemmArgs& p, int prow) {
  if (!p.row_ids) return prow;
  const int r = p.row_ids[prow];
  return (r >= 0 && r < p.a_rows) ? r : -2;
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ f32x4 mfma16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Per-thread staging of one block: 64 activation bytes of one row (half of the block), that row's
// activation scale, and the weight-scale bytes of one column.
struct StageRegs {
  u32x4 a[4];
  float as;
  uint32_t s0, s1;
};

struct Rsrc {
  rsrc_t w, s, a, as;
};

struct StageOffsets {
  uint32_t a, as, s;                         // block-0 offsets (or kOffNone)
};

template <int KIND>
__device__ __forceinline__ void stage_load(const Rsrc& r, const StageOffsets& o, int b, bool valid,
                                           int nblk, StageRegs& d) {
  const uint32_t ub = (uint32_t)b;
  const uint32_t a = valid ? o.a + ub * 128u : kOffNone;
#pragma unroll
  for (int j = 0; j < 4; ++j) d.a[j] = buf_load_x4(r.a, a + 16u * j);
  d.as = u2f(buf_load_u32(r.as, valid ? o.as + ub * 4u : kOffNone));
  if constexpr (KIND == kNV) {
    const uint32_t so = valid ? o.s + ub * 8u : kOffNone;
    d.s0 = buf_load_u32(r.s, so);
    d.s1 = buf_load_u32(r.s, so + 4u);
  } else {
    d.s0 = buf_load_u32(r.s, valid ? o.s + ub * 4u : kOffNone);
    d.s1 = 0u;
  }
  (void)nblk;
}

// Convert the staged activation bytes (with their power-of-two scale folded in) to bf16 and store
// them, with the weight-scale bytes, into an LDS stage.
template <int KIND>
__device__ __forceinline__ void stage_store(Stage& st, const StageRegs& d) {
  const int tid = threadIdx.x, row = tid >> 1, half = tid & 1;
  u32x4 out[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d.a[j][w], d.as, false);
      const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d.a[j][w], d.as, true);
      out[2 * j + (w >> 1)][2 * (w & 1)] = __builtin_bit_cast(uint32_t, lo);
      out[2 * j + (w >> 1)][2 * (w & 1) + 1] = __builtin_bit_cast(uint32_t, hi);
    }
  }
  u32x4* dst = reinterpret_cast<u32x4*>(st.a + row * kARow + half * 128);
#pragma unroll
  for (int q = 0; q < 8; ++q) dst[q] = out[q];
  uint32_t* sd = reinterpret_cast<uint32_t*>(st.s + tid * 8);
  sd[0] = d.s0;
  if constexpr (KIND == kNV) sd[1] = d.s1;
}

// Eight nibbles (k = 8 consecutive) of one column, dequantized to bf16.
template <int KIND>
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float sv) {
  if constexpr (KIND == kNV) {
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    return bf16x8{(__bf16)(p0[0] * sv), (__bf16)(p0[1] * sv), (__bf16)(p1[0] * sv), (__bf16)(p1[1] * sv),
                  (__bf16)(p2[0] * sv), (__bf16)(p2[1] * sv), (__bf16)(p3[0] * sv), (__bf16)(p3[1] * sv)};
  } else {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sv, 0);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sv, 1);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sv, 2);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sv, 3);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
}

template <int KIND>
__device__ __forceinline__ void compute_block(const Stage& st, int wave, const u32x4 (&wq)[kNT],
                                              f32x4 (&acc)[kMT][kNT]) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, g = lane >> 4;
  // Weight scales of this lane's two 16-groups (k = 32g .. 32g+31 of the block) per column tile.
  float sv[kNT][2];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int col = wave * kWaveCols + 16 * nt + c16;
    if constexpr (KIND == kNV) {
      const uint32_t pair = *reinterpret_cast<const uint16_t*>(st.s + col * 8 + 2 * g);
      sv[nt][0] = __builtin_amdgcn_cvt_f32_fp8((int)pair, 0);
      sv[nt][1] = __builtin_amdgcn_cvt_f32_fp8((int)pair, 1);
    } else {
      const uint32_t e8 = st.s[col * 8 + g];             // E8M0 byte of k = 32g .. +32
      sv[nt][0] = u2f(e8 << 23);
      sv[nt][1] = sv[nt][0];
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16x8 bf[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) bf[nt] = dequant8<KIND>(wq[nt][i], sv[nt][i >> 1]);
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(st.a + (16 * mt + c16) * kARow + 64 * g + 16 * i);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = mfma16x16x32_bf16(af, bf[nt], acc[mt][nt]);
    }
  }
}

// One 128 x 256 output tile: packed rows [m0, m0 + mrows) of expert `ex`, columns [n0, n0 + 256).
template <int KIND>
__device__ void run_tile(const GemmArgs& p, const ExpertView& ex, int m0, int mrows, int n0, Stage (&st)[2]) {
  const int tid = threadIdx.x, lane = tid & 63, c16 = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = p.k, nblk = k >> 7;
  constexpr int GS = (KIND == kNV) ? 16 : 32;

  Rsrc r;
  r.w = make_rsrc(ex.w, (uint32_t)p.n * (uint32_t)(k / 2));
  r.s = make_rsrc(ex.s, (uint32_t)p.n * (uint32_t)(k / GS));
  r.a = make_rsrc(p.a_codes, (uint32_t)p.a_rows * (uint32_t)k);
  r.as = make_rsrc(p.a_scales, (uint32_t)p.a_rows * (uint32_t)nblk * 4u);

  StageOffsets so;
  {
    const int row = tid >> 1, half = tid & 1;
    const int ar = row < mrows ? act_row(p, m0 + row) : -1;
    so.a = ar >= 0 ? (uint32_t)ar * (uint32_t)k + 64u * half : kOffNone;
    so.as = ar >= 0 ? (uint32_t)ar * (uint32_t)nblk * 4u : kOffNone;
    const int col = n0 + tid;
    so.s = col < p.n ? (uint32_t)col * (uint32_t)(k / GS) : kOffNone;
  }
  uint32_t wo[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int col = n0 + wave * kWaveCols + 16 * nt + c16;
    wo[nt] = col < p.n ? (uint32_t)col * (uint32_t)(k / 2) + 16u * g : kOffNone;
  }

  f32x4 acc[kMT][kNT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Prologue in the steady-state load order (weights of block b, staging of block b+1, weights of
  // block b+1), each group pinned in place (see the decode kernel for why).
  StageRegs sr;
  stage_load<KIND>(r, so, 0, true, nblk, sr);
  __builtin_amdgcn_sched_barrier(0);
  stage_store<KIND>(st[0], sr);
  u32x4 wq[2][kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) wq[0][nt] = buf_load_x4(r.w, wo[nt]);
  __builtin_amdgcn_sched_barrier(0);
  stage_load<KIND>(r, so, 1, 1 < nblk, nblk, sr);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) wq[1][nt] = buf_load_x4(r.w, 1 < nblk ? wo[nt] + 64u : kOffNone);
  __builtin_amdgcn_sched_barrier(0);

  for (int b = 0; b < nblk; b += 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int bb = b + j;
      if (bb < nblk) {
        lds_barrier();                       // stage bb&1 ready, stage (bb+1)&1 free
        stage_store<KIND>(st[(bb + 1) & 1], sr);
        stage_load<KIND>(r, so, bb + 2, bb + 2 < nblk, nblk, sr);
        __builtin_amdgcn_sched_barrier(0);
        compute_block<KIND>(st[bb & 1], wave, wq[j], acc);
        const int bn = bb + 2;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt)
          wq[j][nt] = buf_load_x4(r.w, bn < nblk ? wo[nt] + (uint32_t)bn * 64u : kOffNone);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  const float post = (KIND == kNV) ? ex.scale2 : 1.0f;
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 16 * mt + 4 * g + v;
      if (row < mrows) {
        const int prow = m0 + row;
        const bool bad = act_row(p, prow) < 0;
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          const int col = n0 + wave * kWaveCols + 16 * nt + c16;
          if (col < p.n) p.out[(size_t)prow * p.n + col] = bad ? __builtin_nanf("") : acc[mt][nt][v] * post;
        }
      }
    }
}

__global__ __launch_bounds__(kThreads, 1) void gemm_prefill_kernel(GemmArgs p, int ntn) {
  __shared__ Stage st[2];
  __shared__ int s_tile[3];
  const int L = blockIdx.x;
  const int t = L / ntn, nt = L % ntn;

  // Find row slice t: expert e owns ceil(rows_e / 128) consecutive slices.
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int E = p.offsets ? p.num_experts : 1;
    int base = 0, found_e = -1, found_m0 = 0, found_rows = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      int lo = 0, hi = 0;
      if (e < E) {
        if (p.offsets) {
          lo = min(max(p.offsets[e], 0), p.total_rows);
          hi = min(max(p.offsets[e + 1], lo), p.total_rows);
        } else {
          hi = p.total_rows;
        }
      }
      const int cnt = (hi - lo + kBM - 1) / kBM;
      int incl = cnt;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
      }
      const int total = __shfl(incl, 63, 64);
      const int excl = incl - cnt;
      if (t >= base + excl && t < base + incl) {
        found_e = e;
        found_m0 = lo + (t - base - excl) * kBM;
        found_rows = min(kBM, hi - found_m0);
      }
      base += total;
      if (t < base) break;
    }
    if (found_e >= 0) {
      s_tile[0] = found_e;
      s_tile[1] = found_m0;
      s_tile[2] = found_rows;
    }
    if (lane == 0 && t >= base) s_tile[0] = -1;
  }
  __syncthreads();
  const int e = s_tile[0];
  if (e < 0) return;
  const int m0 = s_tile[1], mrows = s_tile[2];
  ExpertView ex;
  if (p.offsets) {
    ex = ExpertView{reinterpret_cast<const uint8_t*>(p.w_ptrs[e]), reinterpret_cast<const uint8_t*>(p.s_ptrs[e]),
                    p.scale2s[e], p.kinds[e]};
  } else {
    ex = ExpertView{p.w, p.s, p.scale2, p.kind};
  }
  const int n0 = nt * kBN;
  if (ex.kind == kNV) {
    run_tile<kNV>(p, ex, m0, mrows, n0, st);
  } else if (ex.kind == kMX) {
    run_tile<kMX>(p, ex, m0, mrows, n0, st);
  } else {
    for (int i = threadIdx.x; i < mrows * kBN; i += kThreads) {
      const int rr = m0 + i / kBN, col = n0 + i % kBN;
      if (col < p.n) p.out[(size_t)rr * p.n + col] = __builtin_nanf("");
    }
  }
}

}  // namespace

hipError_t launch_gemm_prefill(const GemmArgs& a, hipStream_t stream) {
  const int ntn = (a.n + kBN - 1) / kBN;
  const int E = a.offsets ? a.num_experts : 1;
  const int64_t slices = ((int64_t)a.total_rows + kBM - 1) / kBM + E;
  const int64_t blocks = slices * ntn;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(gemm_prefill_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, ntn);
  return hipGetLastError();
}

}  // namespace fp4moe
