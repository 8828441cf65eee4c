// gemm_decode.hip -- FP8-activation x block-scaled FP4 expert GEMM for few rows per expert.
//
// What is computed (memra-engine 0.98.0 dsv4_native_gemm_gate.rs page, `f64_ref` / `ExpertRaw`):
//   out[r, c] = sum_j ( sum_{k in group j} E4M3(A[r,k]) * E2M1(W[c,k]) ) * ws[c,j] * as[r, k/128]
// accumulated in f32, with NVFP4 (E4M3 scale per 16, times scale2) or MXFP4 (E8M0 scale per 32)
// weights.  Grouped form: rows packed per expert with a CSR offsets array (kernel_check.rs page,
// f16g grouped GEMM section).
//
// Work decomposition.  A workgroup of 4 wavefronts owns 256 output columns of one expert (128 for
// launches with few rows in total: see launch_gemm_decode); each wavefront owns 64 (32) of them, 4 (2)
// MFMA column tiles, over the whole of k, for every row of a pass of up to 32 activation rows.  With decode-sized row counts a pass covers all rows, so every weight byte
// is read from HBM exactly once.
//
// Data movement (the path is HBM-bound; what costs is the number and geometry of load requests):
//   weights: each lane streams 16 bytes per column tile per 128-wide k block straight into a ring of
//     4 register slots (one per block of a 512-wide k chunk).  With swizzled planes
//     (fp4_weight_swizzle) a load instruction reads 1 KB of consecutive bytes, with the non-temporal
//     cache policy (each weight byte is read once per step), a slot is refilled as soon as its block
//     has been computed, and the weight scales skip the LDS (see run_pass).  With the plain planes a
//     load instruction covers 16 column rows x 64 contiguous bytes, and the ring is refilled two
//     blocks at a time so that both halves of a column's 128-byte line are requested together.
//   activation codes, activation scales and weight scales: staged per 512-wide k chunk through a
//     two-stage LDS ring shared by the 4 wavefronts, loaded as contiguous row pieces (512 bytes of
//     activation codes, 32 or 16 bytes of weight scales per column row).  One activation load serves
//     256 columns.  NVFP4 weight scales are transposed on the way in so that a lane reads the scale
//     pairs of its 4 blocks with one 8-byte LDS read.
//
// Inner step for one 128-wide k block, per lane (c16 = lane%16, g = lane/16):
//   NVFP4: f16 MFMA 16x16x32.  Nibbles -> f16 with the hardware FP4 conversion, times the E4M3
//     scale in f16 (exact); activation bytes -> f16 (exact).  MFMA i of the block pairs lane group g
//     with k = k0 + 32g + 8i .. +8, so the block's four MFMAs cover one activation-scale group and
//     accumulate a partial tile that is scaled by as[r, block] in one f32 FMA.  scale2 multiplies
//     the final sum (exact for power-of-two scale2; otherwise within one f32 rounding of the
//     per-group weight scale, inside the accuracy bound).
//   MXFP4: bf16 MFMA 16x16x32 with the same block structure.  Activation bytes -> bf16 (exact);
//     nibbles -> bf16 with the E8M0 scale applied by the conversion (a pure exponent: exact; bf16
//     because an E8M0 scale can leave the f16 range).  The block-scaled FP8 x FP4 MFMA is not used:
//     it aligns its products to the largest one and drops the low bits of the others before
//     summing (measured: 448 + 2^-6 -> 448), which breaks the f32-accumulation error bound.
//
// Workgroup order is XCD-aware when there are >= 8 experts: consecutive workgroup ids go to
// different XCDs, so ids are arranged such that all column tiles of one expert land on one XCD and
// the expert's activation rows are fetched into one L2 only.  XCD x serves experts x, x+8, x+16, ...
// and, with grouped offsets, takes those with more than 16 rows (two MFMA row tiles, the longer
// workgroups) first: the short ones then fill the end of the launch.  Each workgroup finds its expert
// with two wavefront ballots over the offsets of its XCD's experts (xcd_expert).
#include "device_common.h"
#include "kernels.h"

namespace fp4moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
// CT = MFMA column tiles per wavefront (a template parameter): 4 (64 columns per wavefront, 256 per
// workgroup) or 2 (128 per workgroup, twice the workgroups for launches with few rows).
template <int CT> constexpr int kTileNT = kWaves * 16 * CT;
constexpr int kRows = 32;                    // rows per pass (2 MFMA row tiles)
constexpr int kChunkK = 512;                 // k per LDS stage
constexpr int kBlk = kChunkK / 128;          // 4 blocks of 128 per stage = register ring depth
constexpr int kARow = kChunkK + 16;          // padded LDS row of activation codes (bank spread)
constexpr int kSCol = 40;                    // padded LDS column of one chunk's weight scales
constexpr int kNV = 0;
constexpr int kMX = 1;
constexpr int kSwizzled = 2;                 // kind flag: planes in the swizzled layout

template <int CT>
struct Stage {
  uint8_t a[kRows * kARow];                  // activation codes, [row][512 (+16 pad)]
  float as[kBlk * kRows];                    // activation scales, [block][row]
  uint8_t s[kTileNT<CT> * kSCol];            // weight scales, [column][chunk bytes (+pad)]
};

struct ExpertView {
  const uint8_t* w;
  const uint8_t* s;
  float scale2;
  int kind;
  int rb, re;                                // packed rows [rb, re)
};

// Activation row of packed row `prow`: row_ids[prow] (or prow), -2 when the entry is out of range.
__device__ __forceinline__ int act_row(const GemmArgs& p, int prow) {
  if (!p.row_ids) return prow;
  const int r = p.row_ids[prow];
  return (r >= 0 && r < p.a_rows) ? r : -2;
}

// Workgroup barrier that waits for this wavefront's LDS operations only (__syncthreads would also
// wait for every outstanding global load and drain the weight ring).  The memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Per-thread staging registers of one chunk, and their global byte offsets for chunk 0.  With
// swizzled weight planes (SWZ) the weight scales are not staged: each lane loads its own.
template <int KIND, int CT>
constexpr int kStagedScales = KIND == kNV ? CT / 2 : 1;

template <int KIND, int CT>
struct StageRegs {
  u32x4 a[4];                                 // activation codes: 4 x 16 bytes
  u32x4 s[kStagedScales<KIND, CT>];           // weight scales: 16 bytes per column half (NV) / column (MX)
  float as;                                   // one activation scale (threads < 128)
};

template <int KIND, int CT>
struct StageOffsets {
  uint32_t a[4];                              // row * k + 16 * part, or kOffNone
  uint32_t s[kStagedScales<KIND, CT>];        // column * k/gs + 16 * half, or kOffNone
  uint32_t as;                                // (row * nblk + blk) * 4, or kOffNone
};

struct Rsrc {
  rsrc_t w, s, a, as;
};

template <int KIND, bool SWZ, int CT>
__device__ __forceinline__ void stage_load(const Rsrc& r, const StageOffsets<KIND, CT>& o, int c, bool valid,
                                           StageRegs<KIND, CT>& d) {
  const uint32_t uc = (uint32_t)c;
#pragma unroll
  for (int j = 0; j < 4; ++j) d.a[j] = buf_load_x4(r.a, valid ? o.a[j] + uc * kChunkK : kOffNone);
  if constexpr (!SWZ) {
#pragma unroll
    for (int h = 0; h < kStagedScales<KIND, CT>; ++h)
      d.s[h] = buf_load_x4(r.s, valid ? o.s[h] + uc * (KIND == kNV ? 32u : 16u) : kOffNone);
  }
  d.as = u2f(buf_load_u32(r.as, valid ? o.as + uc * (uint32_t)(kBlk * 4) : kOffNone));
}

// Store one chunk's staged data into an LDS stage.
template <int KIND, bool SWZ, int CT>
__device__ __forceinline__ void stage_store(Stage<CT>& st, const StageRegs<KIND, CT>& d) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = tid + kThreads * j, row = q >> 5, part = q & 31;
    *reinterpret_cast<u32x4*>(st.a + row * kARow + part * 16) = d.a[j];
  }
  if (tid < kRows * kBlk) st.as[(tid & 3) * kRows + (tid >> 2)] = d.as;
  if constexpr (SWZ) {
    return;
  } else if constexpr (KIND == kNV) {
    // The thread holds 16 bytes of one column = blocks {2h, 2h+1} x 4 ushort scale pairs (lane
    // groups g = 0..3).  For each g, the two pairs become one dword at [col][8g + 4h], so the
    // reader lane (column, g) finds the pairs of blocks 0..3 in 8 contiguous bytes.
#pragma unroll
    for (int hh = 0; hh < kStagedScales<KIND, CT>; ++hh) {
      const int q = tid + kThreads * hh, col = q >> 1, h = q & 1;
      const u32x4 v = d.s[hh];
      uint32_t* base = reinterpret_cast<uint32_t*>(st.s + col * kSCol + 4 * h);
      base[0] = __builtin_amdgcn_perm(v[2], v[0], 0x05040100u);   // g0: lo16(v0) | lo16(v2) << 16
      base[2] = __builtin_amdgcn_perm(v[2], v[0], 0x07060302u);   // g1: hi16(v0) | hi16(v2) << 16
      base[4] = __builtin_amdgcn_perm(v[3], v[1], 0x05040100u);   // g2
      base[6] = __builtin_amdgcn_perm(v[3], v[1], 0x07060302u);   // g3
    }
  } else {
    // MXFP4: 16 bytes = blocks 0..3 x 4 lane groups, stored as is at [col][0..15].
    if (tid < kTileNT<CT>) {
      uint64_t* base = reinterpret_cast<uint64_t*>(st.s + tid * kSCol);
      base[0] = ((uint64_t)d.s[0][1] << 32) | d.s[0][0];
      base[1] = ((uint64_t)d.s[0][3] << 32) | d.s[0][2];
    }
  }
}

template <int MT, int CT>
__device__ __forceinline__ void compute_block_nv(const Stage<CT>& st, int bq, const u32x4 (&wq)[CT],
                                                 const uint32_t (&sc)[CT], f32x4 (&acc)[MT][CT]) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, g = lane >> 4;
  f32x4 part[MT][CT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) part[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 aq[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint8_t* ap = st.a + (16 * mt + c16) * kARow + bq * 128 + 32 * g;
    aq[mt][0] = *reinterpret_cast<const u32x4*>(ap);
    aq[mt][1] = *reinterpret_cast<const u32x4*>(ap + 16);
  }
  h16x2 ws[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) ws[ct] = e4m3x2_to_f16<false>(sc[ct]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h16x8 af[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      af[mt] = e4m3x8_to_f16(aq[mt][i >> 1][2 * (i & 1)], aq[mt][i >> 1][2 * (i & 1) + 1]);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const h16x8 bf = e2m1x8_scaled_f16(wq[ct][i], ws[ct][i >> 1]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) part[mt][ct] = mfma16x16x32_f16(af[mt], bf, part[mt][ct]);
    }
  }
  // The partial tile covers exactly one 128-wide activation-scale group: result row 4g+v of row
  // tile mt is scaled by as[16mt + 4g + v, block].
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const f32x4 as = *reinterpret_cast<const f32x4*>(st.as + bq * kRows + 16 * mt + 4 * g);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[mt][ct][v] = fmaf(part[mt][ct][v], as[v], acc[mt][ct][v]);
  }
}

// MXFP4 block: exact bf16 operands (E4M3 activation bytes -> bf16; nibbles -> bf16 with the E8M0
// scale applied by the conversion, a pure exponent) and the same per-block partial tile as NVFP4.
// bf16 rather than f16 because an E8M0 scale can lie outside the f16 range.
template <int MT, int CT>
__device__ __forceinline__ void compute_block_mx(const Stage<CT>& st, int bq, const uint32_t (&sb)[CT],
                                                 const u32x4 (&wq)[CT], f32x4 (&acc)[MT][CT]) {
  const int lane = threadIdx.x & 63, c16 = lane & 15, g = lane >> 4;
  f32x4 part[MT][CT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) part[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 aq[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint8_t* ap = st.a + (16 * mt + c16) * kARow + bq * 128 + 32 * g;
    aq[mt][0] = *reinterpret_cast<const u32x4*>(ap);
    aq[mt][1] = *reinterpret_cast<const u32x4*>(ap + 16);
  }
  // The lane's k = 32g .. +32 of the block is one MXFP4 group: its E8M0 byte sb[ct], used as the
  // exponent field of the conversion's scale operand.
  float sv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) sv[ct] = u2f((sb[ct] & 0xFFu) << 23);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16x8 af[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) af[mt] = e4m3x8_to_bf16(aq[mt][i >> 1][2 * (i & 1)], aq[mt][i >> 1][2 * (i & 1) + 1]);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const bf16x8 bf = e2m1x8_pow2_bf16(wq[ct][i], sv[ct]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) part[mt][ct] = mfma16x16x32_bf16(af[mt], bf, part[mt][ct]);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const f32x4 as = *reinterpret_cast<const f32x4*>(st.as + bq * kRows + 16 * mt + 4 * g);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[mt][ct][v] = fmaf(part[mt][ct][v], as[v], acc[mt][ct][v]);
  }
}

// Scale registers of one 4-block chunk for one lane and column tile, with swizzled planes: the
// NVFP4 scale pairs of blocks 0..3 (8 bytes) or the MXFP4 bytes of blocks 0..3 (4 bytes).
template <int KIND> struct ChunkScale { typedef uint2 T; };
template <> struct ChunkScale<kMX> { typedef uint32_t T; };

template <int KIND>
__device__ __forceinline__ typename ChunkScale<KIND>::T scale_load(rsrc_t r, uint32_t off) {
  if constexpr (KIND == kNV) return buf_load_x2(r, off);
  else return buf_load_u32(r, off);
}

// Weight-stream load: non-temporal for swizzled planes, whose 1 KB runs stream faster that way
// (measured: 357 us against 396 us for the grouped decode step); the plain layout's 16 half lines
// per instruction stream slower with it (451 us against 419 us), so they keep the default policy.
template <bool SWZ>
__device__ __forceinline__ u32x4 wload(rsrc_t r, uint32_t off) {
  if constexpr (SWZ) return buf_load_x4_nt(r, off);
  else return buf_load_x4(r, off);
}

// One pass over the packed rows [m0, mend) (at most 32) for the 256 columns starting at n0.
// SWZ: the expert's planes are in the swizzled layout (fp4_weight_swizzle): a weight load of the
// wavefront reads 1 KB of consecutive bytes, and each lane loads the weight scales of its pieces
// for a whole chunk directly into registers, one chunk ahead, instead of staging them in LDS.
template <int MT, int KIND, bool SWZ, int CT>
__device__ void run_pass(const GemmArgs& p, const ExpertView& ex, int n0, int m0, int mend, Stage<CT> (&st)[2]) {
  const int tid = threadIdx.x, lane = tid & 63, c16 = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = p.k, nblk = k >> 7;
  const int nch = (nblk + kBlk - 1) / kBlk;
  constexpr int GS = (KIND == kNV) ? 16 : 32;
  // Bytes of one block of one lane piece row in the weight plane, of one chunk in the scale plane.
  constexpr uint32_t kWB = SWZ ? 1024u : 64u;
  constexpr uint32_t kSQ = KIND == kNV ? 512u : 256u;

  Rsrc r;
  if constexpr (SWZ) {
    const uint32_t n16 = (uint32_t)(p.n + 15) >> 4;
    r.w = make_rsrc(ex.w, n16 * 16u * (uint32_t)(k / 2));
    r.s = make_rsrc(ex.s, n16 * (uint32_t)nch * kSQ);
  } else {
    r.w = make_rsrc(ex.w, (uint32_t)p.n * (uint32_t)(k / 2));
    r.s = make_rsrc(ex.s, (uint32_t)p.n * (uint32_t)(k / GS));
  }
  r.a = make_rsrc(p.a_codes, (uint32_t)p.a_rows * (uint32_t)k);
  r.as = make_rsrc(p.a_scales, (uint32_t)p.a_rows * (uint32_t)nblk * 4u);

  // Staging offsets for chunk 0.  Rows beyond the pass, and rows whose row_ids entry is invalid,
  // load zeros.  A partial last chunk reads zeros past k (the descriptors end at the planes' ends,
  // and every row's data beyond k belongs to the next row, so those lanes are also masked below by
  // the block check: blocks >= nblk are never computed).
  StageOffsets<KIND, CT> so;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = tid + kThreads * j, row = q >> 5, part = q & 31;
    const int prow = m0 + row;
    const int ar = (row < MT * 16 && prow < mend) ? act_row(p, prow) : -1;
    so.a[j] = ar >= 0 ? (uint32_t)ar * (uint32_t)k + 16u * part : kOffNone;
  }
  {
    const int row = tid >> 2, blk = tid & 3, prow = m0 + row;
    const int ar = (tid < kRows * kBlk && row < MT * 16 && prow < mend) ? act_row(p, prow) : -1;
    so.as = ar >= 0 ? ((uint32_t)ar * (uint32_t)nblk + blk) * 4u : kOffNone;
  }
  if constexpr (!SWZ) {
#pragma unroll
    for (int h = 0; h < kStagedScales<KIND, CT>; ++h) {
      const int q = tid + kThreads * h;
      const int col = KIND == kNV ? (q >> 1) : q, half = KIND == kNV ? (q & 1) : 0;
      so.s[h] = (col < kTileNT<CT> && n0 + col < p.n) ? (uint32_t)(n0 + col) * (uint32_t)(k / GS) + 16u * half
                                                      : kOffNone;
    }
  }
  // Weight stream offsets of this wavefront's 4 column tiles (and, swizzled, of their scales).
  uint32_t wo[CT], sco[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = n0 + wave * (16 * CT) + 16 * ct + c16;
    if constexpr (SWZ) {
      const uint32_t t = (uint32_t)col >> 4, piece = (uint32_t)(16 * g + c16);
      wo[ct] = col < p.n ? t * (uint32_t)nblk * 1024u + 16u * piece : kOffNone;
      sco[ct] = col < p.n ? t * (uint32_t)nch * kSQ + piece * (kSQ / 64u) : kOffNone;
    } else {
      wo[ct] = col < p.n ? (uint32_t)col * (uint32_t)(k / 2) + 16u * g : kOffNone;
      sco[ct] = kOffNone;
    }
  }

  f32x4 acc[MT][CT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Prologue: chunk 0 staged into LDS stage 0, chunk 1 loaded into the staging registers, then the
  // weight ring for the blocks of chunk 0 with (swizzled) the weight scales of chunk 0 after block 0's
  // weights -- the same order of outstanding loads as at the top of every loop iteration (staged
  // chunk first, then weights and scales in refill order), so that the compiler's wait counts,
  // merged over the loop entry and the back edge, stay exact.  Every group of loads is pinned where it is written
  // (sched_barrier): the machine scheduler would otherwise sink loads toward their first use.  All
  // loads are issued on every path (out-of-range ones return zero without touching memory).
  StageRegs<KIND, CT> sr;
  stage_load<KIND, SWZ, CT>(r, so, 0, true, sr);
  __builtin_amdgcn_sched_barrier(0);
  stage_store<KIND, SWZ, CT>(st[0], sr);
  stage_load<KIND, SWZ, CT>(r, so, 1, 1 < nch, sr);
  __builtin_amdgcn_sched_barrier(0);
  typename ChunkScale<KIND>::T scn[CT], scc[CT];   // next chunk's / this chunk's scales (SWZ)
  u32x4 wq[kBlk][CT];
  if constexpr (SWZ) {
    // the steady-state order: block 0's weights, the chunk's scales, blocks 1..3
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) wq[0][ct] = wload<SWZ>(r.w, wo[ct]);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) scn[ct] = scale_load<KIND>(r.s, sco[ct]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 1; j < kBlk; ++j) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) wq[j][ct] = wload<SWZ>(r.w, j < nblk ? wo[ct] + (uint32_t)j * kWB : kOffNone);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else
#pragma unroll
  for (int j = 0; j < kBlk; j += 2) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      wq[j][ct] = wload<SWZ>(r.w, j < nblk ? wo[ct] + (uint32_t)j * kWB : kOffNone);
      wq[j + 1][ct] = wload<SWZ>(r.w, j + 1 < nblk ? wo[ct] + (uint32_t)(j + 1) * kWB : kOffNone);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  for (int c = 0; c < nch; ++c) {
    lds_barrier();                           // stage c&1 complete; stage (c+1)&1 no longer read
    stage_store<KIND, SWZ, CT>(st[(c + 1) & 1], sr);  // chunk c+1 (zeros past the end)
    stage_load<KIND, SWZ, CT>(r, so, c + 2, c + 2 < nch, sr);
    __builtin_amdgcn_sched_barrier(0);
    const Stage<CT>& cur = st[c & 1];
    uint2 scp[CT];                          // NVFP4 scale pairs of blocks 0..3 of this chunk
    uint32_t mxs[CT];                       // MXFP4 scale bytes of blocks 0..3 of this chunk
    if constexpr (SWZ) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        scc[ct] = scn[ct];
        if constexpr (KIND == kNV) scp[ct] = scc[ct];
        else mxs[ct] = scc[ct];
      }
    } else if constexpr (KIND == kNV) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        scp[ct] = *reinterpret_cast<const uint2*>(cur.s + (wave * (16 * CT) + 16 * ct + c16) * kSCol + 8 * g);
    }
#pragma unroll
    for (int bq = 0; bq < kBlk; ++bq) {
      const int b = c * kBlk + bq;
      if (b < nblk) {
        if constexpr (KIND == kNV) {
          uint32_t sc[CT];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) sc[ct] = (bq < 2 ? scp[ct].x : scp[ct].y) >> (16 * (bq & 1));
          compute_block_nv<MT, CT>(cur, bq, wq[bq], sc, acc);
        } else {
          uint32_t sb[CT];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            sb[ct] = SWZ ? mxs[ct] >> (8 * bq)
                         : (uint32_t)cur.s[(wave * (16 * CT) + 16 * ct + c16) * kSCol + 4 * bq + g];
          compute_block_mx<MT, CT>(cur, bq, sb, wq[bq], acc);
        }
      }
      if constexpr (SWZ) {
        // Swizzled: every slot is refilled as soon as its block is computed (1 KB runs: no line
        // halves to pair; measured 335 us against 341 us for the grouped decode step, same bits);
        // the next chunk's scales follow the first refill.
        const int bn = b + kBlk;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          wq[bq][ct] = wload<SWZ>(r.w, bn < nblk ? wo[ct] + (uint32_t)bn * kWB : kOffNone);
        if (bq == 0) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
            scn[ct] = scale_load<KIND>(r.s, c + 1 < nch ? sco[ct] + (uint32_t)(c + 1) * kSQ : kOffNone);
        }
      } else if (bq & 1) {
        // Plain planes: refill two blocks at a time, so that the two 64-byte halves of each
        // column's 128-byte line are requested back to back and the line is fetched from HBM once.
        const int bn = b + kBlk;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          wq[bq - 1][ct] = wload<SWZ>(r.w, bn - 1 < nblk ? wo[ct] + (uint32_t)(bn - 1) * kWB : kOffNone);
          wq[bq][ct] = wload<SWZ>(r.w, bn < nblk ? wo[ct] + (uint32_t)bn * kWB : kOffNone);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Store: the lane holds column (16ct + c16) and rows 4g+v of each row tile.  Non-temporal: the
  // output is not read again by this launch, and keeping it out of the caches leaves them to the
  // activation rows (measured: 346 us against 357 us for the grouped decode step).
  const float post = (KIND == kNV) ? ex.scale2 : 1.0f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int prow = m0 + 16 * mt + 4 * g + v;
      if (prow < mend) {
        const bool bad = act_row(p, prow) < 0;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int col = n0 + wave * (16 * CT) + 16 * ct + c16;
          if (col < p.n)
            __builtin_nontemporal_store(bad ? __builtin_nanf("") : acc[mt][ct][v] * post, &p.out[(size_t)prow * p.n + col]);
        }
      }
    }
}

template <int KIND, bool SWZ, int CT>
__device__ void run_expert(const GemmArgs& p, const ExpertView& ex, int n0, Stage<CT> (&st)[2]) {
  for (int m0 = ex.rb; m0 < ex.re; m0 += kRows) {
    const int mend = min(m0 + kRows, ex.re);
    if (m0 > ex.rb) lds_barrier();           // the previous pass may still be reading the stages
    if (mend - m0 > 16) run_pass<2, KIND, SWZ, CT>(p, ex, n0, m0, mend, st);
    else run_pass<1, KIND, SWZ, CT>(p, ex, n0, m0, mend, st);
  }
}

// Position gi of the order in which XCD x takes its experts x, x+8, x+16, ... (grouped offsets, at
// most 512 experts): those with more than 16 rows first, each class in expert order.  Returns the
// expert, or num_experts past the end of the XCD's list.  Lane j looks at the XCD's j-th expert;
// every lane of the wavefront takes part (ballots), and the result is uniform.
__device__ __forceinline__ int xcd_expert(const GemmArgs& p, int x, int gi) {
  const int lane = threadIdx.x & 63;
  const int nj = (p.num_experts - x + 7) >> 3;
  bool big = false;
  if (lane < nj) {
    const int e = 8 * lane + x;
    const int lo = min(max(p.offsets[e], 0), p.total_rows);
    const int hi = min(max(p.offsets[e + 1], lo), p.total_rows);
    big = hi - lo > 16;
  }
  const uint64_t mbig = __builtin_amdgcn_ballot_w64(big);
  const uint64_t valid = nj >= 64 ? ~0ull : (1ull << nj) - 1;
  const uint64_t below = (1ull << lane) - 1;
  const int pos = big ? __popcll(mbig & below) : __popcll(mbig) + __popcll(valid & ~mbig & below);
  const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < nj && pos == gi);
  return hit ? 8 * (__ffsll((long long)hit) - 1) + x : p.num_experts;
}

template <int CT>
__global__ __launch_bounds__(kThreads, 2) void gemm_decode_kernel(GemmArgs p, int ntn, int xcd_map) {
  constexpr int kTileN = kTileNT<CT>;
  __shared__ Stage<CT> st[2];
  const int L = blockIdx.x;
  int e, nt;
  if (xcd_map) {
    const int idx = L >> 3;
    e = (idx / ntn) * 8 + (L & 7);
    nt = idx % ntn;
    // measured on the 512-token step over 256 experts: 1.3-2.1% faster than the plain order
    if (p.offsets && p.num_experts <= 512) e = __builtin_amdgcn_readfirstlane(xcd_expert(p, L & 7, idx / ntn));
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
  // kinds 0/1: plain planes; 2/3: the same formats in the swizzled layout
  if (ex.kind == kNV) {
    run_expert<kNV, false, CT>(p, ex, n0, st);
  } else if (ex.kind == kMX) {
    run_expert<kMX, false, CT>(p, ex, n0, st);
  } else if (ex.kind == (kNV | kSwizzled)) {
    run_expert<kNV, true, CT>(p, ex, n0, st);
  } else if (ex.kind == (kMX | kSwizzled)) {
    run_expert<kMX, true, CT>(p, ex, n0, st);
  } else {
    for (int i = threadIdx.x; i < (ex.re - ex.rb) * kTileN; i += kThreads) {
      const int r = ex.rb + i / kTileN, col = n0 + i % kTileN;
      if (col < p.n) p.out[(size_t)r * p.n + col] = __builtin_nanf("");
    }
  }
}

}  // namespace

#ifndef FP4MOE_DECODE_NARROW_ROWS
#define FP4MOE_DECODE_NARROW_ROWS 1024
#endif

// Launches with few packed rows in total (a decode step of up to 128 tokens at top-8) leave most
// experts with a few rows: 128-column workgroups (twice as many, three per compute unit) stream
// their weights faster (over the 256 experts of k = 7168, n = 2048: 4 tokens 59.6 us against 66.4,
// 64 tokens 275 against 285, 128 tokens 303 against 307); the full 512-token step (4096 rows) is
// faster with 256 columns per workgroup (358 us against 367).
hipError_t launch_gemm_decode(const GemmArgs& a, hipStream_t stream) {
  const bool narrow = a.total_rows <= FP4MOE_DECODE_NARROW_ROWS;
  const int tile_n = narrow ? kTileNT<2> : kTileNT<4>;
  const int ntn = (a.n + tile_n - 1) / tile_n;
  const int xcd_map = a.num_experts >= 8 ? 1 : 0;
  const int64_t eg = xcd_map ? (int64_t)(a.num_experts + 7) / 8 * 8 : a.num_experts;
  const int64_t blocks = eg * ntn;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (narrow)
    hipLaunchKernelGGL(gemm_decode_kernel<2>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, ntn, xcd_map);
  else
    hipLaunchKernelGGL(gemm_decode_kernel<4>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, ntn, xcd_map);
  return hipGetLastError();
}

}  // namespace fp4moe
