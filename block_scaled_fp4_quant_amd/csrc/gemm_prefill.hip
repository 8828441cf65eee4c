// gemm_prefill.hip -- FP8-activation x block-scaled FP4 expert GEMM for many rows per expert.
//
// Same result as the decode kernel (memra-engine 0.98.0 dsv4_native_gemm_gate.rs page, `f64_ref`):
//   out[r, c] = sum_j ( sum_{k in group j} E4M3(A[r,k]) * E2M1(W[c,k]) ) * ws[c,j] * as[r, k/128]
// accumulated in f32; grouped over experts with a CSR offsets array (kernel_check.rs page, f16g
// grouped GEMM section).  Here the work is a dense contraction, so the kernel is built around the
// matrix cores.
//
// Arithmetic (f16 or bf16 MFMA 32x32x16, every operand exact):
//   A: E4M3 activation byte times its power-of-two row scale as[r, block], converted once per
//      workgroup into LDS with the hardware scaled conversion (the scale only moves the exponent,
//      so the value is exact).  Folding `as` into A removes any per-block partial sums.
//   B (NVFP4, f16 route): nibble -> f16 (hardware FP4 conversion), times the E4M3 weight scale as
//      f16 with packed multiplies (at most 5 significant bits: exact).  Half the conversion work of
//      the bf16 route.  f16 holds E4M3 x 2^t exactly for 2^-15 <= 2^t <= 2^7, so a tile takes this
//      route only when every activation block scale of its rows lies there (real activations:
//      2^-9 .. 2^3); otherwise:
//   B (NVFP4, bf16 route): nibble -> f32, times the E4M3 weight scale in f32, packed to bf16.
//   Either way scale2 multiplies the final f32 sum (exact for power-of-two scale2, otherwise within
//   one f32 rounding of the per-group weight scale); products of the operands are exact in f32.
//   MXFP4: nibble -> bf16 with the E8M0 scale applied by the hardware conversion (a pure exponent:
//      exact).  The block-scaled FP8 x FP4 MFMA is not used: it aligns its products to the largest
//      one before summing and drops the low bits of the others (measured: 448 + 2^-6 -> 448), which
//      breaks the f32-accumulation error bound; the bf16 and f16 MFMAs sum exactly.
//   On gfx950 the 32x32x16 and 16x16x32 bf16 MFMAs issue at the same rate (about 32 cycles), so
//   the 32x32 shape does twice the work per instruction.
//
// Tiling.  A workgroup of 4 wavefronts computes a 128-row x 256-column output tile of one expert:
// each wavefront owns 64 columns (2 MFMA column tiles of 32) of all 128 rows (4 row tiles), 128 f32
// accumulators per lane.  Per 128-wide k block (8 steps of 16), each wavefront streams and
// dequantizes its own weights in registers (a 2-block ring of 32 nibble bytes + scale bytes per
// column tile per lane), while the bf16 activation tile sits in a two-stage LDS ring shared by the
// 4 wavefronts.  Inside a block the steps are software-pipelined: the MFMAs of step s run while
// the weight dequantization of step s+1 is issued and each row tile's A fragment for step s+1 is
// read from LDS right after that row tile's MFMAs, and the conversion of the next block's
// activations into the other LDS stage is spread over the first steps, one 32-row group per step;
// the steps are fenced from one another for the instruction scheduler.  One barrier per block.  Two
// workgroups share a compute unit (256 registers per lane, 139 KB of LDS), so each SIMD interleaves
// two independent wavefronts.  On the f16 route an expert's last row slice computes only its
// occupied 32-row MFMA tiles (32, 64 or 96 rows), which keeps the padding of the skewed per-expert
// row counts small; the bf16 route computes whole slices.
// Activations are staged with 8 lanes per row, so each 16-byte load instruction touches 8 cache
// lines.
//
// Vector instruction budget.  A block costs each wavefront 128 weight conversions and scale
// multiplies whatever the tile's row count, so a short tile issues many vector instructions per MFMA
// and the loop keeps the rest small: only the occupied row groups of the activations are loaded and
// converted; a load past the last block gets its out-of-range offset from one scalar per block
// (kBlkNone) instead of a per-lane select; one packed conversion yields two weight group scales; and
// the LDS stage layout spreads the staging stores over the banks without data selects (stage_store_q).
// Measured together on the prefill workload: 2.6% faster (3485 us against 3576 us; the down-projection
// shape 1934 against 1991 us), identical bits; the step fence adds 0.5-1% on both shapes.
//
// Epilogue.  The accumulators go through LDS (over the activation stages), 64 rows at a time, so that
// each thread writes 16 consecutive bytes of one output row with a non-temporal store; rows whose
// activation scale or row id is invalid were flagged by the scale scan before the main loop and are
// written as NaN.  The fused activation epilogue (swiglu_inter > 0) has its own exchange through LDS.
//
// Work list.  Tiles are (expert, 128-row slice, 256-column slice).  Each workgroup finds its tile by
// a prefix scan of ceil(rows_e / 128) over the device-side offsets (no workspace, no host read of
// the offsets); the grid is sized for the bound ceil(R / 128) + E row slices and surplus workgroups
// exit.  Consecutive workgroups share the row slice (activation reuse in L2); with a multiple of 8
// column slices, a column slice stays on one XCD across row slices (weight reuse in that L2).
#include "device_common.h"
#include "kernels.h"

namespace fp4moe {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBM = 128;                     // rows per tile
static_assert(kThreads == 2 * kBM, "the f16 operand check gives each row two threads");
constexpr int kMT = kBM / 32;                // 4 MFMA row tiles (32 rows) per wavefront
constexpr int kNT = 2;                       // 2 MFMA column tiles (32 columns) per wavefront
constexpr int kWaveCols = 32 * kNT;          // 64
constexpr int kBN = kWaves * kWaveCols;      // 256 columns per tile
constexpr int kSteps = 8;                    // 16-wide k steps per 128-wide block
constexpr int kARow = 128 * 2 + 16;          // bf16 activation row of one block, padded (272 B)
// Block offset of a load past the last block: every plane is smaller than 2^31 bytes, so a valid
// lane's offset plus this is out of range (the load returns zeros) without wrapping past 2^32.
constexpr uint32_t kBlkNone = 0x80000000u;
constexpr int kWDepth = 2;                   // register sets in the weight load ring
constexpr int kADepth = 1;                   // register sets in the activation load ring
constexpr int kUnroll = 2;                   // blocks per loop iteration (a multiple of both depths and of the 2 LDS stages)
constexpr int kNV = 0;
constexpr int kMX = 1;
constexpr int kNV16 = 2;                     // NVFP4 on f16 operands (tiles whose activation scales allow it)
constexpr int kW4 = 3;                       // NVFP4 weights x W4A4 activations (E2M1 x UE4M3), f16 operands
constexpr int kSwizzled = 2;                 // flag in an expert's kind: planes in the swizzled layout

__host__ __device__ constexpr bool is_nv(int kind) { return kind != kMX; }

// Operand type of the MFMAs: bf16, or f16 for kNV16.
template <int KIND> struct OpT { typedef bf16x8 T; };
template <> struct OpT<kNV16> { typedef h16x8 T; };
template <> struct OpT<kW4> { typedef h16x8 T; };

struct Stage {
  uint8_t a[kBM * kARow];                    // bf16 activations (as folded), [row][128 k]
};

struct ExpertView {
  const uint8_t* w;
  const uint8_t* s;
  float scale2;
  int kind;
};

// Per (tile row, thread half): the row uses an activation scale that is not a positive normal power
// of two (set by scan_act_scales before the main loop, read by the epilogues).
__shared__ uint8_t s_rowbad[kThreads];

__device__ __forceinline__ int act_row(const GemmArgs& p, int prow) {
  if (!p.row_ids) return prow;
  const int r = p.row_ids[prow];
  return (r >= 0 && r < p.a_rows) ? r : -2;
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 32x32x16 bf16 MFMA.  Lane l holds A row l%32 (B column l%32) for k = 8*(l/32) .. +8; the f32
// result holds column l%32, rows 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(h16x8 a, h16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// The k order inside a 128-wide block.  Both operands use the same order, so the sum is the same
// set of products: lane half h = l/32 covers k = 64h .. 64h+63, and step s takes k = 64h + 8s .. +8.
// For the weights that is nibble bytes 32h + 4s .. +4 of the column's 64-byte block, i.e. dword s%4
// of the 16-byte chunk s/4 of the lane's 32 bytes; its NVFP4 group is 4h + s/2 (byte s/2 of the
// lane's 4 scale bytes), its MXFP4 group 2h + s/4 (byte s/4 of the lane's 2 scale bytes).

// Per-thread staging of one block.  Eight lanes cover one row's 128 block bytes (one cache line), so
// a 16-byte load instruction touches 8 lines: thread t holds bytes 16*(t%8) .. +16 of rows
// t/8 + 32*i (i = 0..3) and those rows' activation scales.
struct StageRegs {
  u32x4 a[4];
  float as[4];
};

// Per-thread block-0 offsets of the staged rows (kOffNone for rows past the tile or invalid).
struct AOffs {
  uint32_t a[4], as[4];
};

// Weights of one block for one lane: 32 nibble bytes per column tile and its scale bytes.
struct WRegs {
  u32x4 w[kNT][2];
  uint32_t s[kNT];
};

struct Rsrc {
  rsrc_t w, s, a, as;
};

// The activations of block b for the NMT occupied row groups (32 rows each) of the tile.  Past the
// last block the offsets move out of range by kBlkNone, so the loads return zeros.  A lane whose row
// is outside the slice or has an invalid row id (offset kOffNone) may wrap back into the plane and
// load bytes of another row: those rows are never stored, or are stored as NaN from the scan's flags.
template <int KIND, int NMT>
__device__ __forceinline__ void stage_load(const Rsrc& r, const AOffs& o, int b, int nblk, StageRegs& d) {
  const bool valid = b < nblk;
  if constexpr (KIND == kW4) {
    // W4A4: 8 nibble bytes (16 elements, one micro-scale group) and that group's micro-scale byte
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
      const uint2 v = buf_load_x2(r.a, valid && o.a[i] != kOffNone ? o.a[i] + (uint32_t)b * 64u : kOffNone);
      d.a[i] = u32x4{v.x, v.y, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < NMT; ++i)
      d.as[i] = u2f(buf_load_u8(r.as, valid && o.as[i] != kOffNone ? o.as[i] + (uint32_t)b * 8u : kOffNone));
    return;
  }
  const uint32_t sa = valid ? (uint32_t)b * 128u : kBlkNone, ss = valid ? (uint32_t)b * 4u : kBlkNone;
#pragma unroll
  for (int i = 0; i < NMT; ++i) d.a[i] = buf_load_x4(r.a, o.a[i] + sa);
#pragma unroll
  for (int i = 0; i < NMT; ++i) d.as[i] = u2f(buf_load_u32(r.as, o.as[i] + ss));
}

// SWZ: planes in the swizzled layout (fp4_weight_swizzle).  The lane's 32 bytes are then the lane
// pieces 2h and 2h+1 of its column (256 bytes apart), and their scale bytes sit in those pieces'
// rows of the 4-block chunk: (b/4) * chunk bytes + (b%4) * bytes per block, the second piece 16 rows
// further.  wo/so are the block-0 offsets of piece 2h.
template <bool SWZ>
__device__ __forceinline__ void w_load_first(const Rsrc& r, const uint32_t (&wo)[kNT], int b, int nblk, WRegs& d);
template <int KIND, bool SWZ>
__device__ __forceinline__ void w_load_second(const Rsrc& r, const uint32_t (&wo)[kNT], const uint32_t (&so)[kNT],
                                              int b, int nblk, WRegs& d);
template <int KIND, bool SWZ>
__device__ __forceinline__ void w_load(const Rsrc& r, const uint32_t (&wo)[kNT], const uint32_t (&so)[kNT],
                                       int b, int nblk, WRegs& d) {
  w_load_first<SWZ>(r, wo, b, nblk, d);
  w_load_second<KIND, SWZ>(r, wo, so, b, nblk, d);
}

// The two halves of w_load: the first 16 nibble bytes of each column tile (steps 0-3), then the
// second 16 bytes and the scale bytes (steps 4-7 and every step).  As in stage_load, past the last
// block the offsets move out of range by kBlkNone; a lane past the last column (offset kOffNone) may
// wrap into the plane, and its column is never stored.
template <bool SWZ>
__device__ __forceinline__ void w_load_first(const Rsrc& r, const uint32_t (&wo)[kNT], int b, int nblk, WRegs& d) {
  const uint32_t sb = b < nblk ? (uint32_t)b * (SWZ ? 1024u : 64u) : kBlkNone;
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) d.w[nt][0] = buf_load_x4(r.w, wo[nt] + sb);
}

template <int KIND, bool SWZ>
__device__ __forceinline__ void w_load_second(const Rsrc& r, const uint32_t (&wo)[kNT], const uint32_t (&so)[kNT],
                                              int b, int nblk, WRegs& d) {
  const bool valid = b < nblk;
  const uint32_t sb = valid ? (uint32_t)b * (SWZ ? 1024u : 64u) : kBlkNone;
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) d.w[nt][1] = buf_load_x4(r.w, wo[nt] + sb + (SWZ ? 256u : 16u));
  const uint32_t ub = (uint32_t)b;
  const uint32_t ss = !valid ? kBlkNone
                      : SWZ ? (is_nv(KIND) ? (ub >> 2) * 512u + (ub & 3u) * 2u : (ub >> 2) * 256u + (ub & 3u))
                            : ub * (is_nv(KIND) ? 8u : 4u);
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const uint32_t o = so[nt] + ss;
    if constexpr (SWZ) {
      if constexpr (is_nv(KIND)) d.s[nt] = buf_load_u16(r.s, o) | (buf_load_u16(r.s, o + 128u) << 16);
      else d.s[nt] = buf_load_u8(r.s, o) | (buf_load_u8(r.s, o + 64u) << 8);
    } else if constexpr (is_nv(KIND)) {
      d.s[nt] = buf_load_u32(r.s, o);
    } else {
      d.s[nt] = buf_load_u16(r.s, o);
    }
  }
}

// Row i of the staged rows (16 activation bytes): converted to bf16 (f16 for kNV16) with the
// power-of-two row scale folded in (exact: the scale only moves the exponent, and kNV16 tiles keep
// every scaled value inside f16's exact range) and written to the LDS stage.  The two 16-byte halves
// are written in an order that puts the 8 lanes of a row on distinct banks.
template <int KIND>
__device__ __forceinline__ void stage_store_q(Stage& st, const StageRegs& d, int i) {
  const int tid = threadIdx.x, c = tid & 7, row = (tid >> 3) + 32 * i;
  if constexpr (KIND == kW4) {
    // 16 E2M1 values times their UE4M3 micro-scale as f16 (at most 5 significant bits: exact)
    const _Float16 ms = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)f2u(d.as[i]), 0);
    const bool swap = (c >> 2) & 1;                         // the layout below (pair-swapped upper half)
    const h16x8 first = e2m1x8_scaled_f16(d.a[i][0], ms);
    const h16x8 second = e2m1x8_scaled_f16(d.a[i][1], ms);
    uint8_t* dst = st.a + row * kARow + 32 * c;
    *reinterpret_cast<h16x8*>(dst + (swap ? 16 : 0)) = first;
    *reinterpret_cast<h16x8*>(dst + (swap ? 0 : 16)) = second;
    return;
  }
  // The upper half of a row (lanes c >= 4, k 64..127) holds each 32-byte piece pair with its two
  // 16-byte halves swapped: the first store of every lane then goes to +0 (c < 4) or +16 (c >= 4),
  // which spreads one store instruction over the banks, with no data selects; lds_a reads the upper
  // half's pieces at the swapped positions.
  const bool swap = (c >> 2) & 1;
  const uint32_t src[4] = {d.a[i][0], d.a[i][1], d.a[i][2], d.a[i][3]};
  u32x4 first, second;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t p0, p1;
    if constexpr (KIND == kNV16) {
      p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src[w], d.as[i], false));
      p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(src[w], d.as[i], true));
    } else {
      p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[w], d.as[i], false));
      p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src[w], d.as[i], true));
    }
    if (w < 2) {
      first[2 * w] = p0;
      first[2 * w + 1] = p1;
    } else {
      second[2 * (w - 2)] = p0;
      second[2 * (w - 2) + 1] = p1;
    }
  }
  uint8_t* dst = st.a + row * kARow + 32 * c;
  *reinterpret_cast<u32x4*>(dst + (swap ? 16 : 0)) = first;
  *reinterpret_cast<u32x4*>(dst + (swap ? 0 : 16)) = second;
}

// Eight nibbles (k = 8 of one column) of step s, dequantized to bf16.
template <int KIND, int S>
__device__ __forceinline__ typename OpT<KIND>::T dequant_step(const WRegs& w, int nt) {
  const uint32_t q = w.w[nt][S >> 2][S & 3];
  if constexpr (KIND == kNV16 || KIND == kW4) {
    // E2M1 -> f16 (exact), times the E4M3 group scale as f16 (exact; at most 5 significant bits).
    // One packed conversion yields the scales of two groups (bytes 0-1 for steps 0-3, 2-3 after).
    const h16x2 sp = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.s[nt], 1.0f, S >= 4);
    return e2m1x8_scaled_f16(q, sp[(S >> 1) & 1]);
  } else if constexpr (KIND == kNV) {
    // E2M1 -> f32 (exact), times the E4M3 group scale (<= 6 significant bits: exact), -> bf16 (exact)
    const float sv = __builtin_amdgcn_cvt_f32_fp8((int)w.s[nt], S >> 1);
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
    const bf16x2 b0 = {(__bf16)(p0[0] * sv), (__bf16)(p0[1] * sv)};
    const bf16x2 b1 = {(__bf16)(p1[0] * sv), (__bf16)(p1[1] * sv)};
    const bf16x2 b2 = {(__bf16)(p2[0] * sv), (__bf16)(p2[1] * sv)};
    const bf16x2 b3 = {(__bf16)(p3[0] * sv), (__bf16)(p3[1] * sv)};
    return bf16x8{b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
  } else {
    // The E8M0 byte is the exponent field of the scale operand (the conversion applies only it).
    const float sv = u2f(((w.s[nt] >> (8 * (S >> 2))) & 0xFFu) << 23);
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sv, 0);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sv, 1);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sv, 2);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, sv, 3);
    return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
}

template <int KIND>
__device__ __forceinline__ typename OpT<KIND>::T lds_a(const Stage& st, int mt, int s) {
  const int lane = threadIdx.x & 63;
  // lane half h reads k 64h + 8s .. +8, i.e. 16-byte piece 8h + s of the row; the upper half
  // (h = 1) stores its pieces pair-swapped (stage_store_q), so piece 8 + s sits at 8 + (s ^ 1)
  const int h = lane >> 5;
  const int hoff = (s & 1) ? 112 * h : 144 * h;
  return *reinterpret_cast<const typename OpT<KIND>::T*>(st.a + (32 * mt + (lane & 31)) * kARow + hoff + 16 * s);
}

// Fragments of the step the MFMAs consume next.
template <int KIND>
struct Frags {
  typename OpT<KIND>::T a[kMT];
  typename OpT<KIND>::T b[kNT];
};

// One 128-wide k block.  Step s issues its MFMAs while the operands of step s+1 are prepared: 2
// weight dequantizations, and each row tile's A fragment, read from LDS into the same registers
// right after that row tile's MFMAs (no second set of A registers).  Steps 0-3 also convert and
// store the next block's activations, steps 3 and 7 refill the weight slot with the block after next
// (its first 16 bytes per column tile, then the rest), step 4 issues the activation loads of the
// block after, and before step 7 the workgroup meets at the barrier that publishes the next stage.
// Step 7 prepares step 0 of the next block.
template <int KIND, int NMT, bool SWZ>
__device__ __forceinline__ void run_block(const Stage& cur, Stage& nxt, const WRegs& w, const WRegs& wn,
                                          StageRegs& store_src, StageRegs& load_dst, const Rsrc& r,
                                          const AOffs& ao, int b, int nblk, WRegs& wload,
                                          const uint32_t (&wo)[kNT], const uint32_t (&so)[kNT], Frags<KIND>& f,
                                          f32x16 (&acc)[kMT][kNT]) {
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    Frags<KIND> g;
    if (s == kSteps - 1) {
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();                         // next stage complete; this stage fully read
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      switch (s) {
        case 0: g.b[nt] = dequant_step<KIND, 1>(w, nt); break;
        case 1: g.b[nt] = dequant_step<KIND, 2>(w, nt); break;
        case 2: g.b[nt] = dequant_step<KIND, 3>(w, nt); break;
        case 3: g.b[nt] = dequant_step<KIND, 4>(w, nt); break;
        case 4: g.b[nt] = dequant_step<KIND, 5>(w, nt); break;
        case 5: g.b[nt] = dequant_step<KIND, 6>(w, nt); break;
        case 6: g.b[nt] = dequant_step<KIND, 7>(w, nt); break;
        default: g.b[nt] = dequant_step<KIND, 0>(wn, nt); break;
      }
    }
    if (s < NMT) stage_store_q<KIND>(nxt, store_src, s);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = mfma32x32x16(f.a[mt], f.b[nt], acc[mt][nt]);
      f.a[mt] = (s + 1 < kSteps) ? lds_a<KIND>(cur, mt, s + 1) : lds_a<KIND>(nxt, mt, 0);
    }
    if (s == 3) {
      // the first 16 bytes of the slot were last read by step 3's dequantization (issued at s = 2)
      __builtin_amdgcn_sched_barrier(0);
      w_load_first<SWZ>(r, wo, b + kWDepth, nblk, wload);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (s == 4) {
      __builtin_amdgcn_sched_barrier(0);
      stage_load<KIND, NMT>(r, ao, b + 1 + kADepth, nblk, load_dst);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (s == kSteps - 1) {
      __builtin_amdgcn_sched_barrier(0);
      w_load_second<KIND, SWZ>(r, wo, so, b + kWDepth, nblk, wload);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) f.b[nt] = g.b[nt];
    // Keep the steps apart: interleaving one step's MFMAs with the next step's puts each A
    // fragment read right before its first use (measured 0.5-1% slower on both GEMM shapes).
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Fused with the activation (swiglu_inter > 0), a tile covers the h columns [n0, n0 + 128), n0 = 128 q:
// wavefront w computes gate columns n0 + 32 w .. +31 in its first MFMA column tile and the matching
// up columns inter + n0 + 32 w .. +31 in its second, so that every lane holds each gate value next to
// its up value.  Otherwise wavefront w computes columns n0 + 64 w .. +63.
__device__ __forceinline__ int tile_col(const GemmArgs& p, int n0, int wave, int nt) {
  return p.swiglu_inter ? (nt ? p.swiglu_inter : 0) + n0 + 32 * wave : n0 + kWaveCols * wave + 32 * nt;
}

// The fused activation epilogue of one tile (gate/up projection -> h = swiglu -> FP8 codes of h).  The
// tile's 128 h columns of a row are exactly one act-quant group.  swiglu multiplies by the row weight
// last, so every lane first forms t = swiglu with weight 1 from its gate/up pairs and stores t in LDS
// (over the activation stages, which the main loop no longer needs), letting the accumulators die as
// they are consumed.  Two threads then take a row, 64 values each: h = t * w, the row's amax (the
// halves exchange theirs through LDS) and the codes, written as contiguous 16-byte stores.  f32
// rounding is monotone, so max |t * w| = max |t| * |w| exactly; with the unfused route's operations
// in its order everywhere else, codes, scales and h are bit-identical to the grouped GEMM followed by
// swiglu_quant_fp8.  A packed row whose activation row is invalid gets what the unfused route gives
// the grouped GEMM's NaN output: the activation of NaN gate and up values, in every column.
constexpr int kHPitch = 128 + 4;                           // floats per row of the t exchange
template <int NMT, bool ROWCHECK>
__device__ __forceinline__ void swiglu_epilogue(const GemmArgs& p, int m0, int mrows, int n0, float post,
                                                f32x16 (&acc)[kMT][kNT], Stage (&st)[2]) {
  static_assert(kNT == 2 && kWaves == 4, "a wavefront holds 32 gate and 32 up columns");
  static_assert(kThreads == 2 * kBM, "two threads quantize each row");
  static_assert(sizeof(Stage) * 2 >= (kBM * kHPitch + 2 * kBM) * sizeof(float), "exchange space");
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int inter = p.swiglu_inter;
  const float limit = p.swiglu_limit;
  float* tx = reinterpret_cast<float*>(&st[0]);            // [128 rows][kHPitch] t
  float* hmax = tx + kBM * kHPitch;                        // [2 halves][128 rows] max |t|
  __syncthreads();                                         // every wavefront is done with the stages
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 32 * mt + 8 * (v >> 2) + 4 * h + (v & 3);
      tx[row * kHPitch + 32 * wave + c32] = swiglu_one(acc[mt][0][v] * post, acc[mt][1][v] * post, limit, 1.0f);
    }
  __syncthreads();
  const int row = tid & (kBM - 1), half = tid / kBM;
  f32x4 t[16];
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    t[j] = *reinterpret_cast<const f32x4*>(tx + row * kHPitch + 64 * half + 4 * j);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(t[j][0]), fabsf(t[j][1])), fmaxf(fabsf(t[j][2]), fabsf(t[j][3]))));
  }
  hmax[half * kBM + row] = m;
  __syncthreads();
  if (row < mrows) {
    const int prow = m0 + row;
    const float w = p.swiglu_row_w ? p.swiglu_row_w[prow] : 1.0f;
    // FP8 activations: the scale scan flagged the row (bad scale or row id); otherwise look the row up
    const bool bad = ROWCHECK ? (s_rowbad[2 * row] | s_rowbad[2 * row + 1]) != 0 : act_row(p, prow) < 0;
    const float hbad = swiglu_one(__builtin_nanf(""), __builtin_nanf(""), limit, w);
    const float tmax = fmaxf(hmax[row], hmax[kBM + row]);
    const float amax = fmaxf(bad ? fabsf(hbad) : tmax * fabsf(w), 1e-4f);
    const float sc = pow2_ceil_pos(amax * u2f(0x3B124925u));   // 1/448 rounded once to f32
    const float rcp = pow2_recip(sc);                      // h * rcp == h / sc exactly (sc = 2^e)
    const size_t at = (size_t)prow * inter + n0 + 64 * half;
    uint32_t packed[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      f32x4 hv;
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = bad ? hbad : t[j][e] * w;
      const float a0 = fminf(fmaxf(hv[0] * rcp, -448.f), 448.f);
      const float a1 = fminf(fmaxf(hv[1] * rcp, -448.f), 448.f);
      const float a2 = fminf(fmaxf(hv[2] * rcp, -448.f), 448.f);
      const float a3 = fminf(fmaxf(hv[3] * rcp, -448.f), 448.f);
      const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
      packed[j] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, pk, true);
      if (p.h_out) *reinterpret_cast<f32x4*>(p.h_out + at + 4 * j) = hv;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      reinterpret_cast<u32x4*>(p.h_codes + at)[j] =
          u32x4{packed[4 * j], packed[4 * j + 1], packed[4 * j + 2], packed[4 * j + 3]};
    if (half == 0) p.h_scales[(size_t)prow * (inter / 128) + n0 / 128] = sc;
  }
}

// One 128 x 256 output tile: packed rows [m0, m0 + mrows) of expert `ex`, columns [n0, n0 + 256)
// (fused with the activation: the gate and up columns of the h columns [n0, n0 + 128)).
template <int KIND, int NMT, bool SWZ>
__device__ __forceinline__ void run_tile(const GemmArgs& p, const ExpertView& ex, int m0, int mrows, int n0, Stage (&st)[2]) {
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = p.k, nblk = k >> 7;
  constexpr int GS = is_nv(KIND) ? 16 : 32;
  const uint32_t n16 = (uint32_t)(p.n + 15) >> 4, nq = (uint32_t)(nblk + 3) >> 2;

  Rsrc r;
  if constexpr (SWZ) {
    r.w = make_rsrc(ex.w, n16 * 16u * (uint32_t)(k / 2));
    r.s = make_rsrc(ex.s, n16 * nq * (is_nv(KIND) ? 512u : 256u));
  } else {
    r.w = make_rsrc(ex.w, (uint32_t)p.n * (uint32_t)(k / 2));
    r.s = make_rsrc(ex.s, (uint32_t)p.n * (uint32_t)(k / GS));
  }
  if constexpr (KIND == kW4) {
    r.a = make_rsrc(p.a_codes, (uint32_t)p.a_rows * (uint32_t)(k / 2));
    r.as = make_rsrc(p.a_micro, (uint32_t)p.a_rows * (uint32_t)(k / 16));
  } else {
    r.a = make_rsrc(p.a_codes, (uint32_t)p.a_rows * (uint32_t)k);
    r.as = make_rsrc(p.a_scales, (uint32_t)p.a_rows * (uint32_t)nblk * 4u);
  }

  AOffs ao;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = (tid >> 3) + 32 * i;
    const int ar = row < mrows ? act_row(p, m0 + row) : -1;
    if constexpr (KIND == kW4) {
      ao.a[i] = ar >= 0 ? (uint32_t)ar * (uint32_t)(k / 2) + 8u * (tid & 7) : kOffNone;
      ao.as[i] = ar >= 0 ? (uint32_t)ar * (uint32_t)(k / 16) + (uint32_t)(tid & 7) : kOffNone;
    } else {
      ao.a[i] = ar >= 0 ? (uint32_t)ar * (uint32_t)k + 16u * (tid & 7) : kOffNone;
      ao.as[i] = ar >= 0 ? (uint32_t)ar * (uint32_t)nblk * 4u : kOffNone;
    }
  }
  uint32_t wo[kNT], so[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int col = tile_col(p, n0, wave, nt) + c32;
    if constexpr (SWZ) {
      const uint32_t t = (uint32_t)col >> 4, piece = 32u * h + ((uint32_t)col & 15u);   // lane piece 2h
      wo[nt] = col < p.n ? t * (uint32_t)nblk * 1024u + 16u * piece : kOffNone;
      so[nt] = col < p.n ? t * nq * (is_nv(KIND) ? 512u : 256u) + piece * (is_nv(KIND) ? 8u : 4u) : kOffNone;
    } else {
      wo[nt] = col < p.n ? (uint32_t)col * (uint32_t)(k / 2) + 32u * h : kOffNone;
      so[nt] = col < p.n ? (uint32_t)col * (uint32_t)(k / GS) + (is_nv(KIND) ? 4u : 2u) * h : kOffNone;
    }
  }

  f32x16 acc[kMT][kNT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][nt][v] = 0.f;

  // Prologue, in the steady-state load order (block b loads the activations of block b+1+kADepth,
  // then the weights of block b+kWDepth).  Loads past the last block return zeros.
  StageRegs sr[kADepth];
  WRegs wr[kWDepth];
  stage_load<KIND, NMT>(r, ao, 0, nblk, sr[0]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 1; j < kADepth; ++j) {
    stage_load<KIND, NMT>(r, ao, j, nblk, sr[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j + 1 < kWDepth; ++j) {
    w_load<KIND, SWZ>(r, wo, so, j, nblk, wr[j]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int q = 0; q < NMT; ++q) stage_store_q<KIND>(st[0], sr[0], q);
  __builtin_amdgcn_sched_barrier(0);
  w_load_first<SWZ>(r, wo, kWDepth - 1, nblk, wr[kWDepth - 1]);
  __builtin_amdgcn_sched_barrier(0);
  stage_load<KIND, NMT>(r, ao, kADepth, nblk, sr[0]);
  __builtin_amdgcn_sched_barrier(0);
  w_load_second<KIND, SWZ>(r, wo, so, kWDepth - 1, nblk, wr[kWDepth - 1]);
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();
  Frags<KIND> f;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) f.a[mt] = lds_a<KIND>(st[0], mt, 0);
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) f.b[nt] = dequant_step<KIND, 0>(wr[0], nt);

  // Block b reads LDS stage b&1 and weights wr[b%kWDepth]; it stores block b+1 (staged in
  // sr[(b+1)%kADepth]) into the other LDS stage, refills those staging registers with block
  // b+1+kADepth, and refills wr[b%kWDepth] with block b+kWDepth: the first 16 bytes of each column
  // tile at step 3 (dead after step 3's dequantization), the rest at its end.  A block count that is
  // not a multiple of kUnroll runs up to kUnroll-1 all-zero blocks.
  const int nblk_r = (nblk + kUnroll - 1) / kUnroll * kUnroll;
  for (int b = 0; b < nblk_r; b += kUnroll) {
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int ja = (j + 1) % kADepth;
      run_block<KIND, NMT, SWZ>(st[j & 1], st[(j + 1) & 1], wr[j % kWDepth], wr[(j + 1) % kWDepth], sr[ja], sr[ja], r, ao,
                      b + j, nblk, wr[j % kWDepth], wo, so, f, acc);
    }
  }

  const float post = is_nv(KIND) ? ex.scale2 : 1.0f;
  if (p.swiglu_inter) {
    swiglu_epilogue<NMT, KIND != kW4>(p, m0, mrows, n0, post, acc, st);
  } else if (KIND == kW4) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 32 * mt + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row < mrows) {
          const int prow = m0 + row;
          const int arow = act_row(p, prow);             // W4A4 tiles skip the scale scan
          const bool bad = arow < 0;
          const float rsc = bad ? 1.0f : p.a_row_scale[arow];
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) {
            const int col = tile_col(p, n0, wave, nt) + c32;
            if (col < p.n) p.out[(size_t)prow * p.n + col] = bad ? __builtin_nanf("") : acc[mt][nt][v] * (post * rsc);
          }
        }
      }
  } else {
    // Row-contiguous stores: the accumulators go through LDS (over the activation stages, 64 rows
    // per pass), so that each lane then writes 16 consecutive output bytes of one row (a quarter of
    // the store instructions of the accumulator layout, whose lanes hold columns).  Non-temporal:
    // the output is not read again by this launch.
    constexpr int kPitch = kBN + 4;                          // floats per LDS row
    static_assert(sizeof(Stage) * 2 >= 64 * kPitch * sizeof(float), "transpose space");
    float* tx = reinterpret_cast<float*>(&st[0]);
    __syncthreads();                                         // every wavefront is done with the stages
#pragma unroll
    for (int pass = 0; pass < (NMT + 1) / 2; ++pass) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int mt = 2 * pass + q;
        if (mt < NMT) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int rl = 32 * q + 8 * (v >> 2) + 4 * h + (v & 3), row = 64 * pass + rl;
            const bool bad = (s_rowbad[2 * row] | s_rowbad[2 * row + 1]) != 0;
#pragma unroll
            for (int nt = 0; nt < kNT; ++nt)
              tx[rl * kPitch + kWaveCols * wave + 32 * nt + c32] = bad ? __builtin_nanf("") : acc[mt][nt][v] * post;
          }
        }
      }
      __syncthreads();
      {
        // thread t stores columns 4 (t % 64) .. +3 of rows t / 64, t / 64 + 4, ... of the pass
        constexpr int kRowsPerStep = kThreads / (kBN / 4);
        const int c4 = threadIdx.x % (kBN / 4), r0 = threadIdx.x / (kBN / 4), col = n0 + 4 * c4;
        float* dst = p.out + (size_t)(m0 + 64 * pass + r0) * p.n + col;
        const size_t step = (size_t)kRowsPerStep * p.n;
        const float* src = tx + r0 * kPitch + 4 * c4;
        // 16-byte stores need 16-byte aligned rows: n % 4 == 0 and an aligned output base
        const bool vec = ((p.n & 3) | (int)(reinterpret_cast<uintptr_t>(p.out) & 15)) == 0;
#pragma unroll 4
        for (int rl = r0; rl < 64; rl += kRowsPerStep) {
          if (64 * pass + rl < mrows && col < p.n) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(src);
            if (vec) {
              __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (col + e < p.n) __builtin_nontemporal_store(v[e], dst + e);
            }
          }
          dst += step;
          src += kRowsPerStep * kPitch;
        }
      }
      __syncthreads();
    }
  }
}

// The scan of a tile's activation scales before its main loop (FP8 activations only).
// - The activation scale is folded into the A operand by the hardware scaled conversion, which
//   applies only the exponent of its f32 scale: that is exact for the positive normal powers of two
//   that act_quant_fp8 writes, and wrong for anything else.  A row that uses any other value in any
//   128-wide block gets s_rowbad[2 row] | s_rowbad[2 row + 1] set, and the epilogue writes it as NaN.
// - f16 holds E4M3 x 2^t exactly for every code when 2^-15 <= 2^t <= 2^7 (the smallest code step
//   2^-9 stays >= f16's 2^-24, and 448 x 2^7 < 65504).  The return value says whether the scale of
//   every 128-wide activation block of the tile's rows lies in that range (or is 0: rows not loaded),
//   i.e. whether the tile may take the f16 route.  Real activations have block scales of 2^-9 .. 2^3;
//   all-zero or tiny blocks fall back to bf16.
__device__ __forceinline__ bool scan_act_scales(const GemmArgs& p, int m0, int mrows) {
  // two threads per row (kThreads = 2 x kBM): thread half h reads blocks 8j + 4h .. +4 with 16-byte
  // loads, all issued before the first test (past the row's end the buffer reads 0, which passes)
  const int nblk = p.k >> 7, row = threadIdx.x >> 1, h = threadIdx.x & 1;
  const int ar = row < mrows ? act_row(p, m0 + row) : -1;
  const rsrc_t r = make_rsrc(p.a_scales, (uint32_t)p.a_rows * (uint32_t)nblk * 4u);
  const uint32_t base = ar >= 0 ? (uint32_t)ar * (uint32_t)nblk * 4u : kOffNone;
  bool ok = true, bad = false;
  for (int b0 = 4 * h; b0 < nblk; b0 += 32) {
    f32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = b0 + 8 * j;
      v[j] = __builtin_bit_cast(f32x4, buf_load_x4(r, base != kOffNone && b < nblk ? base + 4u * b : kOffNone));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // blocks past the row's end read the next row's scales: harmless for the f16 test (it only
        // gets stricter); the power-of-two test skips them
        const float x = v[j][e];
        ok &= x == 0.0f || (x >= 0x1p-15f && x <= 128.0f);
        const uint32_t bits = f2u(x), ex = bits >> 23;
        const bool pow2 = (bits & 0x807FFFFFu) == 0u && ex >= 1u && ex <= 254u;
        bad |= base != kOffNone && b0 + 8 * j + e < nblk && !pow2;
      }
  }
  bad |= row < mrows && ar < 0;               // an out-of-range row_ids entry: the row is NaN too
  s_rowbad[threadIdx.x] = bad ? 1 : 0;
  return __builtin_amdgcn_readfirstlane(__syncthreads_and(ok)) != 0;
}

// A tile whose weight format the kernel does not take: NaN outputs (fused with the activation: the
// activation of NaN gate and up values).
__device__ __forceinline__ void nan_tile(const GemmArgs& p, int m0, int mrows, int n0, Stage (&st)[2]) {
  if (p.swiglu_inter) {
    f32x16 nacc[kMT][kNT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int v = 0; v < 16; ++v) nacc[mt][nt][v] = __builtin_nanf("");
    swiglu_epilogue<kMT, false>(p, m0, mrows, n0, 1.0f, nacc, st);
    return;
  }
  for (int i = threadIdx.x; i < mrows * kBN; i += kThreads) {
    const int rr = m0 + i / kBN, col = n0 + i % kBN;
    if (col < p.n) p.out[(size_t)rr * p.n + col] = __builtin_nanf("");
  }
}

// NVFP4 on f16 operands: only the occupied 32-row MFMA tiles of the slice are computed.
template <bool SWZ>
__device__ __forceinline__ void run_tile_nv16(const GemmArgs& p, const ExpertView& ex, int m0, int mrows, int nmt,
                                              int n0, Stage (&st)[2]) {
  if (nmt == 1) {
    run_tile<kNV16, 1, SWZ>(p, ex, m0, mrows, n0, st);
  } else if (nmt == 2) {
    run_tile<kNV16, 2, SWZ>(p, ex, m0, mrows, n0, st);
  } else if (nmt == 3) {
    run_tile<kNV16, 3, SWZ>(p, ex, m0, mrows, n0, st);
  } else {
    run_tile<kNV16, 4, SWZ>(p, ex, m0, mrows, n0, st);
  }
}

__global__ __launch_bounds__(kThreads, 2) void gemm_prefill_kernel(GemmArgs p, int ntn) {
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
  // The tile is the same for the whole workgroup: keep it (and everything derived from it, such as
  // the buffer descriptors) in scalar registers.
  const int e = __builtin_amdgcn_readfirstlane(s_tile[0]);
  if (e < 0) return;
  const int m0 = __builtin_amdgcn_readfirstlane(s_tile[1]), mrows = __builtin_amdgcn_readfirstlane(s_tile[2]);
  ExpertView ex;
  if (p.offsets) {
    ex = ExpertView{reinterpret_cast<const uint8_t*>(p.w_ptrs[e]), reinterpret_cast<const uint8_t*>(p.s_ptrs[e]),
                    p.scale2s[e], p.kinds[e]};
  } else {
    ex = ExpertView{p.w, p.s, p.scale2, p.kind};
  }
  const int n0 = nt * (p.swiglu_inter ? 128 : kBN);
  // The last slice of an expert may hold fewer than 128 rows: only its occupied 32-row MFMA tiles
  // are computed.
  const int nmt = (mrows + 31) >> 5;
  // kinds 0/1: plain planes; 2/3: the same formats in the swizzled layout
  const bool swz = ex.kind == (kNV | kSwizzled) || ex.kind == (kMX | kSwizzled);
  const int base_kind = swz ? ex.kind & ~kSwizzled : ex.kind;
  if (p.a_micro) {
    // W4A4 activations: always exact in f16; plain NVFP4 weights only (other kinds give NaN below)
    if (ex.kind == kNV) {
      if (nmt == 1) {
        run_tile<kW4, 1, false>(p, ex, m0, mrows, n0, st);
      } else if (nmt == 2) {
        run_tile<kW4, 2, false>(p, ex, m0, mrows, n0, st);
      } else if (nmt == 3) {
        run_tile<kW4, 3, false>(p, ex, m0, mrows, n0, st);
      } else {
        run_tile<kW4, 4, false>(p, ex, m0, mrows, n0, st);
      }
    } else {
      nan_tile(p, m0, mrows, n0, st);
    }
  } else if (base_kind == kNV || base_kind == kMX) {
    const bool f16_ok = scan_act_scales(p, m0, mrows);
    if (base_kind == kMX) {
      if (swz) run_tile<kMX, 4, true>(p, ex, m0, mrows, n0, st);
      else run_tile<kMX, 4, false>(p, ex, m0, mrows, n0, st);
    } else if (f16_ok) {
      if (swz) run_tile_nv16<true>(p, ex, m0, mrows, nmt, n0, st);
      else run_tile_nv16<false>(p, ex, m0, mrows, nmt, n0, st);
    } else {
      if (swz) run_tile<kNV, 4, true>(p, ex, m0, mrows, n0, st);
      else run_tile<kNV, 4, false>(p, ex, m0, mrows, n0, st);
    }
  } else {
    nan_tile(p, m0, mrows, n0, st);
  }
}

}  // namespace

hipError_t launch_gemm_prefill(const GemmArgs& a, hipStream_t stream) {
  const int ntn = a.swiglu_inter ? a.swiglu_inter / 128 : (a.n + kBN - 1) / kBN;
  const int E = a.offsets ? a.num_experts : 1;
  const int64_t slices = ((int64_t)a.total_rows + kBM - 1) / kBM + E;
  const int64_t blocks = slices * ntn;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(gemm_prefill_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, ntn);
  return hipGetLastError();
}

}  // namespace fp4moe
