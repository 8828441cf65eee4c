// kernels.h -- internal launch interface between the C ABI (capi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4moe {

// One GEMM problem in the layout of fp4moe.h.  Single expert: offsets == nullptr, the planes are
// w/s/kind/scale2 and the rows are 0 .. total_rows-1 (row_ids == nullptr).  Grouped: the planes
// come from the device tables w_ptrs/s_ptrs/kinds/scale2s indexed by expert.
struct GemmArgs {
  const uint8_t* a_codes;
  const float* a_scales;
  const int32_t* row_ids;     // nullable
  int32_t a_rows;
  const int32_t* offsets;     // [num_experts + 1] or nullptr
  int32_t num_experts;
  int32_t total_rows;
  const uint64_t* w_ptrs;
  const uint64_t* s_ptrs;
  const int32_t* kinds;
  const float* scale2s;
  const uint8_t* w;
  const uint8_t* s;
  float scale2;
  int32_t kind;
  float* out;
  int32_t n;
  int32_t k;
  // W4A4 activations (tiled kernel only): a_codes are E2M1 nibbles [a_rows, k/2] with UE4M3
  // micro-scales a_micro [a_rows, k/16] and row scales a_row_scale [a_rows]; a_scales is unused.
  const uint8_t* a_micro;
  const float* a_row_scale;
  // Gate/up projection fused with the expert activation and its FP8 quantization (tiled kernel
  // only; swiglu_inter > 0): columns [0, inter) are the gate, [inter, 2 inter) the up projection,
  // and instead of `out` the kernel writes h_codes [rows, inter], h_scales [rows, inter/128] and, when
  // given, h_out [rows, inter] for h = swiglu(gate, up, swiglu_limit) * swiglu_row_w[row].
  int32_t swiglu_inter;
  float swiglu_limit;
  const float* swiglu_row_w;
  uint8_t* h_codes;
  float* h_scales;
  float* h_out;
};

hipError_t launch_act_quant(const float* x, uint8_t* codes, float* scales, int64_t ngroups,
                            hipStream_t stream);

// The expert activation (swiglu with limit, optional row weight) fused with the FP8 quantization
// of its result; inter % 128 == 0.
hipError_t launch_swiglu_quant(const float* gu, const float* weights, float limit, uint8_t* codes,
                               float* scales, float* h_out, int64_t rows, int32_t inter,
                               hipStream_t stream);

// Routing (route.hip): top-k with softmax weights (experts <= 1024, top_k <= 64); packing of the
// routed pairs per expert with a workspace of route_pack_workspace_elems int32; the row gather
// (16-byte aligned codes); the combine of expert outputs in token order.
hipError_t launch_route_topk(const float* logits, int32_t tokens, int32_t experts, int32_t top_k,
                             int32_t normalize, int32_t* ids, float* weights, hipStream_t stream);
int64_t route_pack_workspace_elems(int32_t tokens, int32_t experts);
hipError_t launch_route_pack(const int32_t* ids, const float* w, int32_t tokens, int32_t top_k,
                             int32_t experts, int32_t* offsets, int32_t* row_ids, int32_t* pair_rows,
                             float* row_w, int32_t* workspace, hipStream_t stream);
hipError_t launch_gather_rows(const uint8_t* codes, const float* scales, int32_t a_rows, int32_t k,
                              const int32_t* row_ids, int32_t rows, uint8_t* out_codes, float* out_scales,
                              hipStream_t stream);
hipError_t launch_combine(const float* y, int32_t y_rows, int32_t n, const int32_t* pair_rows,
                          const float* w, int32_t tokens, int32_t top_k, float* out, hipStream_t stream);

// The bf16-dequant rung (rung.hip): f32 -> bf16, FP4 weights -> bf16 (k % 128 == 0), and a plain
// bf16 GEMM out = a * w^T with f32 accumulation (k % 16 == 0).
hipError_t launch_cvt_bf16(const float* x, uint16_t* out, int64_t count, hipStream_t stream);
hipError_t launch_dequant_bf16(const uint8_t* w, const uint8_t* s, float scale2, int32_t kind, int32_t n,
                               int32_t k, uint16_t* out, hipStream_t stream);
hipError_t launch_gemm_bf16(const uint16_t* a, const uint16_t* w, float* out, int32_t m, int32_t n, int32_t k,
                            hipStream_t stream);

// The W4A4 NVFP4 variant (w4a4.hip): the two-level E2M1 activation quantizer (k % 128 == 0, at most
// 64 kept-out channels), the loudest-channel selection (k <= 8192, one block), and the exact addition
// of the kept channels after the GEMM (the GEMM itself is launch_gemm_prefill with a_micro set).
hipError_t launch_act_quant_fp4(const float* x, const int32_t* skip, int32_t n_skip, int32_t rows, int32_t k,
                                int32_t two_level, uint8_t* codes, uint8_t* micro, float* row_scale,
                                hipStream_t stream);
hipError_t launch_loud_channels(const float* x, int32_t rows, int32_t k, int32_t k_res, int32_t* idx,
                                hipStream_t stream);
hipError_t launch_w4a4_residual(const float* x, const int32_t* res_idx, int32_t k_res, const uint8_t* w,
                                const uint8_t* s, float scale2, float* out, int32_t g, int32_t n, int32_t k,
                                hipStream_t stream);

// The swizzled weight layout (swizzle.hip): plane sizes and the reordering of one expert's planes
// (kind 0 NVFP4 / 1 MXFP4; w, w_out and s_out 16-byte aligned).
int64_t swizzled_weight_bytes(int32_t n, int32_t k);
int64_t swizzled_scale_bytes(int32_t kind, int32_t n, int32_t k);
hipError_t launch_weight_swizzle(const uint8_t* w, const uint8_t* s, int32_t kind, int32_t n, int32_t k,
                                 uint8_t* w_out, uint8_t* s_out, hipStream_t stream);

// Row-streaming kernel for few rows per expert (decode): every expert's weights are read once per
// pass of 32 rows.
hipError_t launch_gemm_decode(const GemmArgs& a, hipStream_t stream);

// Split-k kernel for very few rows: 16-column tiles whose 4, 8 or 16 (single expert, from k) or 8, 4, 2 or 1
// (grouped, picked per launch) wavefronts split k.  Single expert
// (offsets == nullptr): requires gemm_skinny_fits(g, n, k) (g <= 16, k <= 8192).  Grouped: requires
// gemm_skinny_grouped_fits (at most 16 packed rows, 128 when the schedule is forced; k <= 8192;
// at most 1024 experts).
bool gemm_skinny_fits(int32_t g, int32_t n, int32_t k);
bool gemm_skinny_grouped_fits(int64_t total_rows, int32_t num_experts, int32_t n, int32_t k, bool forced);
hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream);

// Tiled matrix-core kernel for many rows per expert (prefill): 128 x 256 output tiles.
hipError_t launch_gemm_prefill(const GemmArgs& a, hipStream_t stream);

// Validation of a grouped call's tables (table_check.hip), one workgroup: status[i] (int32,
// kTableCheckWords of them) receives the smallest index violating condition i, or -1:
// 0 offsets[0] != 0; 1 offsets[e+1] < offsets[e]; 2 offsets[E] != total_rows; 3 row_ids[p] outside
// [0, a_rows) (row_ids may be null); 4 kinds[e] outside 0..3.
constexpr int kTableCheckWords = 5;
hipError_t launch_table_check(const int32_t* offsets, int32_t num_experts, int32_t total_rows, const int32_t* row_ids,
                              int32_t a_rows, const int32_t* kinds, int32_t* status, hipStream_t stream);

}  // namespace fp4moe
