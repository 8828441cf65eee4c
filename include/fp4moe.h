/*
 * fp4moe.h -- C ABI of libfp4moe: FP8 E4M3 activation quantization and the block-scaled FP4
 * (NVFP4 / MXFP4) expert GEMM, for AMD Instinct MI355X (gfx950).
 *
 * Sources the operations are defined by (cited by page title and item):
 *   [GATE]  memra-engine 0.98.0, src/bin/dsv4_native_gemm_gate.rs: `quant_rows` (act-quant), the
 *           `ExpertRaw` layout, `f64_ref` (the quantized GEMM), comparison 2 (error model), and the
 *           FFI calls of the act-quant and FP4 GEMM kernels in `main` (pointer/size/stream
 *           convention, return code 0 = success, kind 0 = NVFP4 / 1 = MXFP4).
 *   [CHECK] memra-engine 0.71.0, src/bin/kernel_check.rs: f16g grouped GEMM section (rows packed
 *           per expert with a CSR offsets array) and the direct-from-quant section (a per-expert
 *           table of weight addresses).
 *   [GATE]  also: the swiglu_limit saturation cell (the clamp math between the gate/up and the down
 *           projection, and its swiglu call with an optional per-row weight).
 *   [CHECK] also: the NVFP4 MMQ W4A4 arms (E2M1 activations with a per-token row scale and a UE4M3
 *           micro-scale per 16; the sub-block-only quantizer; the DYNAMIC-RANGE and RESIDUAL-CHANNEL
 *           arms).
 *   [QWEN]  memra-engine 0.125.0, src/bin/qwen4exp_gpu_gate.rs: the device-router arm (softmax top-k
 *           over router logits; selected ids and their emitted order exact, weights to a few ulp;
 *           ties of duplicates across the cut, all-equal rows, underflow).
 *
 * Conventions for every call:
 *   - All pointers are DEVICE pointers unless marked [host].  Buffers are row-major and densely
 *     packed.  The caller allocates every buffer; the library never allocates, frees or
 *     synchronizes.  Each call only enqueues kernels on `stream` (0 = the null stream) and returns.
 *   - Sizes are int32.  Arguments are validated on the host before anything is enqueued.
 *   - Return value: FP4MOE_OK (0) on success; FP4MOE_EINVAL for an invalid argument (nothing was
 *     enqueued); FP4MOE_ELAUNCH when the HIP runtime reports a launch error; FP4MOE_EDEVICE when
 *     the optional device-side table check (fp4moe_set_debug_checks) finds a grouped call's
 *     tables invalid (nothing but the check was enqueued).  fp4moe_last_error() then holds a
 *     message (per thread).
 *   - Calls that write the same output buffer, or whose inputs another call writes, race unless
 *     the caller orders them (same stream or events).
 */
#ifndef FP4MOE_H
#define FP4MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define FP4MOE_API __attribute__((visibility("default")))
#else
#define FP4MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats (the pages' kind codes), plus a layout flag OR'ed into them: kinds 2 and 3 are
 * NVFP4 and MXFP4 planes in the swizzled layout written by fp4_weight_swizzle. */
enum { FP4MOE_NVFP4 = 0, FP4MOE_MXFP4 = 1, FP4MOE_SWIZZLED = 2 };
enum { FP4MOE_OK = 0, FP4MOE_EINVAL = 1, FP4MOE_ELAUNCH = 2, FP4MOE_EDEVICE = 3 };

/*
 * act_quant_fp8 -- [GATE: quant_rows].  For every row r and every group q of 128 columns:
 *   amax = max over the group of |x|, floored at 1e-4;
 *   s    = the smallest power of two >= f32(amax * f32(1/448));
 *   codes[r, c] = E4M3(clamp(x[r, c] / s, -448, 448)), round to nearest even, sign kept on zero;
 *   scales[r, q] = s.
 * x:      f32 [rows, k], read only.
 * codes:  u8  [rows, k], written (OCP E4M3FN bytes, bias 7, max 448).
 * scales: f32 [rows, k/128], written.
 * Errors: EINVAL if rows < 0, k <= 0, k % 128 != 0, or a pointer is NULL while rows > 0.
 * rows == 0 is a no-op.  Inputs must be finite (NaN/Inf give unspecified codes).
 */
FP4MOE_API int act_quant_fp8(const float* x, uint8_t* codes, float* scales, int32_t rows, int32_t k,
                  hipStream_t stream);

/*
 * fp4_expert_gemm -- [GATE: f64_ref, ExpertRaw].  One expert:
 *   out[r, c] = sum over groups j of ( sum over the gs k in group j of
 *                 E4M3(a_codes[r, k]) * E2M1(nibble(w_packed, c, k)) ) * ws[c, j] * a_scales[r, k/128]
 * with gs = 16 and ws = E4M3(w_scales[c, j]) * scale2 for NVFP4 (kind 0), gs = 32 and
 * ws = 2^(w_scales[c, j] - 127) for MXFP4 (kind 1; scale2 ignored), accumulated in f32.
 * a_codes:  u8  [g, k] E4M3 bytes;  a_scales: f32 [g, k/128], positive normal powers of two as
 *           act_quant_fp8 writes them (a call with more than 16 rows may run the tiled kernel,
 *           which writes NaN for a row using any other value; see fp4_grouped_gemm_gather).
 * w_packed: u8  [n, k/2]: element (c, k) is the low nibble of byte (c, k/2) for even k, the high
 *           nibble for odd k.
 * w_scales: u8  [n, k/16] E4M3 (NVFP4) or [n, k/32] E8M0 (MXFP4).
 * scale2:   [host] f32 per-tensor NVFP4 scale.
 * out:      f32 [g, n], overwritten.
 * Accuracy: |out - exact| <= k * 2^-24 * sum over k of |term| per output (f32 accumulation),
 * for inputs whose products stay in the f32 normal range.
 * kind may also be 2 (NVFP4) or 3 (MXFP4): w_packed and w_scales are then the swizzled planes
 * that fp4_weight_swizzle wrote for this n and k (same values, same result bit for bit).
 * Errors: EINVAL if g < 0, n <= 0, k <= 0, k % 128 != 0, kind not in 0..3, a pointer is NULL
 * while g > 0, or g*k or ceil(n/16)*16*k/2 is 2^31 or more (planes are addressed with 32-bit
 * offsets).  g == 0 is a no-op.
 */
FP4MOE_API int fp4_expert_gemm(const uint8_t* a_codes, const float* a_scales, const uint8_t* w_packed,
                    const uint8_t* w_scales, float scale2, int32_t kind, float* out, int32_t g,
                    int32_t n, int32_t k, hipStream_t stream);

/*
 * fp4_grouped_gemm -- [CHECK: f16g grouped GEMM, CSR offsets; GATE: f64_ref per expert, and the
 * FFI calls in `main` (a workspace passed explicitly, rc 0 = success)].
 * Routed rows packed per expert: packed row p belongs to expert e when
 * offsets[e] <= p < offsets[e+1], and out[p, :] is fp4_expert_gemm of activation row p with expert
 * e's planes, format and scale2.  Experts with no rows cost nothing; both formats may be mixed.
 * a_codes:  u8  [total_rows, k];  a_scales: f32 [total_rows, k/128], packed in the same row order.
 * offsets:  int32 [num_experts + 1], offsets[0] = 0, non-decreasing, offsets[E] = total_rows.
 * total_rows: [host] the packed row count (== offsets[E]; the host never reads offsets).
 * w_ptrs, s_ptrs: u64 [num_experts] device addresses of expert e's w_packed [n, k/2] and
 *           w_scales [n, k/gs] planes.
 * kinds:    int32 [num_experts] (0 NVFP4, 1 MXFP4; 2 and 3 the same formats with swizzled
 *           planes, see fp4_weight_swizzle);  scale2: f32 [num_experts] (NVFP4 only).
 * out:      f32 [total_rows, n], every row overwritten.
 * workspace, workspace_bytes: device scratch of at least fp4_grouped_gemm_workspace_size(...) bytes
 *           (currently 0: NULL with 0 bytes is valid).  Owned by the caller.
 * All tables are read on the device only.  Out-of-range table entries never cause an
 * out-of-bounds access: offsets are clamped to [0, total_rows]; a row whose expert has a kind
 * outside 0..3 is written as NaN.  With fp4moe_set_debug_checks(1) the tables are first validated
 * on the device (offsets[0] = 0, non-decreasing, offsets[E] = total_rows, kinds in 0..3): the call
 * then synchronizes `stream` and returns FP4MOE_EDEVICE, without launching the GEMM, when they fail.
 * a_scales are powers of two, as act_quant_fp8 writes them (see fp4_grouped_gemm_gather).
 * Errors: EINVAL if total_rows < 0, num_experts <= 0, n <= 0, k <= 0, k % 128 != 0, a pointer is
 * NULL while total_rows > 0, workspace is NULL with workspace_bytes > 0, workspace_bytes is below
 * the required size, or total_rows*k or ceil(n/16)*16*k/2 is 2^31 or more.  total_rows == 0 is a
 * no-op.
 */
FP4MOE_API size_t fp4_grouped_gemm_workspace_size(int32_t num_experts, int32_t total_rows, int32_t n, int32_t k);
FP4MOE_API int fp4_grouped_gemm(const uint8_t* a_codes, const float* a_scales, const int32_t* offsets,
                                int32_t num_experts, int32_t total_rows, const uint64_t* w_ptrs,
                                const uint64_t* s_ptrs, const int32_t* kinds, const float* scale2, float* out,
                                int32_t n, int32_t k, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * fp4_grouped_gemm_gather -- fp4_grouped_gemm with the activation rows read through a gather table,
 * so that act_quant_fp8 runs once per token instead of once per routed (token, expert) pair:
 * packed row p's activation is row row_ids[p] of a_codes/a_scales (row p itself when row_ids is
 * NULL).  Same definition, tables, output and debug check as fp4_grouped_gemm; no workspace.
 * a_codes:  u8  [a_rows, k];  a_scales: f32 [a_rows, k/128]  (e.g. one row per token).
 * row_ids:  int32 [total_rows] indices into [0, a_rows), or NULL (then a_rows >= total_rows).
 * A row whose row_ids entry is outside [0, a_rows) is written as NaN (the debug check reports it).
 * a_scales must be positive normal powers of two (act_quant_fp8 writes nothing else): the tiled
 * kernel that runs rows of experts holding many rows folds each scale into the activation operand
 * by its exponent and writes NaN for a row that uses any other value in a group it reads; the
 * other kernels apply any f32 value.
 * Errors: EINVAL if a_rows < 0, total_rows < 0, num_experts <= 0, n <= 0, k <= 0, k % 128 != 0,
 * row_ids is NULL while a_rows < total_rows, a pointer is NULL while total_rows > 0, or a_rows*k
 * or ceil(n/16)*16*k/2 is 2^31 or more.  total_rows == 0 is a no-op.
 */
FP4MOE_API int fp4_grouped_gemm_gather(const uint8_t* a_codes, const float* a_scales, int32_t a_rows,
                                       const int32_t* row_ids, const int32_t* offsets, int32_t num_experts,
                                       int32_t total_rows, const uint64_t* w_ptrs, const uint64_t* s_ptrs,
                                       const int32_t* kinds, const float* scale2, float* out, int32_t n,
                                       int32_t k, hipStream_t stream);

/*
 * fp4_weight_swizzle -- a load-time reordering of one expert's planes ([GATE: ExpertRaw] values,
 * unchanged) into the order in which the GEMM kernels' matrix-core lanes consume them, so that
 * every 64-lane weight load reads one contiguous 1 KB run instead of 16 column rows.  With
 * n16 = ceil(n/16), nblk = k/128, nq = ceil(nblk/4), column c = 16t + j (j < 16), 128-wide k block b,
 * and k piece p < 4 (k = 128b + 32p .. +32 of the block):
 *   w_swz[((t*nblk + b)*64 + 16p + j)*16 + i] = w_packed[c, 64b + 16p + i]          (i < 16)
 *   NVFP4: s_swz[((t*nq + q)*64 + 16p + j)*8 + 2m + e] = w_scales[c, 8(4q+m) + 2p + e]  (m < 4, e < 2)
 *   MXFP4: s_swz[((t*nq + q)*64 + 16p + j)*4 + m]      = w_scales[c, 4(4q+m) + p]       (m < 4)
 * Entries for columns c >= n or blocks 4q+m >= nblk are written as 0.
 * w_packed, w_scales: the plain planes of fp4_expert_gemm ([n, k/2] and [n, k/gs]), read only.
 * kind:   0 (NVFP4) or 1 (MXFP4): the scale plane's format.
 * w_swz:  u8 [fp4_swizzled_weight_bytes(n, k)], written.  s_swz: u8 [fp4_swizzled_scale_bytes(kind,
 *         n, k)], written.  Must not overlap the inputs.  Pass kind | FP4MOE_SWIZZLED to the GEMMs.
 * Errors: EINVAL if n <= 0, k <= 0, k % 128 != 0, kind not 0/1, a pointer is NULL, w_packed, w_swz
 * or s_swz is not 16-byte aligned, or ceil(n/16)*16*k/2 is 2^31 or more.
 * fp4_swizzled_weight_bytes / fp4_swizzled_scale_bytes: the plane sizes in bytes (host-only, no
 * device work): ceil(n/16)*16*k/2 and ceil(n/16)*nq*512 (NVFP4) or *256 (MXFP4); 0 when n <= 0,
 * k is not a positive multiple of 128, or kind is not 0/1.
 */
FP4MOE_API size_t fp4_swizzled_weight_bytes(int32_t n, int32_t k);
FP4MOE_API size_t fp4_swizzled_scale_bytes(int32_t kind, int32_t n, int32_t k);
FP4MOE_API int fp4_weight_swizzle(const uint8_t* w_packed, const uint8_t* w_scales, int32_t kind, int32_t n,
                                  int32_t k, uint8_t* w_swz, uint8_t* s_swz, hipStream_t stream);

/*
 * swiglu_quant_fp8 -- [GATE: the swiglu_limit saturation cell, then quant_rows].  The expert
 * activation between the fused gate/up projection and the down projection, quantized for the down
 * projection's GEMM.  For every row r and column i < inter:
 *   g = min(gu[r, i], limit);  u = clamp(gu[r, inter + i], -limit, limit);
 *   h[r, i] = g * (1 / (1 + exp(-g))) * u * w[r]      (f32 operations in this order; w[r] = 1 when
 *                                                       row_weights is NULL)
 * then codes/scales = act_quant_fp8(h) (same definition as above, per 128 columns of h).
 * gu:          f32 [rows, 2*inter], read only: the gate/up GEMM output, gate columns first.
 * row_weights: f32 [rows] or NULL: a per-row factor (e.g. the routing weight of the packed row).
 * limit:       [host] f32 > 0 (may be +Inf: no clamping).
 * codes:       u8  [rows, inter], written.   scales: f32 [rows, inter/128], written.
 * h_out:       f32 [rows, inter] or NULL: when given, receives h before quantization.
 * Errors: EINVAL if rows < 0, inter <= 0, inter % 128 != 0, limit is not > 0, or a required
 * pointer is NULL while rows > 0.  rows == 0 is a no-op.  exp is the device library's f32 expf, so
 * h agrees with an exact evaluation to a few f32 ulps; inputs must be finite.
 */
FP4MOE_API int swiglu_quant_fp8(const float* gu, const float* row_weights, float limit, uint8_t* codes,
                                float* scales, float* h_out, int32_t rows, int32_t inter,
                                hipStream_t stream);

/*
 * fp4_grouped_gemm_swiglu_quant -- [CHECK: f16g grouped GEMM; GATE: the swiglu_limit saturation cell,
 * then quant_rows].  The gate/up projection of the routed rows with the expert activation and its
 * FP8 quantization applied before anything is written: the result is bit-identical to
 *   gu = fp4_grouped_gemm_gather(..., n = 2*inter, ...)   (the tiled schedule)
 *   swiglu_quant_fp8(gu, row_weights, limit, h_codes, h_scales, h_out, total_rows, inter)
 * without the f32 [total_rows, 2*inter] intermediate.  Expert planes are [2*inter, k/2] (gate columns
 * first, then up), as for fp4_grouped_gemm_gather with n = 2*inter.  A packed row whose row_ids entry is
 * out of range, or whose expert has a kind outside 0..3, enters the activation as NaN gate and up
 * values, exactly as the unfused route's NaN GEMM output would.
 * Arguments as for fp4_grouped_gemm_gather (debug check included) and swiglu_quant_fp8:
 * row_weights: f32 [total_rows] or NULL (per packed row);  limit: [host] f32 > 0 (+Inf: no clamp).
 * h_codes:     u8  [total_rows, inter], 16-byte aligned, written.
 * h_scales:    f32 [total_rows, inter/128], written.
 * h_out:       f32 [total_rows, inter], 16-byte aligned, or NULL: receives h when given.
 * Errors: EINVAL on the conditions of fp4_grouped_gemm_gather (with n = 2*inter), inter not a positive
 * multiple of 128 up to 2^29, limit not > 0, or a misaligned h_codes/h_out.  total_rows == 0 is a
 * no-op.
 */
FP4MOE_API int fp4_grouped_gemm_swiglu_quant(const uint8_t* a_codes, const float* a_scales, int32_t a_rows,
                                  const int32_t* row_ids, const int32_t* offsets, int32_t num_experts,
                                  int32_t total_rows, const uint64_t* w_ptrs, const uint64_t* s_ptrs,
                                  const int32_t* kinds, const float* scale2, int32_t inter, int32_t k,
                                  const float* row_weights, float limit, uint8_t* h_codes, float* h_scales,
                                  float* h_out, hipStream_t stream);

/*
 * route_softmax_topk -- [QWEN: the device-router arm].  For every token t, the top_k experts by
 * router logit, best first, and their softmax weights:
 *   ranking: a larger logit first; equal logits (+0 equal to -0) by the lower expert id; NaN below
 *            every number (NaNs among themselves by id);
 *   m = the largest logit of the row;  e_x = exp(x - m);
 *   topk_weights[t, j] = e_{l[t, id_j]} / D, with D = sum of e over all experts of the row, or over
 *            the top_k selected ones (in selection order) when normalize = 1.
 *   A row holding a NaN, or whose largest logit is +Inf or every logit -Inf, gets NaN weights.
 * logits:       f32 [tokens, experts], read only.
 * topk_ids:     int32 [tokens, top_k], written.   topk_weights: f32 [tokens, top_k], written.
 * normalize:    [host] 0 or 1.
 * Selection compares the f32 logits exactly, so the ids and their order are the exact top-k of the
 * softmax; the weights are f32 (device expf, a tree sum over the row, one division): they agree with
 * an exact evaluation to a relative 2^-24 (|x - m| + mean |x' - m| + log2(experts) + 6) or so.
 * Errors: EINVAL if tokens < 0, experts < 1 or > 1024, top_k < 1 or > min(experts, 64), normalize
 * not 0/1, a pointer NULL while tokens > 0, or 4*tokens*experts >= 2^31.  tokens == 0 is a no-op.
 */
FP4MOE_API int route_softmax_topk(const float* logits, int32_t tokens, int32_t experts, int32_t top_k,
                                  int32_t normalize, int32_t* topk_ids, float* topk_weights,
                                  hipStream_t stream);

/*
 * route_pack_workspace_size -- [host] bytes of device workspace route_pack needs for these sizes:
 * 4 x experts x (ceil(tokens / 64) + 1); 0 for tokens < 0 or experts <= 0.
 */
FP4MOE_API int64_t route_pack_workspace_size(int32_t tokens, int32_t experts);

/*
 * route_pack -- [CHECK: f16g grouped GEMM section, rows packed per expert behind CSR offsets].  The
 * pairs p = t * top_k + j of a routing table are packed per expert: expert e owns the packed rows
 * offsets[e] .. offsets[e+1]-1, experts in ascending id, and inside one expert the pairs in
 * ascending (t, j) order, i.e. ascending token order.  Pairs whose id lies outside [0, experts) are
 * dropped.  The outputs feed fp4_grouped_gemm_gather (row_ids gathers the activation rows, offsets delimits
 * the experts) and moe_combine (pair_rows).
 * topk_ids:     int32 [tokens, top_k], read only (ids of one token may repeat; each pair is a row).
 * topk_weights: f32 [tokens, top_k] or NULL, read only.
 * offsets:      int32 [experts + 1], written; offsets[experts] = the number of packed rows R.
 * row_ids:      int32 [tokens * top_k], rows 0 .. R-1 written: the token of each packed row.
 * pair_rows:    int32 [tokens, top_k], written: the packed row of each pair, -1 if dropped.
 * row_weights:  f32 [tokens * top_k] or NULL: rows 0 .. R-1 receive topk_weights moved to their
 *               packed row (ignored when topk_weights is NULL).
 * workspace:    route_pack_workspace_size(tokens, experts) bytes of device memory, 4-byte aligned,
 *               overwritten (no initial contents needed).
 * Errors: EINVAL if tokens < 0, top_k < 1 or > 64, experts < 1 or > 1024, tokens*top_k >= 2^31, or
 * a required pointer is NULL (offsets and workspace always; the others when tokens > 0).
 * tokens == 0 writes offsets = 0 only.
 */
FP4MOE_API int route_pack(const int32_t* topk_ids, const float* topk_weights, int32_t tokens,
                          int32_t top_k, int32_t experts, int32_t* offsets, int32_t* row_ids,
                          int32_t* pair_rows, float* row_weights, void* workspace, hipStream_t stream);

/*
 * route_pack_noalloc -- for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): route_pack without the workspace argument.
 * Same arguments, outputs, bits and errors as route_pack; the workspace is instead a library-owned
 * device array of 1 MiB per device (allocated when the library is loaded, held until the process
 * ends), so tokens and experts are limited to route_pack_workspace_size(tokens, experts) <= 1 MiB
 * (e.g. 256 experts up to 65,472 tokens; 1024 experts up to 16,320 tokens); larger sizes return
 * FP4MOE_EINVAL.  Allocates nothing.  Every call on one device shares that device's array: calls
 * that overlap on one device (different streams, or host threads without ordering) race and must
 * be serialized by the caller; successive calls on one stream are safe (each overwrites what it
 * reads).
 */
FP4MOE_API int route_pack_noalloc(const int32_t* topk_ids, const float* topk_weights, int32_t tokens,
                                  int32_t top_k, int32_t experts, int32_t* offsets, int32_t* row_ids,
                                  int32_t* pair_rows, float* row_weights, hipStream_t stream);

/*
 * gather_quant_rows -- [CHECK: f16g grouped GEMM section; the packed activation rows].  Copies the
 * act-quant rows row_ids[p] into packed row p: out_codes[p, :] = codes[row_ids[p], :] and
 * out_scales[p, :] = scales[row_ids[p], :].  A row id outside [0, a_rows) gives zero code bytes and
 * NaN scales.  fp4_grouped_gemm_gather reads through row_ids itself; this call builds a contiguous copy
 * (e.g. a send buffer of routed rows).
 * codes:  u8 [a_rows, k], scales: f32 [a_rows, k/128], read only.  row_ids: int32 [rows].
 * out_codes: u8 [rows, k], out_scales: f32 [rows, k/128], written.
 * Errors: EINVAL if a_rows < 0, rows < 0, k <= 0, k % 128 != 0, a required pointer is NULL, codes
 * or out_codes is not 16-byte aligned, or a_rows*k or rows*k >= 2^31.  rows == 0 is a no-op.
 */
FP4MOE_API int gather_quant_rows(const uint8_t* codes, const float* scales, int32_t a_rows, int32_t k,
                                 const int32_t* row_ids, int32_t rows, uint8_t* out_codes,
                                 float* out_scales, hipStream_t stream);

/*
 * moe_combine -- [QWEN: routing; CHECK: packed rows].  The expert outputs back in token order:
 *   out[t, c] = sum over j < top_k of w[t, j] * y[pair_rows[t, j], c]
 * added in j order, one f32 fused multiply-add per term (a plain f32 add when pair_weights is NULL,
 * i.e. w = 1).  Pairs with pair_rows < 0 are skipped; a row at or past y_rows makes the token's whole
 * output row NaN.  Deterministic: no atomics.
 * y:            f32 [y_rows, n], read only (e.g. the grouped GEMM's packed output).
 * pair_rows:    int32 [tokens, top_k], read only (route_pack's output).
 * pair_weights: f32 [tokens, top_k] or NULL.
 * out:          f32 [tokens, n], written.
 * Errors: EINVAL if tokens < 0, y_rows < 0, n <= 0, top_k < 1 or > 64, a required pointer is NULL,
 * or tokens*n or y_rows*n >= 2^31.  tokens == 0 is a no-op.
 */
FP4MOE_API int moe_combine(const float* y, int32_t y_rows, int32_t n, const int32_t* pair_rows,
                           const float* pair_weights, int32_t tokens, int32_t top_k, float* out,
                           hipStream_t stream);

/*
 * The bf16-dequant rung -- [GATE: comparison 3, the class shift against the bf16-dequant rung on
 * the same inputs].  A reference route on unquantized activations and exact weights: cvt_bf16 of
 * the f32 activations, fp4_dequant_bf16 of the expert, gemm_bf16 of the two.  The native path's
 * difference from it is the shift caused by quantizing the activations to E4M3, predicted per
 * output as (2^-4 / sqrt 3) * ||x (.) w||_2.  Not on the hot path.
 *
 * cvt_bf16 -- out[i] = bf16(x[i]): round to nearest, ties to even; NaN stays NaN (sign and the top
 * payload bits kept, quiet bit set).  x: f32 [count]; out: bf16 bit patterns [count].
 * Errors: EINVAL if count < 0 or a pointer is NULL while count > 0.  count == 0 is a no-op.
 */
FP4MOE_API int cvt_bf16(const float* x, uint16_t* out, int64_t count, hipStream_t stream);

/*
 * fp4_dequant_bf16 -- out[c, j] = bf16(f32(E2M1(W[c, j]) * ws[c, j / gs])) with the GEMM's weight
 * scale: ws = f32(E4M3(S) * scale2) for NVFP4 (gs 16), 2^(S - 127) for MXFP4 (gs 32, S = 255 NaN);
 * a NaN result is written as the canonical bf16 NaN 0x7FC0.
 * w_packed: u8 [n, k/2] (4-byte aligned); w_scales: u8 [n, k/gs]; out: bf16 [n, k] (16-byte aligned).
 * Errors: EINVAL if n < 0, k <= 0, k % 128 != 0, kind not 0/1, 2*n*k >= 2^31, a pointer is NULL while
 * n > 0, or an alignment is not met.  n == 0 is a no-op.
 */
FP4MOE_API int fp4_dequant_bf16(const uint8_t* w_packed, const uint8_t* w_scales, float scale2, int32_t kind,
                                int32_t n, int32_t k, uint16_t* out, hipStream_t stream);

/*
 * gemm_bf16 -- out[r, c] = sum_j a[r, j] * w[c, j]: bf16 operands (exact products), f32 accumulation
 * in ascending j over 16-wide steps.  a: bf16 [m, k]; w: bf16 [n, k]; out: f32 [m, n].
 * Errors: EINVAL if m < 0, n <= 0, k <= 0, k % 16 != 0, 2*m*k or 2*n*k >= 2^31, or a pointer is NULL
 * while m > 0.  m == 0 is a no-op.
 */
FP4MOE_API int gemm_bf16(const uint16_t* a, const uint16_t* w, float* out, int32_t m, int32_t n, int32_t k,
                         hipStream_t stream);

/*
 * The W4A4 NVFP4 variant -- [CHECK: the NVFP4 MMQ W4A4 arms].  Lossy (E2M1 activations): held to
 * the pages' relative-error bands and comparisons, not to the FP8 path's bound.
 *
 * act_quant_fp4 -- per row r (f32, each step one IEEE operation):
 *   rs[r] = amax_row / 2688 when two_level = 1 and the row is not all zero, else 1;
 *   micro[r, g] = E4M3(clamp((amax_g / rs) / 6, 2^-9, 448)), round to nearest even; 0 for a zero group;
 *   codes[r, j] = E2M1((x[r, j] / rs) / micro): nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the
 *   even code, capped at 6, sign in bit 3; 0 when micro is 0.  amax over 16-element groups g.
 * Channels listed in skip_channels (int32 [n_skip], device, entries outside [0, k) ignored) count as 0.
 * x: f32 [rows, k] (16-byte aligned); codes: u8 [rows, k/2] (even j in the low nibble, 2-byte
 * aligned); micro: u8 [rows, k/16]; row_scale: f32 [rows].
 * Errors: EINVAL if rows < 0, k <= 0, k % 128 != 0, n_skip outside [0, 64], two_level not 0/1,
 * 4*rows*k >= 2^31, an alignment is not met, or a required pointer is NULL while rows > 0.
 */
FP4MOE_API int act_quant_fp4(const float* x, const int32_t* skip_channels, int32_t n_skip, uint8_t* codes,
                             uint8_t* micro, float* row_scale, int32_t rows, int32_t k, int32_t two_level,
                             hipStream_t stream);

/*
 * loud_channels -- idx[j], j < k_res: the channels with the largest max over rows of |x[r, c]|, the
 * loudest first, ties to the lower channel.  x: f32 [rows, k]; idx: int32 [k_res] (device).
 * Errors: EINVAL if rows < 0, k outside [1, 8192], k_res outside [0, min(k, 64)], 4*rows*k >= 2^31,
 * or a required pointer is NULL.  k_res == 0 is a no-op.
 */
FP4MOE_API int loud_channels(const float* x, int32_t rows, int32_t k, int32_t k_res, int32_t* idx,
                             hipStream_t stream);

/*
 * w4a4_gemm -- out[r, c] = rs[r] * scale2 * sum_j (E2M1(a[r, j]) * micro[r, j/16]) * (E2M1(w[c, j]) *
 * E4M3(S[c, j/16])), f32 accumulation of exact products, plus, for the k_res kept channels res_idx[i],
 * x[r, res_idx[i]] * E2M1(w[c, res_idx[i]]) * f32(E4M3(S) * scale2) (x f32 [g, k]; those channels
 * should be the ones act_quant_fp4 skipped).  NVFP4 weights as in fp4_expert_gemm.  out: f32 [g, n].
 * Errors: EINVAL if g < 0, n <= 0, k <= 0, k % 128 != 0, k_res outside [0, 64], a plane reaches 2^31
 * bytes, or a required pointer is NULL while g > 0.  g == 0 is a no-op.
 */
FP4MOE_API int w4a4_gemm(const uint8_t* a_codes, const uint8_t* a_micro, const float* a_row_scale,
                         const uint8_t* w_packed, const uint8_t* w_scales, float scale2, const float* x,
                         const int32_t* res_idx, int32_t k_res, float* out, int32_t g, int32_t n, int32_t k,
                         hipStream_t stream);

/*
 * fp4moe_set_gemm_schedule -- test and benchmark hook (not part of the method).  The GEMM calls
 * pick a kernel from the host-known rows per expert: a row-streaming kernel (each expert's weights
 * read once per pass of 32 rows; used when total rows <= 32 x experts) or a tiled matrix-core
 * kernel (128 x 256 output tiles); a single-expert call (fp4_expert_gemm) with g <= 16 and
 * k <= 8192, or a grouped call with at most 16 packed rows, k <= 8192 and at most 1024 experts,
 * uses a split-k kernel instead (16-column tiles whose wavefronts split k and sum their tiles in a
 * fixed order: 4, 8 or 16 per tile for a single expert, from k alone; 8, 4, 2 or 1 for a grouped
 * call, from its packed rows, experts and n).  All compute the same definition to the same accuracy bound; only the
 * order of the f32 additions differs.  schedule: 0 = automatic (default), 1 = always row-streaming,
 * 2 = always tiled, 3 = split-k for the calls that fit it (grouped calls with up to 128 packed
 * rows; other calls as 0).  Process-wide; affects calls made after it returns.
 * Errors: EINVAL for any other value.
 */
enum { FP4MOE_SCHEDULE_AUTO = 0, FP4MOE_SCHEDULE_ROWSTREAM = 1, FP4MOE_SCHEDULE_TILED = 2,
       FP4MOE_SCHEDULE_SPLITK = 3 };
FP4MOE_API int fp4moe_set_gemm_schedule(int32_t schedule);

/*
 * fp4moe_set_debug_checks -- a debugging aid (not part of the method).  With on = 1, every grouped
 * call (fp4_grouped_gemm, fp4_grouped_gemm_gather, fp4_grouped_gemm_swiglu_quant) first runs a
 * one-workgroup kernel that validates its tables on the device -- offsets[0] = 0, offsets
 * non-decreasing, offsets[E] = total_rows, every row_ids entry in [0, a_rows), every kind in 0..3 --
 * then synchronizes `stream` and returns FP4MOE_EDEVICE, with the first violation in
 * fp4moe_last_error(), instead of launching the GEMM.  The check's status words are library-owned
 * device memory (one small array per device, shared by all calls on it; calls from several host
 * threads are serialized by a lock).  on = 0 (the default) removes the check and the
 * synchronization.  Process-wide.  Errors: EINVAL for any other value.
 */
FP4MOE_API int fp4moe_set_debug_checks(int32_t on);

/* Message for the last nonzero return code of a call made by this thread ("" if none). */
FP4MOE_API const char* fp4moe_last_error(void);

/* Library version string. */
FP4MOE_API const char* fp4moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FP4MOE_H */
