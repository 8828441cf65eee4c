// capi.hip -- the extern "C" entry points of libfp4moe (declared and documented in
// include/fp4moe.h): host-side argument validation, kernel dispatch, per-thread error messages.
#include <atomic>
#include <mutex>
#include <cstdarg>
#include <cstdio>

#include "fp4moe.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return FP4MOE_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FP4MOE_ELAUNCH, "%s: HIP launch error: %s", what, hipGetErrorString(e));
  return ok();
}

int check_k(int32_t k, const char* what) {
  if (k <= 0 || k % 128 != 0)
    return fail(FP4MOE_EINVAL, "%s: k = %d must be a positive multiple of 128", what, (int)k);
  return FP4MOE_OK;
}

// The GEMM kernels address every operand plane with 32-bit byte offsets: each plane must stay
// below 2^31 bytes.
constexpr int64_t kMaxPlaneBytes = (int64_t)1 << 31;

int check_planes(int64_t a_rows, int32_t n, int32_t k, const char* what) {
  if (a_rows * (int64_t)k >= kMaxPlaneBytes)
    return fail(FP4MOE_EINVAL, "%s: activation plane of %lld x %d bytes exceeds 2^31", what,
                (long long)a_rows, (int)k);
  // the swizzled planes round n up to a multiple of 16 columns
  if ((int64_t)(n + 15) / 16 * 16 * (k / 2) >= kMaxPlaneBytes)
    return fail(FP4MOE_EINVAL, "%s: weight plane of %d x %d bytes exceeds 2^31", what, (int)n, (int)(k / 2));
  return FP4MOE_OK;
}

bool is_gemm_kind(int32_t kind) { return kind >= 0 && kind <= (FP4MOE_MXFP4 | FP4MOE_SWIZZLED); }

// GEMM schedule: row-streaming (decode) kernel for at most 32 rows per expert on average, tiled
// (prefill) kernel otherwise.  Both compute the same definition; the choice only changes the
// order of the f32 additions.  fp4moe_set_gemm_schedule forces one of them (test hook).
std::atomic<int> g_schedule{FP4MOE_SCHEDULE_AUTO};

hipError_t launch_gemm(const fp4moe::GemmArgs& a, int64_t rows, int64_t experts, hipStream_t stream) {
  int s = g_schedule.load(std::memory_order_relaxed);
  // Very few rows: the split-k kernel (the row-streaming kernel would launch only ceil(n/256)
  // workgroups per active expert).
  if ((s == FP4MOE_SCHEDULE_AUTO || s == FP4MOE_SCHEDULE_SPLITK) &&
      (a.offsets ? fp4moe::gemm_skinny_grouped_fits(rows, a.num_experts, a.n, a.k, s == FP4MOE_SCHEDULE_SPLITK)
                 : fp4moe::gemm_skinny_fits((int32_t)rows, a.n, a.k)))
    return fp4moe::launch_gemm_skinny(a, stream);
  if (s == FP4MOE_SCHEDULE_AUTO || s == FP4MOE_SCHEDULE_SPLITK)
    s = (rows <= 32 * experts) ? FP4MOE_SCHEDULE_ROWSTREAM : FP4MOE_SCHEDULE_TILED;
  return s == FP4MOE_SCHEDULE_TILED ? fp4moe::launch_gemm_prefill(a, stream) : fp4moe::launch_gemm_decode(a, stream);
}

// Optional device-side validation of the grouped tables (fp4moe_set_debug_checks).  The status words
// live in a file-scope device array; host code reaches them only through the address that
// hipGetSymbolAddress returns for the current device (the array's name is a host-side stand-in).
__device__ __align__(256) int32_t g_table_status[fp4moe::kTableCheckWords];
std::atomic<int> g_debug_checks{0};
std::mutex g_check_mutex;
constexpr int kMaxDevices = 64;
int32_t* g_status_ptr[kMaxDevices] = {};

int debug_check_tables(const char* what, const int32_t* offsets, int32_t num_experts, int32_t total_rows,
                       const int32_t* row_ids, int32_t a_rows, const int32_t* kinds, hipStream_t stream) {
  if (!g_debug_checks.load(std::memory_order_relaxed)) return FP4MOE_OK;
  std::lock_guard<std::mutex> lock(g_check_mutex);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FP4MOE_ELAUNCH, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FP4MOE_ELAUNCH, "%s: device %d out of range", what, dev);
  if (!g_status_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_table_status));
    if (e != hipSuccess || !p)
      return fail(FP4MOE_ELAUNCH, "%s: hipGetSymbolAddress: %s", what, hipGetErrorString(e));
    g_status_ptr[dev] = static_cast<int32_t*>(p);
  }
  e = fp4moe::launch_table_check(offsets, num_experts, total_rows, row_ids, a_rows, kinds, g_status_ptr[dev], stream);
  if (e != hipSuccess) return fail(FP4MOE_ELAUNCH, "%s: table check launch: %s", what, hipGetErrorString(e));
  int32_t st[fp4moe::kTableCheckWords];
  e = hipMemcpyAsync(st, g_status_ptr[dev], sizeof st, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(FP4MOE_ELAUNCH, "%s: table check readback: %s", what, hipGetErrorString(e));
  if (st[0] >= 0) return fail(FP4MOE_EDEVICE, "%s: device check: offsets[0] is not 0", what);
  if (st[1] >= 0)
    return fail(FP4MOE_EDEVICE, "%s: device check: offsets decrease at expert %d (offsets[%d] < offsets[%d])", what,
                (int)st[1], (int)st[1] + 1, (int)st[1]);
  if (st[2] >= 0) return fail(FP4MOE_EDEVICE, "%s: device check: offsets[%d] != total_rows = %d", what, (int)st[2],
                              (int)total_rows);
  if (st[3] >= 0)
    return fail(FP4MOE_EDEVICE, "%s: device check: row_ids[%d] is outside [0, %d)", what, (int)st[3], (int)a_rows);
  if (st[4] >= 0) return fail(FP4MOE_EDEVICE, "%s: device check: kinds[%d] is not in 0..3", what, (int)st[4]);
  return FP4MOE_OK;
}

// route_pack's body, with its workspace (counts then totals, fully overwritten) given.
int pack_routes(const char* what, const int32_t* topk_ids, const float* topk_weights, int32_t tokens, int32_t top_k,
                int32_t experts, int32_t* offsets, int32_t* row_ids, int32_t* pair_rows, float* row_weights,
                int32_t* workspace, hipStream_t stream) {
  if (tokens < 0) return fail(FP4MOE_EINVAL, "%s: tokens = %d < 0", what, (int)tokens);
  if (top_k < 1 || top_k > 64) return fail(FP4MOE_EINVAL, "%s: top_k = %d must be in [1, 64]", what, (int)top_k);
  if (experts < 1 || experts > 1024)
    return fail(FP4MOE_EINVAL, "%s: experts = %d must be in [1, 1024]", what, (int)experts);
  if ((int64_t)tokens * top_k >= kMaxPlaneBytes)
    return fail(FP4MOE_EINVAL, "%s: tokens x top_k must stay below 2^31", what);
  if (!offsets) return fail(FP4MOE_EINVAL, "%s: offsets is NULL", what);
  if (tokens > 0 && (!topk_ids || !row_ids || !pair_rows))
    return fail(FP4MOE_EINVAL, "%s: NULL buffer with tokens > 0", what);
  return launched(fp4moe::launch_route_pack(topk_ids, topk_weights, tokens, top_k, experts, offsets, row_ids,
                                            pair_rows, topk_weights ? row_weights : nullptr, workspace, stream),
                  what);
}

// The scratch memory of the allocation-free entry point (route_pack_noalloc): route_pack's workspace
// in a file-scope device array of kScratchWords int32 (1 MiB), one copy per device for the life of the
// process.  Host code never uses the array's name as an address: the first call on a device takes
// that device's address with hipGetSymbolAddress and keeps it.  Every call on a device shares its
// copy (each call overwrites what it uses before reading it), so calls that overlap on one device race.
constexpr int64_t kScratchWords = (int64_t)1 << 18;
__device__ __align__(256) int32_t scratch[kScratchWords];
std::mutex g_scratch_mutex;
int32_t* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(const char* what, int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FP4MOE_ELAUNCH, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FP4MOE_ELAUNCH, "%s: device %d out of range", what, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(FP4MOE_ELAUNCH, "%s: hipGetSymbolAddress: %s", what, hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return FP4MOE_OK;
}

// The grouped GEMM behind fp4_grouped_gemm (row_ids == nullptr, a_rows == total_rows) and
// fp4_grouped_gemm_gather.
int grouped_gemm(const char* what, const uint8_t* a_codes, const float* a_scales, int32_t a_rows,
                 const int32_t* row_ids, const int32_t* offsets, int32_t num_experts, int32_t total_rows,
                 const uint64_t* w_ptrs, const uint64_t* s_ptrs, const int32_t* kinds, const float* scale2, float* out,
                 int32_t n, int32_t k, hipStream_t stream) {
  if (a_rows < 0 || total_rows < 0)
    return fail(FP4MOE_EINVAL, "%s: a_rows = %d, total_rows = %d must be >= 0", what, (int)a_rows, (int)total_rows);
  if (num_experts <= 0) return fail(FP4MOE_EINVAL, "%s: num_experts = %d must be positive", what, (int)num_experts);
  if (n <= 0) return fail(FP4MOE_EINVAL, "%s: n = %d must be positive", what, (int)n);
  if (int rc = check_k(k, what)) return rc;
  if (!row_ids && a_rows < total_rows)
    return fail(FP4MOE_EINVAL, "%s: row_ids is NULL but a_rows = %d < total_rows = %d", what, (int)a_rows,
                (int)total_rows);
  if (total_rows == 0) return ok();
  if (!a_codes || !a_scales || !offsets || !w_ptrs || !s_ptrs || !kinds || !scale2 || !out)
    return fail(FP4MOE_EINVAL, "%s: NULL buffer with total_rows > 0", what);
  if (int rc = check_planes(a_rows, n, k, what)) return rc;
  if (int rc = debug_check_tables(what, offsets, num_experts, total_rows, row_ids, a_rows, kinds, stream)) return rc;
  fp4moe::GemmArgs a{};
  a.a_codes = a_codes;
  a.a_scales = a_scales;
  a.row_ids = row_ids;
  a.a_rows = a_rows;
  a.offsets = offsets;
  a.num_experts = num_experts;
  a.total_rows = total_rows;
  a.w_ptrs = w_ptrs;
  a.s_ptrs = s_ptrs;
  a.kinds = kinds;
  a.scale2s = scale2;
  a.out = out;
  a.n = n;
  a.k = k;
  return launched(launch_gemm(a, total_rows, num_experts, stream), what);
}

}  // namespace

extern "C" {

int act_quant_fp8(const float* x, uint8_t* codes, float* scales, int32_t rows, int32_t k,
                  hipStream_t stream) {
  if (rows < 0) return fail(FP4MOE_EINVAL, "act_quant_fp8: rows = %d < 0", (int)rows);
  if (int rc = check_k(k, "act_quant_fp8")) return rc;
  if (rows == 0) return ok();
  if (!x || !codes || !scales) return fail(FP4MOE_EINVAL, "act_quant_fp8: NULL buffer with rows > 0");
  const int64_t ngroups = (int64_t)rows * (k / 128);
  return launched(fp4moe::launch_act_quant(x, codes, scales, ngroups, stream), "act_quant_fp8");
}

int swiglu_quant_fp8(const float* gu, const float* row_weights, float limit, uint8_t* codes,
                     float* scales, float* h_out, int32_t rows, int32_t inter, hipStream_t stream) {
  if (rows < 0) return fail(FP4MOE_EINVAL, "swiglu_quant_fp8: rows = %d < 0", (int)rows);
  if (inter <= 0 || inter % 128 != 0)
    return fail(FP4MOE_EINVAL, "swiglu_quant_fp8: inter = %d must be a positive multiple of 128", (int)inter);
  if (!(limit > 0.0f)) return fail(FP4MOE_EINVAL, "swiglu_quant_fp8: limit must be > 0");
  if (rows == 0) return ok();
  if (!gu || !codes || !scales) return fail(FP4MOE_EINVAL, "swiglu_quant_fp8: NULL buffer with rows > 0");
  return launched(fp4moe::launch_swiglu_quant(gu, row_weights, limit, codes, scales, h_out, rows, inter, stream),
                  "swiglu_quant_fp8");
}

int route_softmax_topk(const float* logits, int32_t tokens, int32_t experts, int32_t top_k, int32_t normalize,
                       int32_t* topk_ids, float* topk_weights, hipStream_t stream) {
  const char* what = "route_softmax_topk";
  if (tokens < 0) return fail(FP4MOE_EINVAL, "%s: tokens = %d < 0", what, (int)tokens);
  if (experts < 1 || experts > 1024)
    return fail(FP4MOE_EINVAL, "%s: experts = %d must be in [1, 1024]", what, (int)experts);
  if (top_k < 1 || top_k > experts || top_k > 64)
    return fail(FP4MOE_EINVAL, "%s: top_k = %d must be in [1, min(experts, 64)]", what, (int)top_k);
  if (normalize != 0 && normalize != 1)
    return fail(FP4MOE_EINVAL, "%s: normalize = %d must be 0 or 1", what, (int)normalize);
  if ((int64_t)tokens * experts * 4 >= kMaxPlaneBytes)
    return fail(FP4MOE_EINVAL, "%s: the logits plane must stay below 2^31 bytes", what);
  if (tokens == 0) return ok();
  if (!logits || !topk_ids || !topk_weights) return fail(FP4MOE_EINVAL, "%s: NULL buffer with tokens > 0", what);
  return launched(fp4moe::launch_route_topk(logits, tokens, experts, top_k, normalize, topk_ids, topk_weights,
                                            stream),
                  what);
}

int64_t route_pack_workspace_size(int32_t tokens, int32_t experts) {
  if (tokens < 0 || experts <= 0) return 0;
  return 4 * fp4moe::route_pack_workspace_elems(tokens, experts);
}

int route_pack(const int32_t* topk_ids, const float* topk_weights, int32_t tokens, int32_t top_k, int32_t experts,
               int32_t* offsets, int32_t* row_ids, int32_t* pair_rows, float* row_weights, void* workspace,
               hipStream_t stream) {
  const char* what = "route_pack";
  if (!workspace) return fail(FP4MOE_EINVAL, "%s: workspace is NULL", what);
  if (reinterpret_cast<uintptr_t>(workspace) & 3) return fail(FP4MOE_EINVAL, "%s: workspace not 4-byte aligned", what);
  return pack_routes(what, topk_ids, topk_weights, tokens, top_k, experts, offsets, row_ids, pair_rows, row_weights,
                     static_cast<int32_t*>(workspace), stream);
}

int route_pack_noalloc(const int32_t* topk_ids, const float* topk_weights, int32_t tokens, int32_t top_k,
                       int32_t experts, int32_t* offsets, int32_t* row_ids, int32_t* pair_rows, float* row_weights,
                       hipStream_t stream) {
  const char* what = "route_pack_noalloc";
  if (tokens >= 0 && experts >= 1 && experts <= 1024) {
    const int64_t words = fp4moe::route_pack_workspace_elems(tokens, experts);
    if (words > kScratchWords)
      return fail(FP4MOE_EINVAL, "%s: %d tokens x %d experts need %lld bytes of scratch; the library's array "
                  "holds %lld", what, (int)tokens, (int)experts, (long long)(4 * words), (long long)(4 * kScratchWords));
  }
  int32_t* ws = nullptr;
  if (int rc = scratch_for_current_device(what, &ws)) return rc;
  return pack_routes(what, topk_ids, topk_weights, tokens, top_k, experts, offsets, row_ids, pair_rows, row_weights,
                     ws, stream);
}

int gather_quant_rows(const uint8_t* codes, const float* scales, int32_t a_rows, int32_t k, const int32_t* row_ids,
                      int32_t rows, uint8_t* out_codes, float* out_scales, hipStream_t stream) {
  const char* what = "gather_quant_rows";
  if (a_rows < 0 || rows < 0)
    return fail(FP4MOE_EINVAL, "%s: a_rows = %d, rows = %d must be >= 0", what, (int)a_rows, (int)rows);
  if (int rc = check_k(k, what)) return rc;
  if ((int64_t)a_rows * k >= kMaxPlaneBytes || (int64_t)rows * k >= kMaxPlaneBytes)
    return fail(FP4MOE_EINVAL, "%s: a code plane of 2^31 bytes or more", what);
  if (rows == 0) return ok();
  if (!row_ids || !out_codes || !out_scales || (a_rows > 0 && (!codes || !scales)))
    return fail(FP4MOE_EINVAL, "%s: NULL buffer with rows > 0", what);
  if ((reinterpret_cast<uintptr_t>(codes) | reinterpret_cast<uintptr_t>(out_codes)) & 15)
    return fail(FP4MOE_EINVAL, "%s: codes and out_codes must be 16-byte aligned", what);
  return launched(fp4moe::launch_gather_rows(codes, scales, a_rows, k, row_ids, rows, out_codes, out_scales, stream),
                  what);
}

int moe_combine(const float* y, int32_t y_rows, int32_t n, const int32_t* pair_rows, const float* pair_weights,
                int32_t tokens, int32_t top_k, float* out, hipStream_t stream) {
  const char* what = "moe_combine";
  if (tokens < 0 || y_rows < 0)
    return fail(FP4MOE_EINVAL, "%s: tokens = %d, y_rows = %d must be >= 0", what, (int)tokens, (int)y_rows);
  if (n <= 0) return fail(FP4MOE_EINVAL, "%s: n = %d must be positive", what, (int)n);
  if (top_k < 1 || top_k > 64) return fail(FP4MOE_EINVAL, "%s: top_k = %d must be in [1, 64]", what, (int)top_k);
  if ((int64_t)tokens * n >= kMaxPlaneBytes || (int64_t)y_rows * n >= kMaxPlaneBytes)
    return fail(FP4MOE_EINVAL, "%s: tokens x n and y_rows x n must stay below 2^31", what);
  if (tokens == 0) return ok();
  if (!pair_rows || !out || (y_rows > 0 && !y)) return fail(FP4MOE_EINVAL, "%s: NULL buffer with tokens > 0", what);
  return launched(fp4moe::launch_combine(y, y_rows, n, pair_rows, pair_weights, tokens, top_k, out, stream), what);
}

int cvt_bf16(const float* x, uint16_t* out, int64_t count, hipStream_t stream) {
  if (count < 0) return fail(FP4MOE_EINVAL, "cvt_bf16: count = %lld < 0", (long long)count);
  if (count == 0) return ok();
  if (!x || !out) return fail(FP4MOE_EINVAL, "cvt_bf16: NULL buffer with count > 0");
  return launched(fp4moe::launch_cvt_bf16(x, out, count, stream), "cvt_bf16");
}

int fp4_dequant_bf16(const uint8_t* w_packed, const uint8_t* w_scales, float scale2, int32_t kind, int32_t n,
                     int32_t k, uint16_t* out, hipStream_t stream) {
  const char* what = "fp4_dequant_bf16";
  if (n < 0) return fail(FP4MOE_EINVAL, "%s: n = %d < 0", what, (int)n);
  if (int rc = check_k(k, what)) return rc;
  if (kind != FP4MOE_NVFP4 && kind != FP4MOE_MXFP4)
    return fail(FP4MOE_EINVAL, "%s: kind = %d is neither 0 (NVFP4) nor 1 (MXFP4)", what, (int)kind);
  if ((int64_t)n * k * 2 >= kMaxPlaneBytes) return fail(FP4MOE_EINVAL, "%s: n x k bf16 values reach 2^31 bytes", what);
  if (n == 0) return ok();
  if (!w_packed || !w_scales || !out) return fail(FP4MOE_EINVAL, "%s: NULL buffer with n > 0", what);
  if (reinterpret_cast<uintptr_t>(out) & 15) return fail(FP4MOE_EINVAL, "%s: out must be 16-byte aligned", what);
  if (reinterpret_cast<uintptr_t>(w_packed) & 3) return fail(FP4MOE_EINVAL, "%s: w_packed must be 4-byte aligned", what);
  return launched(fp4moe::launch_dequant_bf16(w_packed, w_scales, scale2, kind, n, k, out, stream), what);
}

int gemm_bf16(const uint16_t* a, const uint16_t* w, float* out, int32_t m, int32_t n, int32_t k, hipStream_t stream) {
  const char* what = "gemm_bf16";
  if (m < 0 || n <= 0) return fail(FP4MOE_EINVAL, "%s: m = %d must be >= 0 and n = %d > 0", what, (int)m, (int)n);
  if (k <= 0 || k % 16 != 0) return fail(FP4MOE_EINVAL, "%s: k = %d must be a positive multiple of 16", what, (int)k);
  if ((int64_t)m * k * 2 >= kMaxPlaneBytes || (int64_t)n * k * 2 >= kMaxPlaneBytes)
    return fail(FP4MOE_EINVAL, "%s: an operand of 2^31 bytes or more", what);
  if (m == 0) return ok();
  if (!a || !w || !out) return fail(FP4MOE_EINVAL, "%s: NULL buffer with m > 0", what);
  return launched(fp4moe::launch_gemm_bf16(a, w, out, m, n, k, stream), what);
}

int act_quant_fp4(const float* x, const int32_t* skip_channels, int32_t n_skip, uint8_t* codes, uint8_t* micro,
                  float* row_scale, int32_t rows, int32_t k, int32_t two_level, hipStream_t stream) {
  const char* what = "act_quant_fp4";
  if (rows < 0) return fail(FP4MOE_EINVAL, "%s: rows = %d < 0", what, (int)rows);
  if (int rc = check_k(k, what)) return rc;
  if (n_skip < 0 || n_skip > 64) return fail(FP4MOE_EINVAL, "%s: n_skip = %d must be in [0, 64]", what, (int)n_skip);
  if (two_level != 0 && two_level != 1) return fail(FP4MOE_EINVAL, "%s: two_level must be 0 or 1", what);
  if ((int64_t)rows * k * 4 >= kMaxPlaneBytes) return fail(FP4MOE_EINVAL, "%s: x reaches 2^31 bytes", what);
  if (rows == 0) return ok();
  if (!x || !codes || !micro || !row_scale || (n_skip > 0 && !skip_channels))
    return fail(FP4MOE_EINVAL, "%s: NULL buffer with rows > 0", what);
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(codes) & 1))
    return fail(FP4MOE_EINVAL, "%s: x must be 16-byte and codes 2-byte aligned", what);
  return launched(fp4moe::launch_act_quant_fp4(x, skip_channels, n_skip, rows, k, two_level, codes, micro, row_scale,
                                               stream),
                  what);
}

int loud_channels(const float* x, int32_t rows, int32_t k, int32_t k_res, int32_t* idx, hipStream_t stream) {
  const char* what = "loud_channels";
  if (rows < 0) return fail(FP4MOE_EINVAL, "%s: rows = %d < 0", what, (int)rows);
  if (k < 1 || k > 8192) return fail(FP4MOE_EINVAL, "%s: k = %d must be in [1, 8192]", what, (int)k);
  if (k_res < 0 || k_res > 64 || k_res > k)
    return fail(FP4MOE_EINVAL, "%s: k_res = %d must be in [0, min(k, 64)]", what, (int)k_res);
  if ((int64_t)rows * k * 4 >= kMaxPlaneBytes) return fail(FP4MOE_EINVAL, "%s: x reaches 2^31 bytes", what);
  if (k_res == 0) return ok();
  if (!idx || (rows > 0 && !x)) return fail(FP4MOE_EINVAL, "%s: NULL buffer", what);
  return launched(fp4moe::launch_loud_channels(x, rows, k, k_res, idx, stream), what);
}

int w4a4_gemm(const uint8_t* a_codes, const uint8_t* a_micro, const float* a_row_scale, const uint8_t* w_packed,
              const uint8_t* w_scales, float scale2, const float* x, const int32_t* res_idx, int32_t k_res, float* out,
              int32_t g, int32_t n, int32_t k, hipStream_t stream) {
  const char* what = "w4a4_gemm";
  if (g < 0) return fail(FP4MOE_EINVAL, "%s: g = %d < 0", what, (int)g);
  if (n <= 0) return fail(FP4MOE_EINVAL, "%s: n = %d must be positive", what, (int)n);
  if (int rc = check_k(k, what)) return rc;
  if (k_res < 0 || k_res > 64) return fail(FP4MOE_EINVAL, "%s: k_res = %d must be in [0, 64]", what, (int)k_res);
  if (int rc = check_planes(g, n, k, what)) return rc;
  if ((int64_t)g * k * 4 >= kMaxPlaneBytes) return fail(FP4MOE_EINVAL, "%s: x reaches 2^31 bytes", what);
  if (g == 0) return ok();
  if (!a_codes || !a_micro || !a_row_scale || !w_packed || !w_scales || !out || (k_res > 0 && (!x || !res_idx)))
    return fail(FP4MOE_EINVAL, "%s: NULL buffer with g > 0", what);
  fp4moe::GemmArgs a{};
  a.a_codes = a_codes;
  a.a_micro = a_micro;
  a.a_row_scale = a_row_scale;
  a.a_rows = g;
  a.num_experts = 1;
  a.total_rows = g;
  a.w = w_packed;
  a.s = w_scales;
  a.scale2 = scale2;
  a.kind = FP4MOE_NVFP4;
  a.out = out;
  a.n = n;
  a.k = k;
  if (int rc = launched(fp4moe::launch_gemm_prefill(a, stream), what)) return rc;
  if (k_res == 0) return ok();
  return launched(fp4moe::launch_w4a4_residual(x, res_idx, k_res, w_packed, w_scales, scale2, out, g, n, k, stream),
                  what);
}

int fp4_expert_gemm(const uint8_t* a_codes, const float* a_scales, const uint8_t* w_packed,
                    const uint8_t* w_scales, float scale2, int32_t kind, float* out, int32_t g,
                    int32_t n, int32_t k, hipStream_t stream) {
  if (g < 0) return fail(FP4MOE_EINVAL, "fp4_expert_gemm: g = %d < 0", (int)g);
  if (n <= 0) return fail(FP4MOE_EINVAL, "fp4_expert_gemm: n = %d must be positive", (int)n);
  if (int rc = check_k(k, "fp4_expert_gemm")) return rc;
  if (!is_gemm_kind(kind))
    return fail(FP4MOE_EINVAL, "fp4_expert_gemm: kind = %d is not 0/1 (NVFP4/MXFP4) or 2/3 (swizzled)", (int)kind);
  if (g == 0) return ok();
  if (!a_codes || !a_scales || !w_packed || !w_scales || !out)
    return fail(FP4MOE_EINVAL, "fp4_expert_gemm: NULL buffer with g > 0");
  if (int rc = check_planes(g, n, k, "fp4_expert_gemm")) return rc;
  fp4moe::GemmArgs a{};
  a.a_codes = a_codes;
  a.a_scales = a_scales;
  a.a_rows = g;
  a.num_experts = 1;
  a.total_rows = g;
  a.w = w_packed;
  a.s = w_scales;
  a.scale2 = scale2;
  a.kind = kind;
  a.out = out;
  a.n = n;
  a.k = k;
  return launched(launch_gemm(a, g, 1, stream), "fp4_expert_gemm");
}

size_t fp4_grouped_gemm_workspace_size(int32_t num_experts, int32_t total_rows, int32_t n, int32_t k) {
  (void)num_experts;
  (void)total_rows;
  (void)n;
  (void)k;
  return 0;  // every grouped kernel finds its tiles from the offsets on the device
}

int fp4_grouped_gemm(const uint8_t* a_codes, const float* a_scales, const int32_t* offsets, int32_t num_experts,
                     int32_t total_rows, const uint64_t* w_ptrs, const uint64_t* s_ptrs, const int32_t* kinds,
                     const float* scale2, float* out, int32_t n, int32_t k, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  const char* what = "fp4_grouped_gemm";
  if (!workspace && workspace_bytes > 0)
    return fail(FP4MOE_EINVAL, "%s: workspace is NULL but workspace_bytes = %zu", what, workspace_bytes);
  const size_t need = fp4_grouped_gemm_workspace_size(num_experts, total_rows, n, k);
  if (workspace_bytes < need)
    return fail(FP4MOE_EINVAL, "%s: workspace of %zu bytes, %zu needed", what, workspace_bytes, need);
  return grouped_gemm(what, a_codes, a_scales, total_rows, nullptr, offsets, num_experts, total_rows, w_ptrs, s_ptrs,
                      kinds, scale2, out, n, k, stream);
}

int fp4_grouped_gemm_gather(const uint8_t* a_codes, const float* a_scales, int32_t a_rows, const int32_t* row_ids,
                            const int32_t* offsets, int32_t num_experts, int32_t total_rows, const uint64_t* w_ptrs,
                            const uint64_t* s_ptrs, const int32_t* kinds, const float* scale2, float* out, int32_t n,
                            int32_t k, hipStream_t stream) {
  return grouped_gemm("fp4_grouped_gemm_gather", a_codes, a_scales, a_rows, row_ids, offsets, num_experts, total_rows,
                      w_ptrs, s_ptrs, kinds, scale2, out, n, k, stream);
}

int fp4_grouped_gemm_swiglu_quant(const uint8_t* a_codes, const float* a_scales, int32_t a_rows,
                                  const int32_t* row_ids, const int32_t* offsets, int32_t num_experts,
                                  int32_t total_rows, const uint64_t* w_ptrs, const uint64_t* s_ptrs,
                                  const int32_t* kinds, const float* scale2, int32_t inter, int32_t k,
                                  const float* row_weights, float limit, uint8_t* h_codes, float* h_scales,
                                  float* h_out, hipStream_t stream) {
  const char* what = "fp4_grouped_gemm_swiglu_quant";
  if (a_rows < 0 || total_rows < 0)
    return fail(FP4MOE_EINVAL, "%s: a_rows = %d, total_rows = %d must be >= 0", what, (int)a_rows, (int)total_rows);
  if (num_experts <= 0) return fail(FP4MOE_EINVAL, "%s: num_experts = %d must be positive", what, (int)num_experts);
  if (inter <= 0 || inter % 128 != 0 || inter > (1 << 29))
    return fail(FP4MOE_EINVAL, "%s: inter = %d must be a positive multiple of 128 up to 2^29", what, (int)inter);
  if (int rc = check_k(k, what)) return rc;
  if (!(limit > 0.0f)) return fail(FP4MOE_EINVAL, "%s: limit must be > 0", what);
  if (!row_ids && a_rows < total_rows)
    return fail(FP4MOE_EINVAL, "%s: row_ids is NULL but a_rows = %d < total_rows = %d", what, (int)a_rows,
                (int)total_rows);
  if (total_rows == 0) return ok();
  if (!a_codes || !a_scales || !offsets || !w_ptrs || !s_ptrs || !kinds || !scale2 || !h_codes || !h_scales)
    return fail(FP4MOE_EINVAL, "%s: NULL buffer with total_rows > 0", what);
  if ((reinterpret_cast<uintptr_t>(h_codes) | reinterpret_cast<uintptr_t>(h_out)) & 15)
    return fail(FP4MOE_EINVAL, "%s: h_codes and h_out must be 16-byte aligned", what);
  if (int rc = check_planes(a_rows, 2 * inter, k, what)) return rc;
  if (int rc = debug_check_tables(what, offsets, num_experts, total_rows, row_ids, a_rows, kinds, stream)) return rc;
  fp4moe::GemmArgs a{};
  a.a_codes = a_codes;
  a.a_scales = a_scales;
  a.row_ids = row_ids;
  a.a_rows = a_rows;
  a.offsets = offsets;
  a.num_experts = num_experts;
  a.total_rows = total_rows;
  a.w_ptrs = w_ptrs;
  a.s_ptrs = s_ptrs;
  a.kinds = kinds;
  a.scale2s = scale2;
  a.n = 2 * inter;
  a.k = k;
  a.swiglu_inter = inter;
  a.swiglu_limit = limit;
  a.swiglu_row_w = row_weights;
  a.h_codes = h_codes;
  a.h_scales = h_scales;
  a.h_out = h_out;
  return launched(fp4moe::launch_gemm_prefill(a, stream), what);
}

size_t fp4_swizzled_weight_bytes(int32_t n, int32_t k) {
  if (n <= 0 || k <= 0 || k % 128 != 0) return 0;
  return (size_t)fp4moe::swizzled_weight_bytes(n, k);
}

size_t fp4_swizzled_scale_bytes(int32_t kind, int32_t n, int32_t k) {
  if (n <= 0 || k <= 0 || k % 128 != 0 || (kind != FP4MOE_NVFP4 && kind != FP4MOE_MXFP4)) return 0;
  return (size_t)fp4moe::swizzled_scale_bytes(kind, n, k);
}

int fp4_weight_swizzle(const uint8_t* w_packed, const uint8_t* w_scales, int32_t kind, int32_t n, int32_t k,
                       uint8_t* w_swz, uint8_t* s_swz, hipStream_t stream) {
  const char* what = "fp4_weight_swizzle";
  if (n <= 0) return fail(FP4MOE_EINVAL, "%s: n = %d must be positive", what, (int)n);
  if (int rc = check_k(k, what)) return rc;
  if (kind != FP4MOE_NVFP4 && kind != FP4MOE_MXFP4)
    return fail(FP4MOE_EINVAL, "%s: kind = %d is neither 0 (NVFP4) nor 1 (MXFP4)", what, (int)kind);
  if (int rc = check_planes(0, n, k, what)) return rc;
  if (!w_packed || !w_scales || !w_swz || !s_swz) return fail(FP4MOE_EINVAL, "%s: NULL buffer", what);
  if ((reinterpret_cast<uintptr_t>(w_packed) | reinterpret_cast<uintptr_t>(w_swz) |
       reinterpret_cast<uintptr_t>(s_swz)) & 15)
    return fail(FP4MOE_EINVAL, "%s: w_packed, w_swz and s_swz must be 16-byte aligned", what);
  return launched(fp4moe::launch_weight_swizzle(w_packed, w_scales, kind, n, k, w_swz, s_swz, stream), what);
}

int fp4moe_set_gemm_schedule(int32_t schedule) {
  if (schedule < FP4MOE_SCHEDULE_AUTO || schedule > FP4MOE_SCHEDULE_SPLITK)
    return fail(FP4MOE_EINVAL, "fp4moe_set_gemm_schedule: schedule = %d is not 0, 1, 2 or 3", (int)schedule);
  g_schedule.store(schedule, std::memory_order_relaxed);
  return ok();
}

int fp4moe_set_debug_checks(int32_t on) {
  if (on != 0 && on != 1) return fail(FP4MOE_EINVAL, "fp4moe_set_debug_checks: on = %d is not 0 or 1", (int)on);
  g_debug_checks.store(on, std::memory_order_relaxed);
  return ok();
}

const char* fp4moe_last_error(void) { return g_err; }

const char* fp4moe_version(void) { return "libfp4moe 0.1.0 (gfx950)"; }

}  // extern "C"
