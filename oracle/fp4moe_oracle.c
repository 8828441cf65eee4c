/*
 * fp4moe_oracle.c -- plain, slow CPU oracle for the FP8-activation x block-scaled FP4 expert GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load this library.  The product path (the HIP library) never calls it, shares no code,
 * header, table or helper with it, and must fail loudly instead of falling back to it.
 *
 * Sources (the pages this oracle is written from; cited by page title and item):
 *   [GATE]   memra-engine 0.98.0, src/bin/dsv4_native_gemm_gate.rs -- `quant_rows` (act-quant),
 *            `ExpertRaw` (weight layout), `f64_ref` (f64 reference of the quantized GEMM),
 *            comparison 2 in the module doc and in `main` (the f32 error model).
 *   [CHECK]  memra-engine 0.71.0, src/bin/kernel_check.rs -- F8-E4M3 matvec section, the CPU e4m3
 *            decode closure (sign, 4-bit exponent with bias 7, 3-bit mantissa, subnormals, NaN);
 *            f16g grouped GEMM section (CSR row offsets per expert).
 *   [QWEN]   memra-engine 0.125.0, src/bin/qwen4exp_gpu_gate.rs -- NVFP4 synthetic checkpoint rows;
 *            the device-router arm (softmax top-k over router logits, ids and order exact, ties).
 *   [GATE] also supplies the expert activation between the projections: the swiglu_limit
 *            saturation cell (its clamp math and its swiglu call, whose last pointer argument is
 *            an optional per-row weight).
 *
 * Readings where the pages are silent (each is listed with its reason in the design notes):
 *   - E2M1 values: the pages import a table without printing it; the OCP MX E2M1 grid
 *     {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign bit is used (8 magnitudes, maximum 6).
 *   - E8M0: 2^(c-127) for c in 0..254, c = 255 is NaN.
 *   - f32 -> E4M3 encode: round to nearest, ties to even mantissa, subnormal spacing 2^-9 down
 *     to zero, sign kept on zero, saturating at 448.
 *   - pow2_ceil(p): the smallest power of two >= p (an exact power of two maps to itself).
 *
 * Precision: the act-quant follows the page in f32 arithmetic; the GEMM accumulates in f64 in
 * ascending k, every product being exact in f64.  Build with -O2 -ffp-contract=off and no
 * fast-math, so that each f32 operation is one IEEE operation.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------------------------------------
 * Element decoders
 * ------------------------------------------------------------------------------------------- */

/* E2M1 (FP4) value of a 4-bit code [GATE: the imported E2M1 table, indexed by nibble].
 * Closed form of the OCP grid: exponent field e = bits 2..1, mantissa m = bit 0;
 * e == 0 is the subnormal 0.5*m, otherwise (1 + m/2) * 2^(e-1); bit 3 is the sign. */
double or_e2m1_value(unsigned code) {
    unsigned e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : (1.0 + 0.5 * (double)m) * ldexp(1.0, (int)e - 1);
    return (code & 8u) ? -mag : mag;
}

/* E4M3 (FP8) value of a byte [CHECK: CPU e4m3 decode]: sign bit 7, exponent bits 6..3 with
 * bias 7, mantissa bits 2..0; exponent 0 is subnormal m * 2^-9; exponent 15 with mantissa 7 is
 * NaN; everything else is (1 + m/8) * 2^(e-7). */
double or_e4m3_value(unsigned byte) {
    unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
    double v;
    if (e == 0)
        v = (double)m * ldexp(1.0, -9);
    else if (e == 15 && m == 7)
        return NAN;
    else
        v = (1.0 + (double)m / 8.0) * ldexp(1.0, (int)e - 7);
    return s ? -v : v;
}

/* E8M0 value of a byte [GATE: the imported e8m0_to_f32]: a pure biased exponent, 2^(c-127);
 * c = 255 is NaN. */
double or_e8m0_value(unsigned byte) {
    if (byte == 255u) return NAN;
    return ldexp(1.0, (int)byte - 127);
}

/* f32 -> E4M3 byte [GATE: the imported f32_to_fp8_e4m3, applied to values already clamped to
 * +-448].  Round to nearest, ties to the even code (code LSB == mantissa LSB), magnitudes above
 * 448 saturate to 448, and the sign bit of x is kept even when the magnitude rounds to zero.
 * Found by a binary search over the 127 finite non-negative codes, which increase with the code,
 * then one exact comparison with the midpoint of the two neighbours. */
unsigned or_e4m3_encode(float x) {
    uint32_t bits;
    memcpy(&bits, &x, sizeof bits);
    unsigned sign = (bits >> 31) & 1u;
    double a = fabs((double)x);
    unsigned r;
    if (a >= 448.0) {
        r = 0x7Eu;
    } else {
        unsigned lo = 0, hi = 0x7Eu; /* invariant: value(lo) <= a < value(hi) */
        while (hi - lo > 1) {
            unsigned mid = (lo + hi) / 2;
            if (or_e4m3_value(mid) <= a) lo = mid; else hi = mid;
        }
        double mid = 0.5 * (or_e4m3_value(lo) + or_e4m3_value(hi)); /* exact in f64 */
        if (a < mid) r = lo;
        else if (a > mid) r = hi;
        else r = (lo & 1u) ? hi : lo;
    }
    return (sign << 7) | r;
}

void or_e4m3_encode_many(const float* x, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)or_e4m3_encode(x[i]);
}

/* ---------------------------------------------------------------------------------------------
 * Activation quantization [GATE: quant_rows]
 * ------------------------------------------------------------------------------------------- */

/* Smallest power of two >= p, for finite p > 0 (reading of the imported pow2_ceil). */
float or_pow2_ceil(float p) {
    int e;
    float f = frexpf(p, &e); /* p = f * 2^e, f in [0.5, 1) */
    if (f == 0.5f) return p;
    return ldexpf(1.0f, e);
}

/* The step of one block of 128 consecutive activations [GATE: quant_rows, the activation
 * quantizer]: the largest magnitude in the block, never below the floor 1e-4 (the f32 literal),
 * times 1/448 rounded once to f32, in one f32 multiply, rounded up to a power of two. */
static float block_step(const float* v) {
    float peak = 1e-4f;
    for (int i = 0; i < 128; ++i) {
        float m = fabsf(v[i]);
        if (m > peak) peak = m;
    }
    return or_pow2_ceil(peak * (float)(1.0 / 448.0));
}

/* Activation quantization by its definition: every element of a row is divided by the step of the
 * 128-column block it sits in, clamped to +-448 and encoded as E4M3; the steps are the scales.
 * x: f32 [rows, k] row-major; codes: u8 [rows, k]; scales: f32 [rows, k/128].  k % 128 == 0. */
void or_act_quant(const float* x, int64_t rows, int64_t k, uint8_t* codes, float* scales) {
    const int64_t nblk = k / 128;
    for (int64_t row = 0; row < rows; ++row) {
        const float* xr = x + row * k;
        float* step = scales + row * nblk;
        for (int64_t b = 0; b < nblk; ++b) step[b] = block_step(xr + 128 * b);
        for (int64_t col = 0; col < k; ++col) {
            float q = xr[col] / step[col / 128];
            if (q > 448.0f) q = 448.0f;
            else if (q < -448.0f) q = -448.0f;
            codes[row * k + col] = (uint8_t)or_e4m3_encode(q);
        }
    }
}

/* ---------------------------------------------------------------------------------------------
 * Quantized GEMM, f64 route [GATE: ExpertRaw, f64_ref]
 * ------------------------------------------------------------------------------------------- */

enum { OR_NVFP4 = 0, OR_MXFP4 = 1 };

/* Weight scale of column c, group j: NVFP4 = f32(E4M3(S) * scale2) rounded once to f32,
 * MXFP4 = E8M0(S) [GATE: the ws match in f64_ref]. */
static double weight_scale(int kind, uint8_t sbyte, float scale2) {
    if (kind == OR_NVFP4) {
        float ws = (float)or_e4m3_value(sbyte) * scale2;
        return (double)ws;
    }
    return (double)(float)or_e8m0_value(sbyte);
}

/* One output of one expert, the defining sum written out term by term [GATE: f64_ref]:
 *   out[r, c] = sum over t < k of  E4M3(A[r, t]) * E2M1(W[c, t]) * (ws(c, t / gs) * as[r, t / 128])
 * where W[c, t] is the low nibble of byte t/2 of column c's row for even t and the high nibble for
 * odd t, ws is the weight scale of the group holding t (gs = 16 NVFP4, 32 MXFP4) and as the
 * activation scale of the 128-block holding t.  Every term is formed in f64 (exact for the
 * power-of-two activation scales act-quant writes) and the terms are added in ascending t; `mag`
 * is the same sum of |term|, the scale of the f32 error bound. */
static void dot_one(const uint8_t* A, const float* AS, const uint8_t* W, const uint8_t* S, float scale2,
                    int kind, int64_t k, int64_t r, int64_t c, double* sum_out, double* mag_out) {
    const int64_t gs = (kind == OR_NVFP4) ? 16 : 32;
    double sum = 0.0, mag = 0.0;
    for (int64_t t = 0; t < k; ++t) {
        const double act = or_e4m3_value(A[r * k + t]);
        const uint8_t pair = W[c * (k / 2) + t / 2];
        const double wt = or_e2m1_value((t % 2 == 0) ? (pair & 0x0Fu) : (unsigned)(pair >> 4));
        const double scale = weight_scale(kind, S[c * (k / gs) + t / gs], scale2) * (double)AS[r * (k / 128) + t / 128];
        const double term = act * wt * scale;
        sum += term;
        mag += fabs(term);
    }
    *sum_out = sum;
    *mag_out = mag;
}

typedef struct {
    const uint8_t* a_codes; const float* a_scales; const uint8_t* w; const uint8_t* s;
    float scale2; int kind; int64_t g, n, k; double* out; double* absp;
    int64_t r0, r1;
} gemm_job;

static void* gemm_rows(void* p) {
    gemm_job* j = (gemm_job*)p;
    for (int64_t r = j->r0; r < j->r1; ++r)
        for (int64_t c = 0; c < j->n; ++c)
            dot_one(j->a_codes, j->a_scales, j->w, j->s, j->scale2, j->kind, j->k, r, c,
                     &j->out[r * j->n + c], &j->absp[r * j->n + c]);
    return NULL;
}

/* Full single-expert GEMM: out, absp f64 [g, n].  Rows are split over nthreads threads; each
 * output is computed by exactly one thread with the same ascending-k sum. */
void or_expert_gemm(const uint8_t* a_codes, const float* a_scales, const uint8_t* w,
                    const uint8_t* s, float scale2, int kind, int64_t g, int64_t n, int64_t k,
                    double* out, double* absp, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > g) nthreads = (int)(g > 0 ? g : 1);
    pthread_t th[256];
    gemm_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        gemm_job jb = {a_codes, a_scales, w, s, scale2, kind, g, n, k, out, absp,
                       g * t / nthreads, g * (t + 1) / nthreads};
        jobs[t] = jb;
    }
    if (nthreads == 1) { gemm_rows(&jobs[0]); return; }
    for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, gemm_rows, &jobs[t]);
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* Selected outputs of a single expert: for each i, (rows[i], cols[i]) -> out[i], absp[i]. */
void or_expert_gemm_points(const uint8_t* a_codes, const float* a_scales, const uint8_t* w,
                           const uint8_t* s, float scale2, int kind, int64_t k,
                           const int64_t* rows, const int64_t* cols, int64_t count,
                           double* out, double* absp) {
    for (int64_t i = 0; i < count; ++i)
        dot_one(a_codes, a_scales, w, s, scale2, kind, k, rows[i], cols[i], &out[i], &absp[i]);
}

/* ---------------------------------------------------------------------------------------------
 * Grouped GEMM: rows packed per expert [CHECK: f16g grouped GEMM, CSR offsets; GATE: f64_ref per
 * expert].  Expert e owns rows offsets[e] .. offsets[e+1]-1 of A and of out, and multiplies them
 * by its own planes w_ptrs[e], s_ptrs[e] (host addresses) in format kinds[e] with scale2[e].
 * ------------------------------------------------------------------------------------------- */

typedef struct {
    const uint8_t* a_codes; const float* a_scales; const int32_t* offsets; int32_t num_experts;
    const uint8_t* const* w_ptrs; const uint8_t* const* s_ptrs; const int32_t* kinds;
    const float* scale2; int64_t n, k; double* out; double* absp;
    int64_t row0, r0, r1;
} grouped_job;

static int32_t expert_of_row(const int32_t* offsets, int32_t num_experts, int64_t row) {
    for (int32_t e = 0; e < num_experts; ++e)
        if (row >= offsets[e] && row < offsets[e + 1]) return e;
    return -1;
}

static void* grouped_rows(void* p) {
    grouped_job* j = (grouped_job*)p;
    const int64_t kq = j->k / 128;
    for (int64_t r = j->r0; r < j->r1; ++r) {
        int32_t e = expert_of_row(j->offsets, j->num_experts, r);
        if (e < 0) continue;
        for (int64_t c = 0; c < j->n; ++c) {
            /* dot_one indexes A and as by row: pass the row's own base with r = 0. */
            dot_one(j->a_codes + r * j->k, j->a_scales + r * kq, j->w_ptrs[e], j->s_ptrs[e],
                     j->scale2[e], j->kinds[e], j->k, 0, c, &j->out[(r - j->row0) * j->n + c],
                     &j->absp[(r - j->row0) * j->n + c]);
        }
    }
    return NULL;
}

/* Grouped GEMM over the rows [row0, row1) of the packed activation matrix: out, absp f64
 * [row1-row0, n] (row-major, first row = row0).  Rows outside every segment are left untouched. */
void or_grouped_gemm(const uint8_t* a_codes, const float* a_scales, const int32_t* offsets,
                     int32_t num_experts, const uint8_t* const* w_ptrs,
                     const uint8_t* const* s_ptrs, const int32_t* kinds, const float* scale2,
                     int64_t n, int64_t k, int64_t row0, int64_t row1, double* out, double* absp,
                     int nthreads) {
    const int64_t rows = row1 - row0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > rows) nthreads = (int)(rows > 0 ? rows : 1);
    pthread_t th[256];
    grouped_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        grouped_job jb = {a_codes, a_scales, offsets, num_experts, w_ptrs, s_ptrs, kinds, scale2,
                          n, k, out, absp, row0,
                          row0 + rows * t / nthreads, row0 + rows * (t + 1) / nthreads};
        jobs[t] = jb;
    }
    if (nthreads == 1) { grouped_rows(&jobs[0]); return; }
    for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, grouped_rows, &jobs[t]);
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* Selected outputs of the grouped GEMM: (rows[i] in the packed order, cols[i]).  A row outside
 * every segment yields NaN. */
void or_grouped_gemm_points(const uint8_t* a_codes, const float* a_scales, const int32_t* offsets,
                            int32_t num_experts, const uint8_t* const* w_ptrs,
                            const uint8_t* const* s_ptrs, const int32_t* kinds,
                            const float* scale2, int64_t k, const int64_t* rows,
                            const int64_t* cols, int64_t count, double* out, double* absp) {
    const int64_t kq = k / 128;
    for (int64_t i = 0; i < count; ++i) {
        int32_t e = expert_of_row(offsets, num_experts, rows[i]);
        if (e < 0) { out[i] = NAN; absp[i] = NAN; continue; }
        dot_one(a_codes + rows[i] * k, a_scales + rows[i] * kq, w_ptrs[e], s_ptrs[e], scale2[e],
                 kinds[e], k, 0, cols[i], &out[i], &absp[i]);
    }
}

/* ---------------------------------------------------------------------------------------------
 * Dequantize-then-dense route [GATE: comparison 3, the bf16-dequant rung, computed here in f64]
 * ------------------------------------------------------------------------------------------- */

/* Wd[c,k] = E2M1(W[c,k]) * ws[c, k/gs], f64 [n, k]. */
void or_dequant_weights(const uint8_t* w, const uint8_t* s, float scale2, int kind, int64_t n,
                        int64_t k, double* wd) {
    const int64_t gs = (kind == OR_NVFP4) ? 16 : 32;
    for (int64_t c = 0; c < n; ++c)
        for (int64_t kk = 0; kk < k; ++kk) {
            uint8_t byte = w[c * (k / 2) + (kk >> 1)];
            unsigned code = (kk & 1) ? (byte >> 4) : (byte & 0x0Fu);
            wd[c * k + kk] = or_e2m1_value(code) * weight_scale(kind, s[c * (k / gs) + kk / gs], scale2);
        }
}

/* Ad[r,k] = E4M3(A[r,k]) * as[r, k/128], f64 [g, k]. */
void or_dequant_acts(const uint8_t* a_codes, const float* a_scales, int64_t g, int64_t k,
                     double* ad) {
    for (int64_t r = 0; r < g; ++r)
        for (int64_t kk = 0; kk < k; ++kk)
            ad[r * k + kk] = or_e4m3_value(a_codes[r * k + kk]) * (double)a_scales[r * (k / 128) + kk / 128];
}

/* ---------------------------------------------------------------------------------------------
 * Expert activation between the gate/up and the down projection [GATE: the swiglu_limit
 * saturation cell -- its clamp math and its swiglu call]
 * ------------------------------------------------------------------------------------------- */

/* h[r, i] = silu(min(g, limit)) * clamp(u, -limit, limit) * w[r], computed in f64, where
 * g = gu[r, i] and u = gu[r, inter + i] (gu f32 [rows, 2*inter]: the fused gate/up GEMM output,
 * gate columns first), silu(t) = t / (1 + exp(-t)), and w[r] = 1 when w is NULL.  The gate is
 * clamped from above only and the up projection on both sides, both before the product.  The
 * routing weight is a per-row factor applied before the result is quantized again. */
void or_swiglu(const float* gu, int64_t rows, int64_t inter, const float* w, float limit, double* h) {
    const double lim = (double)limit;
    for (int64_t r = 0; r < rows; ++r) {
        const double wr = w ? (double)w[r] : 1.0;
        const float* gate = gu + r * 2 * inter;
        const float* up = gate + inter;
        for (int64_t i = 0; i < inter; ++i) {
            double g = (double)gate[i];
            double u = (double)up[i];
            if (g > lim) g = lim;
            if (u > lim) u = lim;
            if (u < -lim) u = -lim;
            h[r * inter + i] = g / (1.0 + exp(-g)) * u * wr;
        }
    }
}

/* ---------------------------------------------------------------------------------------------
 * Routing around the grouped GEMM [QWEN: the device-router arm -- softmax top-k over the router
 * logits, selected ids and their emitted order exact, weights to a few ulp, tie batteries of
 * duplicates straddling the cut, all-equal rows and underflow; CHECK: f16g grouped GEMM section --
 * routed rows packed per expert, CSR offsets].  Readings where the pages are silent:
 *   - selection is on the logits (softmax is strictly increasing, so this is the top-k of the exact
 *     probabilities, with no ties created by rounding or underflow of the probabilities);
 *   - a logit ranks above another when it is larger; equal logits (+0 and -0 are equal) rank by
 *     the lower expert id; NaN ranks below every number, NaNs among themselves by id;
 *   - experts are emitted best first;
 *   - weight = exp(l - m) / sum over all experts of exp(l' - m), m the largest logit (the softmax
 *     probability of the selected expert); with `normalize`, the sum runs over the k selected
 *     experts only (the probabilities renormalized over the selection);
 *   - pairs (t, j) are packed per expert in ascending expert id, and inside one expert in
 *     ascending (t, j) order, i.e. ascending token order; ids outside [0, E) are dropped;
 *   - the combine sums, for each token, weight * expert output over its k pairs.
 * ------------------------------------------------------------------------------------------- */

/* 1 when logit a of expert ia ranks above logit b of expert ib. */
static int ranks_above(float a, int64_t ia, float b, int64_t ib) {
    const int na = isnan(a), nb = isnan(b);
    if (na || nb) return (na && nb) ? ia < ib : nb;
    if (a != b) return a > b;
    return ia < ib;
}

/* ids[t, j]: the j-th best expert of token t; weights[t, j]: its softmax weight in f64.
 * logits f32 [tokens, experts]; ids int32 and weights f64 [tokens, top_k]; taken: scratch of
 * `experts` bytes. */
void or_route_topk(const float* logits, int64_t tokens, int64_t experts, int64_t top_k,
                   int normalize, uint8_t* taken, int32_t* ids, double* weights) {
    for (int64_t t = 0; t < tokens; ++t) {
        const float* l = logits + t * experts;
        memset(taken, 0, (size_t)experts);
        for (int64_t j = 0; j < top_k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < experts; ++e)
                if (!taken[e] && (best < 0 || ranks_above(l[e], e, l[best], best))) best = e;
            taken[best] = 1;
            ids[t * top_k + j] = (int32_t)best;
        }
        /* softmax over every expert; NaN in, NaN out, and an infinite maximum gives inf - inf */
        double m = -INFINITY;
        int any_nan = 0;
        for (int64_t e = 0; e < experts; ++e) {
            if (isnan(l[e])) any_nan = 1;
            else if ((double)l[e] > m) m = (double)l[e];
        }
        double denom = 0.0;
        if (normalize) {
            for (int64_t j = 0; j < top_k; ++j) denom += exp((double)l[ids[t * top_k + j]] - m);
        } else {
            for (int64_t e = 0; e < experts; ++e) denom += exp((double)l[e] - m);
        }
        if (any_nan) denom = NAN;
        for (int64_t j = 0; j < top_k; ++j)
            weights[t * top_k + j] = exp((double)l[ids[t * top_k + j]] - m) / denom;
    }
}

/* Packs the pairs p = t * top_k + j per expert.  offsets int32 [experts + 1]; row_ids int32
 * [pairs]: token of each packed row; pair_rows int32 [pairs]: packed row of each pair, -1 when
 * the pair's id is outside [0, experts); row_w f32 [pairs] (optional): w[p] moved to its row.
 * Rows past offsets[experts] are left untouched. */
void or_route_pack(const int32_t* ids, const float* w, int64_t tokens, int64_t top_k,
                   int64_t experts, int32_t* offsets, int32_t* row_ids, int32_t* pair_rows,
                   float* row_w) {
    const int64_t pairs = tokens * top_k;
    for (int64_t p = 0; p < pairs; ++p) pair_rows[p] = -1;
    int64_t r = 0;
    for (int64_t e = 0; e < experts; ++e) {
        offsets[e] = (int32_t)r;
        for (int64_t p = 0; p < pairs; ++p) {
            if (ids[p] != e) continue;
            row_ids[r] = (int32_t)(p / top_k);
            pair_rows[p] = (int32_t)r;
            if (row_w) row_w[r] = w[p];
            ++r;
        }
    }
    offsets[experts] = (int32_t)r;
}

/* out[t, c] = sum over j of w[t, j] * y[pair_rows[t, j], c] in f64 (w = 1 when NULL), and
 * abs_out[t, c] the same sum of magnitudes.  Pairs with pair_rows < 0 are skipped; a row index
 * at or past y_rows makes the token's outputs NaN. */
void or_combine(const float* y, int64_t y_rows, int64_t n, const int32_t* pair_rows,
                const float* w, int64_t tokens, int64_t top_k, double* out, double* abs_out) {
    for (int64_t t = 0; t < tokens; ++t)
        for (int64_t c = 0; c < n; ++c) {
            double s = 0.0, a = 0.0;
            for (int64_t j = 0; j < top_k; ++j) {
                const int64_t p = t * top_k + j;
                const int64_t r = pair_rows[p];
                if (r < 0) continue;
                if (r >= y_rows) { s = NAN; a = NAN; break; }
                const double term = (w ? (double)w[p] : 1.0) * (double)y[r * n + c];
                s += term;
                a += fabs(term);
            }
            out[t * n + c] = s;
            abs_out[t * n + c] = a;
        }
}

/* out_codes[p] = codes[row_ids[p]] and out_scales[p] = scales[row_ids[p]] row by row (k code
 * bytes and k/128 scales per row); a row id outside [0, a_rows) gives code bytes 0 and NaN
 * scales. */
void or_gather_rows(const uint8_t* codes, const float* scales, int64_t a_rows, int64_t k,
                    const int32_t* row_ids, int64_t rows, uint8_t* out_codes, float* out_scales) {
    const int64_t nq = k / 128;
    for (int64_t p = 0; p < rows; ++p) {
        const int64_t r = row_ids[p];
        const int ok = r >= 0 && r < a_rows;
        for (int64_t i = 0; i < k; ++i) out_codes[p * k + i] = ok ? codes[r * k + i] : 0;
        for (int64_t q = 0; q < nq; ++q) out_scales[p * nq + q] = ok ? scales[r * nq + q] : NAN;
    }
}

/* ---------------------------------------------------------------------------------------------
 * The bf16-dequant rung [GATE: comparison 3 -- the unquantized activations converted to bf16, the
 * expert weights dequantized to bf16, a bf16 GEMM with f32 output; the class shift of the native
 * path against it].  Readings where the page is silent (it prints the calls, not the kernels):
 *   - f32 -> bf16 rounds to nearest, ties to even; NaN stays NaN (sign and top payload bits kept,
 *     quiet bit set);
 *   - a weight's rung value is the f32 product E2M1 x ws (ws as in the GEMM), rounded to bf16; a
 *     NaN scale gives the canonical quiet NaN 0x7FC0 (the sign and payload of a NaN produced by
 *     arithmetic are not fixed by IEEE 754);
 *   - the bf16 GEMM sums the exact products of the bf16 values (here in f64).
 * ------------------------------------------------------------------------------------------- */

uint16_t or_bf16_bits(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if (isnan(x)) return (uint16_t)((u >> 16) | 0x0040u);
    const uint32_t lower = u & 0xFFFFu, upper = u >> 16;
    /* round to nearest; on an exact tie keep the even upper half */
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) return (uint16_t)(upper + 1u);
    return (uint16_t)upper;
}

double or_bf16_value(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

void or_cvt_bf16(const float* x, int64_t count, uint16_t* out) {
    for (int64_t i = 0; i < count; ++i) out[i] = or_bf16_bits(x[i]);
}

void or_dequant_bf16(const uint8_t* w, const uint8_t* s, float scale2, int kind, int64_t n, int64_t k,
                     uint16_t* out) {
    const int64_t gs = (kind == OR_NVFP4) ? 16 : 32;
    for (int64_t c = 0; c < n; ++c)
        for (int64_t kk = 0; kk < k; ++kk) {
            const uint8_t byte = w[c * (k / 2) + (kk >> 1)];
            const unsigned code = (kk & 1) ? (byte >> 4) : (byte & 0x0Fu);
            const float ws = (float)weight_scale(kind, s[c * (k / gs) + kk / gs], scale2);
            const float v = (float)or_e2m1_value(code) * ws;
            out[c * k + kk] = isnan(v) ? 0x7FC0u : or_bf16_bits(v);
        }
}

/* out[r, c] = sum over k of bf16(a[r, k]) * bf16(w[c, k]) in f64 (every product exact), and abs_out
 * the sum of magnitudes. */
void or_gemm_bf16(const uint16_t* a, const uint16_t* w, int64_t m, int64_t n, int64_t k, double* out,
                  double* abs_out) {
    for (int64_t r = 0; r < m; ++r)
        for (int64_t c = 0; c < n; ++c) {
            double acc = 0.0, mag = 0.0;
            for (int64_t kk = 0; kk < k; ++kk) {
                const double p = or_bf16_value(a[r * k + kk]) * or_bf16_value(w[c * k + kk]);
                acc += p;
                mag += fabs(p);
            }
            out[r * n + c] = acc;
            abs_out[r * n + c] = mag;
        }
}

/* ---------------------------------------------------------------------------------------------
 * W4A4 NVFP4 variant [CHECK: the NVFP4 MMQ W4A4 arms -- E2M1 activations with a two-level scale
 * (a per-token row scale from the row amax, then a UE4M3 micro-scale per 16-element sub-block of
 * amax_sub / 6), the sub-block-only quantizer it replaced, the DYNAMIC-RANGE arm (tokens scaled by
 * decades) and the RESIDUAL-CHANNEL arm (the k loudest channels kept out of the E2M1 path and added
 * back exactly)].  Lossy: the pages hold it to informational relative errors and two hard
 * comparisons.  Readings where the pages are silent:
 *   - E2M1 values are the OCP grid (as for the weights); the micro-scale is an unsigned E4M3 byte;
 *   - row scale rs = amax_row / 2688 (6 x 448: the largest sub-block then gets micro-scale 448),
 *     rs = 1 without the row level or for an all-zero row;
 *   - micro-scale = E4M3 encoding (round to nearest even) of (amax_sub / rs) / 6 clamped to
 *     [2^-9, 448] -- the smallest and largest UE4M3 values, the clamps the pages speak of -- and 0
 *     for an all-zero sub-block;
 *   - code = E2M1 encoding (round to nearest, ties to the even code, saturating at 6) of
 *     (x / rs) / micro, 0 when the micro-scale decodes to 0; each operation one f32 operation;
 *   - loudest channels: by the largest |x| over all tokens, ties to the lower index.
 * ------------------------------------------------------------------------------------------- */

/* E2M1 code of a finite f32 value: nearest grid point, ties to the even code, magnitude capped at 6,
 * sign bit 3 (kept also when the magnitude rounds to 0). */
unsigned or_e2m1_encode(float v) {
    const double a = fabs((double)v);
    unsigned best = 7;
    if (a < 6.0) {
        unsigned lo = 0;
        while (lo < 7 && or_e2m1_value(lo + 1) <= a) ++lo;      /* value(lo) <= a < value(lo + 1) */
        const double mid = 0.5 * (or_e2m1_value(lo) + or_e2m1_value(lo + 1));
        best = a < mid ? lo : (a > mid ? lo + 1 : ((lo & 1u) ? lo + 1 : lo));
    }
    return (signbit(v) ? 8u : 0u) | best;
}

void or_act_quant_fp4(const float* x, int64_t rows, int64_t k, int two_level, uint8_t* codes,
                      uint8_t* micro, float* row_scale) {
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * k;
        float amax = 0.0f;
        for (int64_t i = 0; i < k; ++i) amax = fmaxf(amax, fabsf(xr[i]));
        const float rs = (two_level && amax > 0.0f) ? amax / 2688.0f : 1.0f;
        row_scale[r] = rs;
        for (int64_t g = 0; g < k / 16; ++g) {
            float asub = 0.0f;
            for (int64_t i = 0; i < 16; ++i) asub = fmaxf(asub, fabsf(xr[16 * g + i]));
            const float t = asub / rs;
            const float want = t / 6.0f;
            const unsigned mb = want > 0.0f ? or_e4m3_encode(fminf(fmaxf(want, 0x1p-9f), 448.0f)) & 0x7Fu : 0u;
            micro[r * (k / 16) + g] = (uint8_t)mb;
            const float dec = (float)or_e4m3_value(mb);
            for (int64_t i = 0; i < 16; i += 2) {
                unsigned c[2];
                for (int h = 0; h < 2; ++h) {
                    const float y = xr[16 * g + i + h] / rs;
                    c[h] = dec > 0.0f ? or_e2m1_encode(y / dec) : 0u;
                }
                codes[r * (k / 2) + (16 * g + i) / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
}

/* Dequantized W4A4 activations, f64 [rows, k]: rs * micro * E2M1(code). */
void or_dequant_acts_fp4(const uint8_t* codes, const uint8_t* micro, const float* row_scale, int64_t rows,
                         int64_t k, double* out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t i = 0; i < k; ++i) {
            const uint8_t byte = codes[r * (k / 2) + i / 2];
            const unsigned code = (i & 1) ? (byte >> 4) : (byte & 0x0Fu);
            out[r * k + i] = (double)row_scale[r] * or_e4m3_value(micro[r * (k / 16) + i / 16]) *
                             or_e2m1_value(code);
        }
}

/* The k_res loudest channels (largest max over tokens of |x|, ties to the lower index), in that
 * order. */
void or_loud_channels(const float* x, int64_t rows, int64_t k, int64_t k_res, uint8_t* taken, int32_t* idx) {
    memset(taken, 0, (size_t)k);
    for (int64_t j = 0; j < k_res; ++j) {
        int64_t best = -1;
        float best_v = -1.0f;
        for (int64_t c = 0; c < k; ++c) {
            if (taken[c]) continue;
            float m = 0.0f;
            for (int64_t r = 0; r < rows; ++r) m = fmaxf(m, fabsf(x[r * k + c]));
            if (m > best_v) { best_v = m; best = c; }
        }
        taken[best] = 1;
        idx[j] = (int32_t)best;
    }
}

/* W4A4 GEMM in f64 on the quantized operands: out[r, c] = sum_k A(r, k) W(c, k) with A the
 * dequantized activations above and W = E2M1 x ws (NVFP4, ws = f32(E4M3 x scale2)); plus, when
 * k_res > 0, the exact contribution of the kept channels: sum_j x[r, idx_j] W(c, idx_j) (those
 * channels must be zero in the quantized activations).  abs_out: the sum of magnitudes. */
void or_w4a4_gemm(const uint8_t* a_codes, const uint8_t* a_micro, const float* a_rs, const uint8_t* w,
                  const uint8_t* s, float scale2, int64_t g, int64_t n, int64_t k, const float* x,
                  const int32_t* idx, int64_t k_res, double* ad_scratch, double* wd_scratch, double* out,
                  double* abs_out) {
    or_dequant_acts_fp4(a_codes, a_micro, a_rs, g, k, ad_scratch);
    or_dequant_weights(w, s, scale2, OR_NVFP4, n, k, wd_scratch);
    for (int64_t r = 0; r < g; ++r)
        for (int64_t c = 0; c < n; ++c) {
            double acc = 0.0, mag = 0.0;
            for (int64_t i = 0; i < k; ++i) {
                const double p = ad_scratch[r * k + i] * wd_scratch[c * k + i];
                acc += p;
                mag += fabs(p);
            }
            for (int64_t j = 0; j < k_res; ++j) {
                const double p = (double)x[r * k + idx[j]] * wd_scratch[c * k + idx[j]];
                acc += p;
                mag += fabs(p);
            }
            out[r * n + c] = acc;
            abs_out[r * n + c] = mag;
        }
}
