// device_common.h -- gfx950 device helpers shared by the libfp4moe kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4moe {

typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------- buffer loads
// Raw buffer loads through a descriptor held in SGPRs: a 32-bit byte offset per lane, and any
// access that ends past `bytes` returns zero.  Callers mark inactive lanes with kOffNone so their
// loads return zero without a branch.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOffNone = 0x80000000u;      // every buffer is < 2^31 bytes
constexpr int kRsrcWord3 = 0x00020000;         // gfx9 family: 32-bit data format, raw addressing

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4 buf_load_x4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// Non-temporal 16-byte load (cache policy NT): for data streamed once, such as the expert weight
// planes of a decode step.  Measured on MI355X: a plain streaming read kernel moves 6.2 TB/s with
// the default policy and 6.8 TB/s with NT.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ u32x4 buf_load_x4_nt(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCachePolicyNT));
}
__device__ __forceinline__ uint2 buf_load_x2(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load_u32(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load_u16(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load_u8(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// ----------------------------------------------------------------------------------- bit helpers
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// Smallest power of two >= p for a positive normal finite p: keep p if its mantissa is zero,
// otherwise clear the mantissa and add one to the exponent.
__device__ __forceinline__ float pow2_ceil_pos(float p) {
  const uint32_t u = f2u(p);
  return u2f((u & 0x007FFFFFu) ? ((u & 0x7F800000u) + 0x00800000u) : u);
}

// Exact reciprocal of a power of two 2^E with biased exponent in [1, 253].
__device__ __forceinline__ float pow2_recip(float s) {
  return u2f((254u - (f2u(s) >> 23)) << 23);
}

// The expert activation between the gate/up and the down projection (swiglu with limit), in the
// order of the f32 operations both of its kernels use: min/clamp, expf, one correctly rounded
// division, then gate * sigmoid * up * weight.
__device__ __forceinline__ float swiglu_one(float g, float u, float limit, float w) {
  g = fminf(g, limit);
  u = fminf(fmaxf(u, -limit), limit);
  return g * (1.0f / (1.0f + expf(-g))) * u * w;
}

// --------------------------------------------------------------------------- cross-lane maximum
// DPP controls (gfx9 encoding): quad permutations and row (16-lane) mirrors.
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
// ds_swizzle bit-mask mode: and 0x1F, or 0, xor 0x10 -> exchange with lane ^ 16 inside 32 lanes.
constexpr int kSwizzleXor16 = 0x401F;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return u2f((uint32_t)__builtin_amdgcn_mov_dpp((int)f2u(v), CTRL, 0xF, 0xF, false));
}

// Maximum of a non-negative value over each aligned group of 32 lanes (a half wavefront).
__device__ __forceinline__ float halfwave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
  v = fmaxf(v, u2f((uint32_t)__builtin_amdgcn_ds_swizzle((int)f2u(v), kSwizzleXor16)));
  return v;
}

// --------------------------------------------------------------------------- FP8 / FP4 -> f16
// E4M3 bytes 0,1 (HI=false) or 2,3 (HI=true) of w -> two exact f16 values.
template <bool HI>
__device__ __forceinline__ h16x2 e4m3x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Eight E4M3 bytes (two dwords, byte order = element order) -> f16x8 operand.
__device__ __forceinline__ h16x8 e4m3x8_to_f16(uint32_t lo, uint32_t hi) {
  const h16x2 a = e4m3x2_to_f16<false>(lo), b = e4m3x2_to_f16<true>(lo);
  const h16x2 c = e4m3x2_to_f16<false>(hi), d = e4m3x2_to_f16<true>(hi);
  return h16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight E2M1 nibbles (one dword, low nibble first) times one f16 scale -> f16x8 operand.  The
// hardware conversion only applies a scale's exponent, so it runs with scale 1 and the E4M3 weight
// scale (up to 4 significant bits) is applied with packed f16 multiplies: an E2M1 value times an
// E4M3 value has at most 6 significant bits and lies in [2^-10, 2688], so every product is exact.
__device__ __forceinline__ h16x8 e2m1x8_scaled_f16(uint32_t w, _Float16 s) {
  const h16x2 ss = {s, s};
  const h16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const h16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const h16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const h16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  return h16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// --------------------------------------------------------------------------- FP8 / FP4 -> bf16
// Eight E4M3 bytes (two dwords, byte order = element order) -> exact bf16x8 operand.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight E2M1 nibbles (one dword, low nibble first) times a power of two -> bf16x8.  The hardware
// conversion applies the exponent field of `pow2` (an E8M0 scale placed in the f32 exponent bits),
// so the result is exact.
__device__ __forceinline__ bf16x8 e2m1x8_pow2_bf16(uint32_t w, float pow2) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, pow2, 0);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, pow2, 1);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, pow2, 2);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, pow2, 3);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// ------------------------------------------------------------------------------ matrix cores
// 16x16x32 f16 MFMA.  Lane l holds A row l%16 (B column l%16) for k = 8*(l/16) .. +8; the f32
// result holds column l%16, rows 4*(l/16) .. +4.
__device__ __forceinline__ f32x4 mfma16x16x32_f16(h16x8 a, h16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA, same lane layout as the f16 one.
__device__ __forceinline__ f32x4 mfma16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace fp4moe
