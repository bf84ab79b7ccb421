// dg_device.h - device helpers for the gfx950 kernels: e4m3 encoding, bf16 rounding,
// FP8 MFMA wrappers and operand vector types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kQ = 128;  // scale granularity along K, and the weight block edge

// ---------------------------------------------------------------------------------
// fp32 -> OCP E4M3FN, round to nearest even, saturating at +-448, sign of zero kept.
// The format (bias 7, 3 mantissa bits, subnormals below 2^-6, max finite 448) is OCP
// E4M3FN, fixed by the 448 bound the DeepSeek-V3 repo review quotes ("Risks" 6).
// Normal range: round the fp32 pattern at mantissa bit 20 and rebias the exponent.
// Subnormal range (|y| < 2^-6): |y| * 512 is exact, and rint() rounds half to even.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  uint32_t bits = __float_as_uint(y);
  uint32_t sign = (bits >> 24) & 0x80u;
  uint32_t mag = bits & 0x7FFFFFFFu;
  uint32_t code;
  if (mag >= 0x43E00000u) {          // |y| >= 448 (and inf): saturate
    code = 0x7Eu;
  } else if (mag < 0x3C800000u) {    // |y| < 2^-6
    code = (uint32_t)__builtin_rintf(__uint_as_float(mag) * 512.0f);
  } else {
    uint32_t r = (mag + 0x7FFFFu + ((mag >> 20) & 1u)) >> 20;
    code = r - (120u << 3);            // exponent bias 127 -> 7
    code = code > 0x7Eu ? 0x7Eu : code;
  }
  return sign | code;
}

// Four fp32 values -> four e4m3 codes (byte i = code of value i) with gfx950's conversion
// instruction (v_cvt_pk_fp8_f32: OCP E4M3FN, round to nearest even). It does not saturate:
// it agrees with e4m3_encode for |y| <= 464 (below the midpoint between 448 and 480 every
// value rounds to at most 448), which callers must guarantee.
__device__ __forceinline__ uint32_t e4m3_hw_pack4(float y0, float y1, float y2, float y3) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, (int)lo, true);
}

// The smallest power of two >= v (v >= 0), and >= 2^-126, from the fp32 bits: a normal v
// with a zero mantissa is a power of two already; otherwise the exponent goes up by one.
// This is the UE8M0 (power-of-two) scale of the casts.
__device__ __forceinline__ float pow2_ceil(float v) {
  const uint32_t b = __float_as_uint(v);
  if (b < 0x00800000u) return __uint_as_float(0x00800000u);  // 0 and subnormals
  const uint32_t e = (b >> 23) + ((b & 0x007FFFFFu) ? 1u : 0u);
  return __uint_as_float(e << 23);
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite or NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// One 16x16x128 FP8 (e4m3 x e4m3) MFMA into a fresh fp32 partial. Operand lane layout:
// lane l supplies row (l & 15) of its 16-row strip and 32 K-bytes (group l >> 4); A and
// B pair byte-for-byte within a lane group, so any fixed split of the 128 K bytes over
// (group, byte) works if A and B use the same one. Output: lane l, element r holds row
// 4 * (l >> 4) + r, column l & 15.
__device__ __forceinline__ v4f mfma_f8_16x16x128(const v8i& a, const v8i& b) {
  v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

// c + 2^(ea-127) * 2^(eb-127) * (A . B) on the matrix unit (block-scaled form): ea is the
// E8M0 scale this lane supplies for its A row (l & 15), eb the one for its B column; both
// in byte 0 of the operand. The scale covers the 32 K values of the lane's group, so a
// scale shared by a whole 128-K block is the same in every lane group.
__device__ __forceinline__ v4f mfma_f8_16x16x128_scaled(const v8i& a, const v8i& b, const v4f& c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

__device__ __forceinline__ v8i cat8(const v4i& lo, const v4i& hi) {
  v8i r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Work-group index remap so that consecutively numbered logical tiles run on the same
// XCD (workgroups are dealt to the 8 XCDs round-robin; each XCD has its own L2).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t hw_id, uint32_t nwg) {
  constexpr uint32_t kXcd = 8;
  uint32_t q = nwg / kXcd, r = nwg % kXcd;
  uint32_t x = hw_id % kXcd, i = hw_id / kXcd;
  return x * q + (x < r ? x : r) + i;
}

}  // namespace dg
