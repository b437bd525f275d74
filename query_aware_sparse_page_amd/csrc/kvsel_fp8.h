// fp8 pages: OCP 8-bit floating point E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa
// bits; exponent field 0 subnormal; S.1111.111 NaN; largest finite 448) with one fp32 scale per
// (physical page, KV head) tile, a code standing for its value times the scale.
//
// Decoding uses the hardware conversion (v_cvt_pk_f32_fp8, E4M3 in the OCP encoding on gfx950);
// every E4M3 value is exactly a bf16 value, so the high half of the fp32 result is its bf16.
// Encoding (the quantizer only) is written out: round to nearest, ties to an even mantissa,
// magnitudes from 448 up saturating to 448, the sign bit kept.
// Summaries of an fp8 page are bf16, rounded outward from the dequantized extremes (lo toward
// -inf, hi toward +inf), so a page score computed from them bounds q.k over the page's keys.
#pragma once

#include "kvsel_device.h"

namespace kvsel {

constexpr float FP8_MAX = 448.0f;

// Element tag of an fp8 pool in the launch templates (one E4M3 code).
struct fp8_t {
  uint8_t bits;
};

__device__ __forceinline__ uint2 load8(const void* p) { return *reinterpret_cast<const uint2*>(p); }
typedef unsigned int u32x2_nt_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 load8_nt(const void* p) {
  const u32x2_nt_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_nt_t*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void store8(void* p, const uint2& v) { *reinterpret_cast<uint2*>(p) = v; }

// Codes 4i .. 4i+3 of one 32-bit word as fp32 (exact).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t word, float* f) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);  // bytes 0, 1
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);   // bytes 2, 3
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

// 8 codes (byte e of the little-endian pair is element e) as fp32.
__device__ __forceinline__ void fp8x8_to_f32(const uint2& c, float* f) {
  fp8x4_to_f32(c.x, f);
  fp8x4_to_f32(c.y, f + 4);
}

// 8 codes as 8 packed bf16 (the layout of unpack<bf16_t> / pack<bf16_t>), exactly.
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(const uint2& c) {
  float f[8];
  fp8x8_to_f32(c, f);
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (__float_as_uint(f[2 * i]) >> 16) | (__float_as_uint(f[2 * i + 1]) & 0xffff0000u);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// E4M3 code of y: round to nearest, ties to an even mantissa, saturating at 448 (NaN -> 0x7F).
__device__ __forceinline__ uint32_t f32_to_fp8(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (!(a == a)) return 0x7Fu;
  if (a >= FP8_MAX) return sign | 0x7Eu;
  if (a < 0.015625f) {  // below 2^-6: subnormal codes m * 2^-9, m = 0..8 (8 is the smallest normal)
    return sign | (uint32_t)rintf(a * 512.0f);
  }
  int E;
  (void)frexpf(a, &E);                        // a = m * 2^E, 0.5 <= m < 1: binade [2^(E-1), 2^E)
  float t = rintf(ldexpf(a, 4 - E));          // 8 .. 16: the value in eighths of the binade's base
  int e = E - 1 + 7;                          // exponent field
  if (t == 16.0f) {
    t = 8.0f;
    ++e;
  }
  return sign | ((uint32_t)e << 3) | ((uint32_t)t - 8u);
}

// bf16 bits of an exact fp64 value rounded toward -inf (UP = false) or +inf (UP = true).
// Truncating to fp32 and then to bf16 is truncation to bf16; an inexact value then moves one step
// away from zero when that is the requested direction.
template <bool UP>
__device__ __forceinline__ uint32_t f64_to_bf16_directed(double x) {
  uint32_t b = __float_as_uint(__double2float_rz(x)) >> 16;
  const bool exact = (double)__uint_as_float(b << 16) == x;
  const bool neg = x < 0.0;
  if (!exact && (UP ? !neg : neg)) b += 1;
  return b;
}

}  // namespace kvsel
