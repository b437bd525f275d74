// Device helpers shared by the kvsel kernels (gfx950, wave64).
//
// Element types: float, or bf16 stored as uint16 bits (bf16_t). Every K/V/summary row is read
// as 16-byte vectors: a lane holds VEC = 16 / sizeof(element) consecutive channels of one row,
// LPR = D / VEC lanes cover a row, and one wave-wide load covers RPW = 64 / LPR rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvsel {

struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct elem_traits;
template <>
struct elem_traits<float> {
  static constexpr int VEC = 4;
};
template <>
struct elem_traits<bf16_t> {
  static constexpr int VEC = 8;
};

template <typename T, int D>
struct row_map {
  static constexpr int VEC = elem_traits<T>::VEC;
  static constexpr int LPR = D / VEC;   // lanes per row
  static constexpr int RPW = 64 / LPR;  // rows per wave-wide load
  static_assert(D % VEC == 0 && 64 % LPR == 0, "row does not tile a wave");
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Round an fp32 value to the element type and widen it back.
template <typename T>
__device__ __forceinline__ float round_to_elem(float x);
template <>
__device__ __forceinline__ float round_to_elem<float>(float x) { return x; }
template <>
__device__ __forceinline__ float round_to_elem<bf16_t>(float x) {
  // gfx950's v_cvt_pk_bf16_f32: round to nearest even, the bits of f32_to_bf16_bits for every
  // finite value, in one instruction
  return (float)(__bf16)x;
}

// Min / max of summary extremes (page summaries, their tail refresh and the append's running
// update): IEEE 754-2019 minimum / maximum, so a NaN key propagates and -0 < +0; gfx950 has them as
// native three-operand instructions (v_minimum3_f32 / v_maximum3_f32), where fminf / fmaxf also
// need a quieting step per operand.
__device__ __forceinline__ float tmin(float a, float b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ float tmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
typedef unsigned int u32x4_nt_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  const u32x4_nt_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// Unpack one 16-byte vector into VEC floats.
template <typename T>
__device__ __forceinline__ void unpack(const uint4& v, float* f);
template <>
__device__ __forceinline__ void unpack<float>(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}
template <>
__device__ __forceinline__ void unpack<bf16_t>(const uint4& v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Pack VEC floats (already representable in T) into one 16-byte vector.
template <typename T>
__device__ __forceinline__ uint4 pack(const float* f);
template <>
__device__ __forceinline__ uint4 pack<float>(const float* f) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                    __float_as_uint(f[3]));
}
template <>
__device__ __forceinline__ uint4 pack<bf16_t>(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = f32_to_bf16_bits(f[2 * i]) | (f32_to_bf16_bits(f[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Load one element of type T (scalar) as float.
template <typename T>
__device__ __forceinline__ float load_elem(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<bf16_t>(const bf16_t* p, size_t i) {
  return bf16_to_f32(p[i].bits);
}

template <typename T>
__device__ __forceinline__ void store_elem(T* p, size_t i, float x);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, size_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void store_elem<bf16_t>(bf16_t* p, size_t i, float x) {
  p[i].bits = (uint16_t)f32_to_bf16_bits(x);
}

// ------------------------------------------------------------------------------------------
// Rotary rotation of one lane's slice of a key row (rotate-half pairs (i, i + D/2)).
//
// The lane holds channels [c0, c0 + VEC) of a row in `x`; its partner lane (lane ^ (LPR / 2))
// holds the paired channels. Every product and every sum is rounded to fp32 on its own (FP
// contraction off), and the result is rounded to the element type, so the kernels that rotate
// on the fly (summaries, attention) and the one that materializes (rope shift) agree bit for
// bit. `row` < 0 means: leave the slice unchanged. Must be called by all lanes of the wave.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float rot_mul(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ float rot_sub(float a, float b) {
#pragma clang fp contract(off)
  return a - b;
}
__device__ __forceinline__ float rot_add(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}

__device__ __forceinline__ float lane_xor_f32(float v, int m);  // defined below

template <typename T, int D>
__device__ __forceinline__ void rope_rotate_slice(float* x, int c0, int row, const float* __restrict__ cos_t,
                                                  const float* __restrict__ sin_t) {
  constexpr int VEC = row_map<T, D>::VEC;
  constexpr int LPR = row_map<T, D>::LPR;
  constexpr int HALF = D / 2;
  float partner[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) partner[e] = lane_xor_f32(x[e], LPR / 2);
  if (row < 0) return;
  const bool first = c0 < HALF;
  const int i0 = first ? c0 : c0 - HALF;
  const float* cr = cos_t + (size_t)row * HALF + i0;
  const float* sr = sin_t + (size_t)row * HALF + i0;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const float c = cr[e], s = sr[e];
    float y;
    if (first)
      y = rot_sub(rot_mul(x[e], c), rot_mul(partner[e], s));  // x_i c - x_{i+D/2} s
    else
      y = rot_add(rot_mul(x[e], c), rot_mul(partner[e], s));  // x_{i+D/2} c + x_i s
    x[e] = round_to_elem<T>(y);
  }
}

// ------------------------------------------------------------------------------------------
// Cross-lane primitives on DPP and the gfx950 permlane swaps (no LDS round trip).
// ------------------------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, BANK_MASK, false);
}

// DPP controls: quad permutations, mirrors, row shifts and row broadcasts.
constexpr int DPP_QUAD_XOR1 = 0xb1;    // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4e;    // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118;
constexpr int DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;

// Inclusive wave-wide scan (lane 0 first) of an associative op with identity `id`.
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, uint32_t id, Op op) {
  v = op(v, dpp_u32<DPP_ROW_SHR1>(id, v));
  v = op(v, dpp_u32<DPP_ROW_SHR2>(id, v));
  v = op(v, dpp_u32<DPP_ROW_SHR4, 0xf, 0xe>(id, v));
  v = op(v, dpp_u32<DPP_ROW_SHR8, 0xf, 0xc>(id, v));
  v = op(v, dpp_u32<DPP_ROW_BCAST15, 0xa>(id, v));
  v = op(v, dpp_u32<DPP_ROW_BCAST31, 0xc>(id, v));
  return v;
}
__device__ __forceinline__ uint32_t wave_scan_add(uint32_t v) {
  return wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = wave_scan(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = wave_scan(v, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Value of lane ^ 16 and lane ^ 32 (gfx950 permlane swaps).
__device__ __forceinline__ uint32_t xor16_u32(uint32_t v) {
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return ((threadIdx.x >> 4) & 1) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t xor32_u32(uint32_t v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ __forceinline__ float xor16_f32(float v) { return __uint_as_float(xor16_u32(__float_as_uint(v))); }
__device__ __forceinline__ float xor32_f32(float v) { return __uint_as_float(xor32_u32(__float_as_uint(v))); }
// The value of lane (lane ^ m), m a power of two fixed at compile time after unrolling: the lane
// swaps above for m = 16 and 32, DPP row_ror:8 for m = 8 (a rotation by 8 inside a row of 16
// lanes is lane ^ 8), ds_bpermute otherwise.
__device__ __forceinline__ float lane_xor_f32(float v, int m) {
  if (m == 8) return __uint_as_float(dpp_u32<0x128>(0u, __float_as_uint(v)));
  return m == 16 ? xor16_f32(v) : m == 32 ? xor32_f32(v) : __shfl_xor(v, m);
}

// op over the whole wave, in every lane (butterfly: quad xor 1 and 2, half-row and row mirrors on
// DPP, then the lane ^ 16 and lane ^ 32 swaps).
template <class Op>
__device__ __forceinline__ float wave_allreduce_f32(float x, Op op) {
  x = op(x, __uint_as_float(dpp_u32<DPP_QUAD_XOR1>(0u, __float_as_uint(x))));
  x = op(x, __uint_as_float(dpp_u32<DPP_QUAD_XOR2>(0u, __float_as_uint(x))));
  x = op(x, __uint_as_float(dpp_u32<DPP_ROW_HALF_MIRROR>(0u, __float_as_uint(x))));
  x = op(x, __uint_as_float(dpp_u32<DPP_ROW_MIRROR>(0u, __float_as_uint(x))));
  x = op(x, xor16_f32(x));
  x = op(x, xor32_f32(x));
  return x;
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint32_t lo = dpp_u32<CTRL>(0u, (uint32_t)u), hi = dpp_u32<CTRL>(0u, (uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double xor16_f64(double x) {
  const uint64_t u = __double_as_longlong(x);
  return __longlong_as_double((long long)(((uint64_t)xor16_u32((uint32_t)(u >> 32)) << 32) |
                                          xor16_u32((uint32_t)u)));
}
__device__ __forceinline__ double xor32_f64(double x) {
  const uint64_t u = __double_as_longlong(x);
  return __longlong_as_double((long long)(((uint64_t)xor32_u32((uint32_t)(u >> 32)) << 32) |
                                          xor32_u32((uint32_t)u)));
}

// Sum over aligned segments of SEG lanes (SEG in {4, 8, 16, 32, 64}); every lane of a segment
// gets the segment's sum (butterflies: quad xor 1, quad xor 2, half-row mirror, row mirror,
// then lane ^ 16 and lane ^ 32).
template <int SEG>
__device__ __forceinline__ double seg_sum_f64(double x) {
  x += dpp_f64<DPP_QUAD_XOR1>(x);
  x += dpp_f64<DPP_QUAD_XOR2>(x);
  if (SEG >= 8) x += dpp_f64<DPP_ROW_HALF_MIRROR>(x);
  if (SEG >= 16) x += dpp_f64<DPP_ROW_MIRROR>(x);
  if (SEG >= 32) x += xor16_f64(x);
  if (SEG >= 64) x += xor32_f64(x);
  return x;
}

// Orderable key of an fp32 score: unsigned order == float order; -0 and +0 map together.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace kvsel
