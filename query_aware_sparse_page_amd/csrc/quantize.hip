// fp8 quantization of a cache's pages (kvsel_quantize_pages): every (physical page, KV head) tile
// of K, and of V, gets the scale amax / 448 (fp32; 1 for an all-zero tile) and every value the
// E4M3 code of fp32(x / scale) (correctly rounded division, then round to nearest even with
// saturation, kvsel_fp8.h).
//
// One wave per tile. A tile's P * D values are one contiguous run in either pool layout, and
// neither the scale nor the coding depends on the order inside it, so the wave reads the run
// flat: lane l takes the 16-byte vectors l, l + 64, ... (coalesced), finds the tile's amax with a
// wave-wide max, and writes each vector's codes as one 8-byte (bf16 source) or 4-byte (f32
// source) store at the same position of the code run.
#include "kvsel_fp8.h"
#include "kvsel_internal.h"

namespace kvsel {

constexpr int QUANT_WAVES = 4;

template <typename T, int N>  // N = P * D values per tile
__global__ __launch_bounds__(QUANT_WAVES * 64) void quantize_kernel(const T* __restrict__ src,
                                                                   uint8_t* __restrict__ codes,
                                                                   float* __restrict__ scale,
                                                                   long tiles) {
  constexpr int VEC = elem_traits<T>::VEC;  // values per 16-byte vector
  constexpr int LOADS = N / (64 * VEC);     // vectors per lane
  static_assert(N % (64 * VEC) == 0, "a tile is a whole number of wave-wide loads");
  const long tile = (long)blockIdx.x * QUANT_WAVES + (threadIdx.x >> 6);
  if (tile >= tiles) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const T* in = src + tile * N;
  uint4 raw[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) raw[i] = load16(in + ((size_t)i * 64 + lane) * VEC);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    float x[VEC];
    unpack<T>(raw[i], x);
#pragma unroll
    for (int e = 0; e < VEC; ++e) amax = fmaxf(amax, fabsf(x[e]));
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, lane_xor_f32(amax, m));
  const float s = amax > 0.0f ? __fdiv_rn(amax, FP8_MAX) : 1.0f;
  if (lane == 0) scale[tile] = s;
  uint8_t* out = codes + tile * N;
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    float x[VEC];
    unpack<T>(raw[i], x);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < VEC; ++e) w[e >> 2] |= f32_to_fp8(__fdiv_rn(x[e], s)) << (8 * (e & 3));
    uint8_t* dst = out + ((size_t)i * 64 + lane) * VEC;
    if constexpr (VEC == 8)
      store8(dst, make_uint2(w[0], w[1]));
    else
      *reinterpret_cast<uint32_t*>(dst) = w[0];
  }
}

template <typename T, int N>
static void launch_quantize_n(const void* src, uint8_t* codes, float* scale, long tiles,
                              hipStream_t stream) {
  const unsigned blocks = (unsigned)((tiles + QUANT_WAVES - 1) / QUANT_WAVES);
  hipLaunchKernelGGL((quantize_kernel<T, N>), dim3(blocks), dim3(QUANT_WAVES * 64), 0, stream,
                     (const T*)src, codes, scale, tiles);
}

template <typename T>
static void launch_quantize_t(int n, const void* src, uint8_t* codes, float* scale, long tiles,
                              hipStream_t stream) {
  switch (n) {
    case 1024: launch_quantize_n<T, 1024>(src, codes, scale, tiles, stream); break;
    case 2048: launch_quantize_n<T, 2048>(src, codes, scale, tiles, stream); break;
    default: launch_quantize_n<T, 4096>(src, codes, scale, tiles, stream); break;
  }
}

hipError_t launch_quantize(const LaunchKV& src, uint8_t* k_codes, float* k_scale, uint8_t* v_codes,
                           float* v_scale, hipStream_t stream) {
  const long tiles = (long)src.Npp * src.Hkv;
  const int n = src.P * src.D;  // 1024, 2048 or 4096
  for (int pass = 0; pass < (v_codes ? 2 : 1); ++pass) {
    const void* in = pass == 0 ? src.k_pool : src.v_pool;
    uint8_t* codes = pass == 0 ? k_codes : v_codes;
    float* scale = pass == 0 ? k_scale : v_scale;
    if (src.dtype == 0) launch_quantize_t<float>(n, in, codes, scale, tiles, stream);
    else launch_quantize_t<bf16_t>(n, in, codes, scale, tiles, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvsel
