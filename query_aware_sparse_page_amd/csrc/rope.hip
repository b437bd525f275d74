// Rotary re-positioning of keys: the cos/sin table and the materialized rotation.
//
// rope_table_kernel: one thread per (row, pair i): angle = (first + row) * inv_freq[i] in fp64,
// cos / sin in fp64, each rounded once to fp32. The D/2 inverse frequencies theta^(-2i/D) depend
// on theta and D only; the host evaluates them once per call with the C library's pow and passes
// them by value, so every device angle is the exact fp64 product of the position and that value.
//
// rope_shift_kernel: one wave per (physical page, KV head); rows are read and written as 16-byte
// slices and rotated by rope_rotate_slice (the routine the summary and attention kernels use
// when they rotate on the fly, so all three produce identical bits).
#include <math.h>

#include "kvsel_device.h"
#include "kvsel_internal.h"

namespace kvsel {

__global__ __launch_bounds__(256) void rope_table_kernel(InvFreq inv_freq, int D, int first,
                                                         int n_rows, float* __restrict__ cos_t,
                                                         float* __restrict__ sin_t) {
  const int half = D / 2;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)n_rows * half) return;
  const int r = (int)(idx / half), i = (int)(idx % half);
  const double a = (double)(first + r) * inv_freq.v[i];
  cos_t[idx] = (float)cos(a);
  sin_t[idx] = (float)sin(a);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_shift_kernel(const T* k_in, T* k_out,
                                                         int Hkv, int P, int Npp, RopeArgs rope,
                                                         int in_place) {
  using M = row_map<T, D>;
  constexpr int VEC = M::VEC, LPR = M::LPR, RPW = M::RPW;
  const int lane = threadIdx.x & 63;
  const long unit = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= (long)Npp * Hkv) return;
  const int p = (int)(unit / Hkv), j = (int)(unit % Hkv);
  const int prow = rope.page_row[p];
  if (prow < 0 && in_place) return;
  const int rg = lane / LPR, c0 = (lane % LPR) * VEC;
  const size_t tile = ((size_t)p * Hkv + j) * P * D;
  for (int s = rg; s < P; s += RPW) {  // P is a multiple of RPW: every lane runs the same count
    float x[VEC];
    unpack<T>(load16(k_in + tile + (size_t)s * D + c0), x);
    rope_rotate_slice<T, D>(x, c0, prow < 0 ? -1 : prow + rope.row_step * s, rope.cos, rope.sin);
    store16(k_out + tile + (size_t)s * D + c0, pack<T>(x));
  }
}

hipError_t launch_rope_table(double theta, int D, int first_position, int n_rows, float* cos_t,
                             float* sin_t, hipStream_t stream) {
  const long total = (long)n_rows * (D / 2);
  if (total == 0) return hipSuccess;
  InvFreq inv;
  for (int i = 0; i < D / 2; ++i) inv.v[i] = pow(theta, -(2.0 * i) / D);
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     inv, D, first_position, n_rows, cos_t, sin_t);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_rope_shift_t(const LaunchKV& kv, const RopeArgs& rope, void* k_out,
                                      hipStream_t stream) {
  const long units = (long)kv.Npp * kv.Hkv;
  hipLaunchKernelGGL((rope_shift_kernel<T, D>), dim3((unsigned)((units + 3) / 4)), dim3(256), 0,
                     stream, (const T*)kv.k_pool, (T*)k_out, kv.Hkv, kv.P, kv.Npp, rope,
                     k_out == kv.k_pool ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_rope_shift(const LaunchKV& kv, const RopeArgs& rope, void* k_out,
                             hipStream_t stream) {
  if (kv.dtype == 0) {
    if (kv.D == 64) return launch_rope_shift_t<float, 64>(kv, rope, k_out, stream);
    return launch_rope_shift_t<float, 128>(kv, rope, k_out, stream);
  }
  if (kv.D == 64) return launch_rope_shift_t<bf16_t, 64>(kv, rope, k_out, stream);
  return launch_rope_shift_t<bf16_t, 128>(kv, rope, k_out, stream);
}

}  // namespace kvsel
