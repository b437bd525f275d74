// Page-summary build: channel-wise min / max of the valid keys of each (logical page, KV head),
// stored sequence-major, summ[b][j][n][lo | hi][D], so that scoring reads each list's summaries
// as one contiguous run with no page-table hop.
//
// One wave reduces one (page, KV head) tile of P x D keys: each lane loads 16-byte
// slices of rows (coalesced: LPR lanes cover one row, so one wave-wide load reads RPW whole
// rows), keeps a running min / max per channel, then the RPW row groups are folded with
// cross-lane exchanges and the first row group writes the lo and hi rows (16 bytes per lane).
// Min / max are exact, so the result does not depend on the reduction order.
#include "kvsel_device.h"
#include "kvsel_fp8.h"
#include "kvsel_internal.h"
#include "kvsel_score.h"

namespace kvsel {

// The (sequence b, logical page n, KV head j) tile of a wave, its physical page and its valid
// rows; false when the wave has none. tail_only: each sequence's last live page.
__device__ __forceinline__ bool summary_unit(long unit, const int32_t* __restrict__ page_table,
                                             const int32_t* __restrict__ seq_lens, int B, int Hkv,
                                             int P, int maxp, int maxn, int Npp, int tail_only,
                                             int& b, int& n, int& j, int& p, int& valid) {
  if (tail_only) {
    if (unit >= (long)B * Hkv) return false;
    b = (int)(unit / Hkv);
    j = (int)(unit % Hkv);
    const int L = seq_lens[b];
    if (L <= 0) return false;
    n = min((L - 1) / P, maxn - 1);  // a longer sequence: its last live page (all P rows)
  } else {
    if (unit >= (long)B * maxn * Hkv) return false;  // live pages only; maxp is the row stride
    b = (int)(unit / ((long)maxn * Hkv));
    const int rem = (int)(unit % ((long)maxn * Hkv));
    n = rem / Hkv;
    j = rem % Hkv;
    if (n * P >= seq_lens[b]) return false;
  }
  const int L = seq_lens[b];
  p = min(max(page_table[(size_t)b * maxp + n], 0), Npp - 1);  // clamp like every reader
  valid = min(P, L - n * P);
  return true;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void summaries_kernel(const T* __restrict__ k_pool,
                                                        const int32_t* __restrict__ page_table,
                                                        const int32_t* __restrict__ seq_lens, int B,
                                                        int Hkv, int P, int maxp, int maxn, int Npp,
                                                        int tail_only,
                                                        const int32_t* __restrict__ page_fill,
                                                        RopeArgs rope, T* __restrict__ summ) {
  using M = row_map<T, D>;
  const int lane = threadIdx.x & 63;
  const long unit = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  int b, n, j, p, valid;
  if (!summary_unit(unit, page_table, seq_lens, B, Hkv, P, maxp, maxn, Npp, tail_only, b, n, j, p,
                    valid))
    return;
  const int rg = lane / M::LPR;
  const int c0 = (lane % M::LPR) * M::VEC;
  float lo[M::VEC], hi[M::VEC];
  tile_minmax<T, D>(k_pool + ((size_t)p * Hkv + j) * P * D, valid, page_fill, P, lane, p,
                    rope_row_index(rope, b, n, p), rope, lo, hi);
  if (rg == 0) {
    T* out = summ + (((size_t)b * Hkv + j) * maxp + n) * 2 * D;
    store16(out + c0, pack<T>(lo));
    store16(out + D + c0, pack<T>(hi));
  }
}

// fp8 pools: the tile's extremes times its scale, rounded outward to bf16 (tile_minmax_fp8).
template <int D>
__global__ __launch_bounds__(256) void summaries_fp8_kernel(const uint8_t* __restrict__ k_pool,
                                                            const float* __restrict__ k_scale,
                                                            const int32_t* __restrict__ page_table,
                                                            const int32_t* __restrict__ seq_lens,
                                                            int B, int Hkv, int P, int maxp,
                                                            int maxn, int Npp, int tail_only,
                                                            const int32_t* __restrict__ page_fill,
                                                            bf16_t* __restrict__ summ) {
  using M = row_map<bf16_t, D>;
  const int lane = threadIdx.x & 63;
  const long unit = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  int b, n, j, p, valid;
  if (!summary_unit(unit, page_table, seq_lens, B, Hkv, P, maxp, maxn, Npp, tail_only, b, n, j, p,
                    valid))
    return;
  float lo[M::VEC], hi[M::VEC];
  tile_minmax_fp8<D>(k_pool + ((size_t)p * Hkv + j) * P * D, valid, page_fill, p, P, lane,
                     k_scale[(size_t)p * Hkv + j], lo, hi);
  if (lane < M::LPR) {
    bf16_t* out = summ + (((size_t)b * Hkv + j) * maxp + n) * 2 * D + lane * M::VEC;
    store16(out, pack<bf16_t>(lo));
    store16(out + D, pack<bf16_t>(hi));
  }
}

template <typename T, int D>
static hipError_t launch_summaries_t(const LaunchKV& kv, const RopeArgs& rope, int tail_only,
                                     void* summ, hipStream_t stream) {
  const long units = tail_only ? (long)kv.B * kv.Hkv : (long)kv.B * kv.maxn * kv.Hkv;
  const long blocks = (units + 3) / 4;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((summaries_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const T*)kv.k_pool, kv.page_table, kv.seq_lens, kv.B, kv.Hkv, kv.P, kv.maxp,
                     kv.maxn, kv.Npp, tail_only, kv.page_fill, rope, (T*)summ);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_summaries_fp8(const LaunchKV& kv, int tail_only, void* summ,
                                       hipStream_t stream) {
  const long units = tail_only ? (long)kv.B * kv.Hkv : (long)kv.B * kv.maxn * kv.Hkv;
  const long blocks = (units + 3) / 4;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((summaries_fp8_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint8_t*)kv.k_pool, kv.k_scale, kv.page_table, kv.seq_lens, kv.B,
                     kv.Hkv, kv.P, kv.maxp, kv.maxn, kv.Npp, tail_only, kv.page_fill,
                     (bf16_t*)summ);
  return hipGetLastError();
}

hipError_t launch_summaries(const LaunchKV& kv, const RopeArgs& rope, int tail_only, void* summ,
                            hipStream_t stream) {
  if (kv.dtype == 2)
    return kv.D == 64 ? launch_summaries_fp8<64>(kv, tail_only, summ, stream)
                      : launch_summaries_fp8<128>(kv, tail_only, summ, stream);
  if (kv.dtype == 0) {
    if (kv.D == 64) return launch_summaries_t<float, 64>(kv, rope, tail_only, summ, stream);
    return launch_summaries_t<float, 128>(kv, rope, tail_only, summ, stream);
  }
  if (kv.D == 64) return launch_summaries_t<bf16_t, 64>(kv, rope, tail_only, summ, stream);
  return launch_summaries_t<bf16_t, 128>(kv, rope, tail_only, summ, stream);
}

}  // namespace kvsel
