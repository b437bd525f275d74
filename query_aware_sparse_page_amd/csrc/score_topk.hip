// Query-aware page scoring, top-k page selection and the speculative-reuse decision.
//
// score_kernel: one block covers 4 * PPW logical pages of one (sequence, KV head); LPR lanes
// read a page's lo and hi rows as 16-byte slices (coalesced), multiply by the group's query
// slice in fp64 (every bf16 x bf16 or fp32 x fp32 product is exact in fp64), pick q*hi for
// q >= 0 and q*lo otherwise, and fold the LPR lanes. One fp64 -> fp32 rounding per score.
//
// topk_kernel: one block per (sequence, KV head). Exact radix select (4 passes of 8-bit digits,
// most significant first) finds the k-th largest orderable score key T; pages with key > T are
// taken, and pages with key == T are taken in ascending page order until k are chosen (ties go
// to the lower index). A ballot-based block prefix sum writes the chosen pages in ascending
// order. The same block evaluates the speculative-reuse decision for its (sequence, KV head).
#include "kvsel_device.h"
#include "kvsel_internal.h"

namespace kvsel {

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void score_kernel(const T* __restrict__ summ,
                                                    const T* __restrict__ q,
                                                    const int32_t* __restrict__ page_table,
                                                    const int32_t* __restrict__ seq_lens, int Hkv,
                                                    int P, int maxp, float* __restrict__ scores) {
  using M = row_map<T, D>;
  constexpr int VEC = M::VEC, LPR = M::LPR;
  constexpr int PPW = 64 / LPR;  // pages per wave
  const int b = blockIdx.z, j = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int L = seq_lens[b];
  const int N = L > 0 ? (L + P - 1) / P : 0;
  const int c0 = (lane % LPR) * VEC;
  const int n = blockIdx.x * (4 * PPW) + w * PPW + lane / LPR;
  const bool active = n < N;

  const int Hq = Hkv * G;
  double qd[G][VEC];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float f[VEC];
    unpack<T>(load16(q + ((size_t)b * Hq + j * G + g) * D + c0), f);
#pragma unroll
    for (int e = 0; e < VEC; ++e) qd[g][e] = (double)f[e];
  }
  float lo[VEC], hi[VEC];
  if (active) {
    const int p = page_table[(size_t)b * maxp + n];
    const T* s = summ + ((size_t)p * Hkv + j) * 2 * D;
    unpack<T>(load16(s + c0), lo);
    unpack<T>(load16(s + D + c0), hi);
  } else {
#pragma unroll
    for (int e = 0; e < VEC; ++e) lo[e] = hi[e] = 0.0f;
  }
  double acc = 0.0;
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const double x = (double)(qd[g][e] >= 0.0 ? hi[e] : lo[e]);
      acc = fma(qd[g][e], x, acc);
    }
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m);
  if (active && (lane % LPR) == 0) scores[((size_t)b * Hkv + j) * maxp + n] = (float)acc;
}

constexpr int TK_THREADS = 512;
constexpr int TK_WAVES = TK_THREADS / 64;
constexpr int TK_LDS_KEYS = 8192;

template <typename T, int D>
__global__ __launch_bounds__(TK_THREADS) void topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int Hkv, int G, int P,
    int maxp, int k, int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt,
    ReuseArgs reuse, const T* __restrict__ q) {
  __shared__ uint32_t keys[TK_LDS_KEYS];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_cnt[2][TK_WAVES];
  __shared__ uint32_t s_prefix, s_remaining;
  __shared__ double s_cos[8];
  __shared__ int s_corr;

  const int j = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int L = seq_lens[b];
  const int N = L > 0 ? (L + P - 1) / P : 0;
  const size_t list = (size_t)b * Hkv + j;
  const float* sc = scores + list * maxp;
  int32_t* out = sel_idx + list * k;
  const bool reuse_on = reuse.q_prev != nullptr;

  // ---- speculative-reuse decision: mean over the group of cos(q, q_prev), fp64 ----
  int corrected = 1;
  if (reuse_on) {
    if (w < G) {
      const int h = j * G + w;
      const T* a = q + ((size_t)b * Hkv * G + h) * D;
      const T* c = (const T*)reuse.q_prev + ((size_t)b * Hkv * G + h) * D;
      double dot = 0.0, na = 0.0, nb = 0.0;
      for (int d = lane; d < D; d += 64) {
        const double x = (double)load_elem<T>(a, d), y = (double)load_elem<T>(c, d);
        dot = fma(x, y, dot);
        na = fma(x, x, na);
        nb = fma(y, y, nb);
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        dot += __shfl_xor(dot, m);
        na += __shfl_xor(na, m);
        nb += __shfl_xor(nb, m);
      }
      if (lane == 0) s_cos[w] = dot / (sqrt(na) * sqrt(nb));
    }
    __syncthreads();
    if (tid == 0) {
      double csum = 0.0;
      for (int g = 0; g < G; ++g) csum += s_cos[g];
      const double C = csum / G;
      const int corr = (reuse.first_step || C < reuse.tau) ? 1 : 0;
      s_corr = corr;
      reuse.corrected[list] = (uint8_t)corr;
      if (reuse.similarity) reuse.similarity[list] = C;
    }
    __syncthreads();
    corrected = s_corr;
  }
  const bool write_used = reuse_on && corrected;

  if (N <= k) {
    for (int i = tid; i < k; i += TK_THREADS) {
      const int v = i < N ? i : -1;
      out[i] = v;
      if (write_used) reuse.used_idx[list * k + i] = v;
    }
  } else {
    const bool cached = N <= TK_LDS_KEYS;
    if (cached)
      for (int i = tid; i < N; i += TK_THREADS) keys[i] = score_key(sc[i]);
    if (tid == 0) {
      s_prefix = 0;
      s_remaining = (uint32_t)k;
    }
    __syncthreads();
    uint32_t prefix = 0, mask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += TK_THREADS) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < N; i += TK_THREADS) {
        const uint32_t u = cached ? keys[i] : score_key(sc[i]);
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (w == 0) {
        uint32_t h[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) h[t] = hist[4 * lane + t];
        const uint32_t own = h[0] + h[1] + h[2] + h[3];
        uint32_t suf = own;  // inclusive suffix sum over lanes >= lane
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t t = __shfl_down(suf, o);
          if (lane + o < 64) suf += t;
        }
        const uint32_t rem = s_remaining;
        uint32_t cum = suf - own;  // elements in bins above this lane's four
#pragma unroll
        for (int t = 3; t >= 0; --t) {
          const uint32_t after = cum + h[t];
          if (cum < rem && after >= rem) {
            s_prefix = prefix | ((uint32_t)(4 * lane + t) << shift);
            s_remaining = rem - cum;
          }
          cum = after;
        }
      }
      __syncthreads();
      prefix = s_prefix;
      mask |= 0xffu << shift;
    }
    const uint32_t T_key = prefix;
    const uint32_t need_eq = s_remaining;
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    uint32_t base_eq = 0, base_sel = 0;
    for (int t0 = 0; t0 < N; t0 += TK_THREADS) {
      const int i = t0 + tid;
      const uint32_t u = i < N ? (cached ? keys[i] : score_key(sc[i])) : 0u;
      const bool gt = i < N && u > T_key;
      const bool eq = i < N && u == T_key;
      const unsigned long long eqm = __ballot(eq);
      if (lane == 0) wave_cnt[0][w] = (uint32_t)__popcll(eqm);
      __syncthreads();
      uint32_t eq_before = base_eq + (uint32_t)__popcll(eqm & lt_mask), eq_tot = 0;
      for (int v = 0; v < TK_WAVES; ++v) {
        if (v < w) eq_before += wave_cnt[0][v];
        eq_tot += wave_cnt[0][v];
      }
      const bool sel = gt || (eq && eq_before < need_eq);
      const unsigned long long selm = __ballot(sel);
      if (lane == 0) wave_cnt[1][w] = (uint32_t)__popcll(selm);
      __syncthreads();
      uint32_t pos = base_sel + (uint32_t)__popcll(selm & lt_mask), sel_tot = 0;
      for (int v = 0; v < TK_WAVES; ++v) {
        if (v < w) pos += wave_cnt[1][v];
        sel_tot += wave_cnt[1][v];
      }
      if (sel && pos < (uint32_t)k) {
        out[pos] = i;
        if (write_used) reuse.used_idx[list * k + pos] = i;
      }
      base_eq += eq_tot;
      base_sel += sel_tot;
      __syncthreads();
    }
  }
  const int cnt = N < k ? N : k;
  if (tid == 0) sel_cnt[list] = cnt;
  if (reuse_on) {
    if (corrected) {
      if (tid == 0) reuse.used_cnt[list] = cnt;
    } else {
      for (int i = tid; i < k; i += TK_THREADS) reuse.used_idx[list * k + i] = reuse.prev_idx[list * k + i];
      if (tid == 0) reuse.used_cnt[list] = reuse.prev_cnt[list];
    }
  }
}

template <typename T, int D, int G>
static hipError_t launch_score_t(const LaunchKV& kv, const void* summ, const void* q,
                                 float* scores, hipStream_t stream) {
  constexpr int PPB = 4 * (64 / row_map<T, D>::LPR);
  const dim3 grid((unsigned)((kv.maxp + PPB - 1) / PPB), (unsigned)kv.Hkv, (unsigned)kv.B);
  hipLaunchKernelGGL((score_kernel<T, D, G>), grid, dim3(256), 0, stream, (const T*)summ,
                     (const T*)q, kv.page_table, kv.seq_lens, kv.Hkv, kv.P, kv.maxp, scores);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_score_topk_t(const LaunchKV& kv, const void* summ, const void* q, int k,
                                      int32_t* sel_idx, int32_t* sel_cnt, float* scores,
                                      const ReuseArgs& reuse, hipStream_t stream) {
  hipError_t e;
  switch (kv.G) {
    case 1: e = launch_score_t<T, D, 1>(kv, summ, q, scores, stream); break;
    case 2: e = launch_score_t<T, D, 2>(kv, summ, q, scores, stream); break;
    case 4: e = launch_score_t<T, D, 4>(kv, summ, q, scores, stream); break;
    default: e = launch_score_t<T, D, 8>(kv, summ, q, scores, stream); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((topk_kernel<T, D>), dim3((unsigned)kv.Hkv, (unsigned)kv.B), dim3(TK_THREADS),
                     0, stream, scores, kv.seq_lens, kv.Hkv, kv.G, kv.P, kv.maxp, k, sel_idx,
                     sel_cnt, reuse, (const T*)q);
  return hipGetLastError();
}

hipError_t launch_score_topk(const LaunchKV& kv, const void* summ, const void* q, int k,
                             int32_t* sel_idx, int32_t* sel_cnt, float* scores,
                             const ReuseArgs& reuse, hipStream_t stream) {
  if (kv.dtype == 0) {
    if (kv.D == 64)
      return launch_score_topk_t<float, 64>(kv, summ, q, k, sel_idx, sel_cnt, scores, reuse, stream);
    return launch_score_topk_t<float, 128>(kv, summ, q, k, sel_idx, sel_cnt, scores, reuse, stream);
  }
  if (kv.D == 64)
    return launch_score_topk_t<bf16_t, 64>(kv, summ, q, k, sel_idx, sel_cnt, scores, reuse, stream);
  return launch_score_topk_t<bf16_t, 128>(kv, summ, q, k, sel_idx, sel_cnt, scores, reuse, stream);
}

}  // namespace kvsel
