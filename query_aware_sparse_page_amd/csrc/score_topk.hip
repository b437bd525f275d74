// Query-aware page scoring, top-k page selection and the speculative-reuse decision.
//
// score_kernel: one block per (page chunk, list), list = (sequence, KV head) varying fastest.
// Each block scores 4 * PPW pages: LPR lanes read a page's lo and hi rows as 16-byte slices
// (coalesced), multiply by the group's query slice in fp64 (a bf16 x bf16 or fp32 x fp32 product
// is exact in fp64), take q*hi for q >= 0 and q*lo otherwise, and fold the LPR lanes; one
// fp64 -> fp32 rounding per score. With the tail refresh on, the block holding a sequence's last
// page first rebuilds that page's summary from the key pool (the page a decode step appends to),
// writes it, and scores it from the fresh values.
//
// topk_kernel: one block per list. An exact radix select over orderable 32-bit score keys
// (4 passes of 8-bit digits, most significant first) finds the k-th largest key T; pages with
// key > T are taken, pages with key == T are taken in ascending page order until k are chosen
// (ties go to the lower index), and a ballot-based block prefix sum writes them in ascending
// order. The same block evaluates the speculative-reuse decision.
//
// The two kernels are separate launches on purpose: a "last block of the list does the top-k"
// fusion needs a device-scope release / acquire per block, which on this GPU writes back and
// invalidates the XCD's L2 and measured slower than the second launch.
#include "kvsel_device.h"
#include "kvsel_internal.h"

namespace kvsel {

constexpr int SEL_THREADS = 256;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_LDS_KEYS = 8192;

struct SelectArgs {
  const void* k_pool;
  void* summ;
  const void* q;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int Hkv, P, maxp, k, nlists, nchunks, refresh_tail;
  RopeArgs rope;
  float* scores;
  int32_t* sel_idx;
  int32_t* sel_cnt;
  ReuseArgs reuse;
};

struct TopkSmem {
  uint32_t keys[SEL_LDS_KEYS];
  uint32_t hist[256];
  uint32_t wave_cnt[2][SEL_WAVES];
  uint32_t prefix, remaining;
  double cosv[8];
  int corr;
};

// Min / max of the valid rows of one (page, KV head) tile, computed by one wave. On return the
// lanes of row group 0 hold lo / hi of channels [c0, c0 + VEC).
template <typename T, int D>
__device__ __forceinline__ void tile_minmax(const T* tile, int valid, int P, int lane, int prow,
                                            const RopeArgs& rope, float* lo, float* hi) {
  using M = row_map<T, D>;
  constexpr int VEC = M::VEC, LPR = M::LPR, RPW = M::RPW;
  constexpr int MAX_LOADS = 32 / RPW;
  const int rg = lane / LPR;
  const int c0 = (lane % LPR) * VEC;
  uint4 raw[MAX_LOADS];
#pragma unroll
  for (int i = 0; i < MAX_LOADS; ++i) {
    const int s = rg + i * RPW;
    raw[i] = (s < valid) ? load16(tile + (size_t)s * D + c0) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    lo[e] = __int_as_float(0x7f800000);
    hi[e] = __int_as_float(0xff800000);
  }
#pragma unroll
  for (int i = 0; i < MAX_LOADS; ++i) {
    const int s = rg + i * RPW;
    if (i * RPW >= P) break;
    float x[VEC];
    unpack<T>(raw[i], x);
    if (rope.page_row)
      rope_rotate_slice<T, D>(x, c0, prow < 0 ? -1 : prow + rope.row_step * s, rope.cos, rope.sin);
    if (s < valid) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        lo[e] = fminf(lo[e], x[e]);
        hi[e] = fmaxf(hi[e], x[e]);
      }
    }
  }
#pragma unroll
  for (int m = LPR; m < 64; m <<= 1) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      lo[e] = fminf(lo[e], __shfl_xor(lo[e], m));
      hi[e] = fmaxf(hi[e], __shfl_xor(hi[e], m));
    }
  }
}

// Exact top-k of the N scores of one list, by the whole block; writes out[0..k) ascending
// (padded with -1) and, when `used` is non-null, the same list there too.
__device__ void block_topk(const float* __restrict__ sc, int N, int k, int32_t* __restrict__ out,
                           int32_t* __restrict__ used, TopkSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (N <= k) {
    for (int i = tid; i < k; i += SEL_THREADS) {
      const int v = i < N ? i : -1;
      out[i] = v;
      if (used) used[i] = v;
    }
    return;
  }
  const bool cached = N <= SEL_LDS_KEYS;
  if (cached)
    for (int i = tid; i < N; i += SEL_THREADS) sm.keys[i] = score_key(sc[i]);
  if (tid == 0) {
    sm.prefix = 0;
    sm.remaining = (uint32_t)k;
  }
  __syncthreads();
  uint32_t prefix = 0, mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += SEL_THREADS) sm.hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < N; i += SEL_THREADS) {
      const uint32_t u = cached ? sm.keys[i] : score_key(sc[i]);
      if ((u & mask) == prefix) atomicAdd(&sm.hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (w == 0) {
      uint32_t h[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) h[t] = sm.hist[4 * lane + t];
      const uint32_t own = h[0] + h[1] + h[2] + h[3];
      uint32_t suf = own;  // inclusive suffix sum over lanes >= lane
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_down(suf, o);
        if (lane + o < 64) suf += t;
      }
      const uint32_t rem = sm.remaining;
      uint32_t cum = suf - own;  // elements in the bins above this lane's four
#pragma unroll
      for (int t = 3; t >= 0; --t) {
        const uint32_t after = cum + h[t];
        if (cum < rem && after >= rem) {
          sm.prefix = prefix | ((uint32_t)(4 * lane + t) << shift);
          sm.remaining = rem - cum;
        }
        cum = after;
      }
    }
    __syncthreads();
    prefix = sm.prefix;
    mask |= 0xffu << shift;
  }
  const uint32_t T_key = prefix;
  const uint32_t need_eq = sm.remaining;
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  uint32_t base_eq = 0, base_sel = 0;
  for (int t0 = 0; t0 < N; t0 += SEL_THREADS) {
    const int i = t0 + tid;
    const uint32_t u = i < N ? (cached ? sm.keys[i] : score_key(sc[i])) : 0u;
    const bool gt = i < N && u > T_key;
    const bool eq = i < N && u == T_key;
    const unsigned long long eqm = __ballot(eq);
    if (lane == 0) sm.wave_cnt[0][w] = (uint32_t)__popcll(eqm);
    __syncthreads();
    uint32_t eq_before = base_eq + (uint32_t)__popcll(eqm & lt_mask), eq_tot = 0;
#pragma unroll
    for (int v = 0; v < SEL_WAVES; ++v) {
      if (v < w) eq_before += sm.wave_cnt[0][v];
      eq_tot += sm.wave_cnt[0][v];
    }
    const bool sel = gt || (eq && eq_before < need_eq);
    const unsigned long long selm = __ballot(sel);
    if (lane == 0) sm.wave_cnt[1][w] = (uint32_t)__popcll(selm);
    __syncthreads();
    uint32_t pos = base_sel + (uint32_t)__popcll(selm & lt_mask), sel_tot = 0;
#pragma unroll
    for (int v = 0; v < SEL_WAVES; ++v) {
      if (v < w) pos += sm.wave_cnt[1][v];
      sel_tot += sm.wave_cnt[1][v];
    }
    if (sel && pos < (uint32_t)k) {
      out[pos] = i;
      if (used) used[pos] = i;
    }
    base_eq += eq_tot;
    base_sel += sel_tot;
    __syncthreads();
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(SEL_THREADS) void score_kernel(SelectArgs a) {
  using M = row_map<T, D>;
  constexpr int VEC = M::VEC, LPR = M::LPR;
  constexpr int PPW = 64 / LPR;          // pages per wave
  constexpr int PPB = SEL_WAVES * PPW;   // pages per block
  __shared__ float s_tail[2][D];

  const int list = blockIdx.x % a.nlists;
  const int chunk = blockIdx.x / a.nlists;
  const int b = list / a.Hkv, j = list % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int P = a.P;
  const int L = a.seq_lens[b];
  const int N = L > 0 ? (L + P - 1) / P : 0;
  const int n0 = chunk * PPB;
  const int Hq = a.Hkv * G;
  const T* q = (const T*)a.q;
  const int c0 = (lane % LPR) * VEC;

  // ---- decode-time refresh of the tail page's summary ----
  const bool has_tail = a.refresh_tail && N > 0 && N - 1 >= n0 && N - 1 < n0 + PPB;
  if (has_tail) {
    if (w == 0) {
      const int n = N - 1;
      const int p = a.page_table[(size_t)b * a.maxp + n];
      const int valid = L - n * P;
      const int prow = a.rope.page_row ? a.rope.page_row[p] : -1;
      float lo[VEC], hi[VEC];
      tile_minmax<T, D>((const T*)a.k_pool + ((size_t)p * a.Hkv + j) * P * D, valid, P, lane, prow,
                        a.rope, lo, hi);
      if (lane < LPR) {
        T* out = (T*)a.summ + ((size_t)p * a.Hkv + j) * 2 * D;
        store16(out + c0, pack<T>(lo));
        store16(out + D + c0, pack<T>(hi));
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          s_tail[0][c0 + e] = lo[e];
          s_tail[1][c0 + e] = hi[e];
        }
      }
    }
    __syncthreads();
  }

  // ---- scores of this block's pages ----
  {
    const int n = n0 + w * PPW + lane / LPR;
    const bool active = n < N;
    double qd[G][VEC];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float f[VEC];
      unpack<T>(load16(q + ((size_t)b * Hq + j * G + g) * D + c0), f);
#pragma unroll
      for (int e = 0; e < VEC; ++e) qd[g][e] = (double)f[e];
    }
    float lo[VEC], hi[VEC];
    if (active && has_tail && n == N - 1) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        lo[e] = s_tail[0][c0 + e];
        hi[e] = s_tail[1][c0 + e];
      }
    } else if (active) {
      const int p = a.page_table[(size_t)b * a.maxp + n];
      const T* s = (const T*)a.summ + ((size_t)p * a.Hkv + j) * 2 * D;
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
    if (active && (lane % LPR) == 0) a.scores[(size_t)list * a.maxp + n] = (float)acc;
  }

}

template <typename T, int D, int G>
__global__ __launch_bounds__(SEL_THREADS) void topk_kernel(SelectArgs a) {
  __shared__ TopkSmem sm;
  const int list = blockIdx.x;
  const int b = list / a.Hkv, j = list % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int P = a.P;
  const int L = a.seq_lens[b];
  const int N = L > 0 ? (L + P - 1) / P : 0;
  const int Hq = a.Hkv * G;
  const T* q = (const T*)a.q;

  int corrected = 1;
  const bool reuse_on = a.reuse.q_prev != nullptr;
  if (reuse_on) {
    if (w < G) {
      // mean over the group of cos(q, q_prev) in fp64
      double dot = 0.0, na = 0.0, nb = 0.0;
      for (int g = w; g < G; g += SEL_WAVES) {
        const int h = j * G + g;
        const T* x = q + ((size_t)b * Hq + h) * D;
        const T* y = (const T*)a.reuse.q_prev + ((size_t)b * Hq + h) * D;
        dot = na = nb = 0.0;
        for (int d = lane; d < D; d += 64) {
          const double xv = (double)load_elem<T>(x, d), yv = (double)load_elem<T>(y, d);
          dot = fma(xv, yv, dot);
          na = fma(xv, xv, na);
          nb = fma(yv, yv, nb);
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          dot += __shfl_xor(dot, m);
          na += __shfl_xor(na, m);
          nb += __shfl_xor(nb, m);
        }
        if (lane == 0) sm.cosv[g] = dot / (sqrt(na) * sqrt(nb));
      }
    }
    __syncthreads();
    if (tid == 0) {
      double csum = 0.0;
      for (int g = 0; g < G; ++g) csum += sm.cosv[g];
      const double C = csum / G;
      const int corr = (a.reuse.first_step || C < a.reuse.tau) ? 1 : 0;
      sm.corr = corr;
      a.reuse.corrected[list] = (uint8_t)corr;
      if (a.reuse.similarity) a.reuse.similarity[list] = C;
    }
    __syncthreads();
    corrected = sm.corr;
  }
  int32_t* used = (reuse_on && corrected) ? a.reuse.used_idx + (size_t)list * a.k : nullptr;
  block_topk(a.scores + (size_t)list * a.maxp, N, a.k, a.sel_idx + (size_t)list * a.k, used, sm);
  const int cnt = N < a.k ? N : a.k;
  if (tid == 0) a.sel_cnt[list] = cnt;
  if (reuse_on) {
    if (corrected) {
      if (tid == 0) a.reuse.used_cnt[list] = cnt;
    } else {
      for (int i = tid; i < a.k; i += SEL_THREADS)
        a.reuse.used_idx[(size_t)list * a.k + i] = a.reuse.prev_idx[(size_t)list * a.k + i];
      if (tid == 0) a.reuse.used_cnt[list] = a.reuse.prev_cnt[list];
    }
  }
}

template <typename T, int D>
static int pages_per_select_block() {
  return SEL_WAVES * (64 / row_map<T, D>::LPR);
}

int select_blocks_per_list(const LaunchKV& kv) {
  const int ppb = kv.dtype == 0 ? (kv.D == 64 ? pages_per_select_block<float, 64>()
                                              : pages_per_select_block<float, 128>())
                                : (kv.D == 64 ? pages_per_select_block<bf16_t, 64>()
                                              : pages_per_select_block<bf16_t, 128>());
  return (kv.maxp + ppb - 1) / ppb;
}

template <typename T, int D, int G>
static hipError_t launch_select_t(const SelectArgs& a, hipStream_t stream) {
  const long blocks = (long)a.nlists * a.nchunks;
  hipLaunchKernelGGL((score_kernel<T, D, G>), dim3((unsigned)blocks), dim3(SEL_THREADS), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((topk_kernel<T, D, G>), dim3((unsigned)a.nlists), dim3(SEL_THREADS), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_select_g(int G, const SelectArgs& a, hipStream_t stream) {
  switch (G) {
    case 1: return launch_select_t<T, D, 1>(a, stream);
    case 2: return launch_select_t<T, D, 2>(a, stream);
    case 4: return launch_select_t<T, D, 4>(a, stream);
    default: return launch_select_t<T, D, 8>(a, stream);
  }
}

hipError_t launch_score_topk(const LaunchKV& kv, const RopeArgs& rope, void* summ, const void* q,
                             int k, int flags, int32_t* sel_idx, int32_t* sel_cnt, float* scores,
                             const ReuseArgs& reuse, hipStream_t stream) {
  SelectArgs a;
  a.k_pool = kv.k_pool;
  a.summ = summ;
  a.q = q;
  a.page_table = kv.page_table;
  a.seq_lens = kv.seq_lens;
  a.Hkv = kv.Hkv;
  a.P = kv.P;
  a.maxp = kv.maxp;
  a.k = k;
  a.nlists = kv.B * kv.Hkv;
  a.nchunks = select_blocks_per_list(kv);
  a.refresh_tail = (flags & 1) ? 1 : 0;
  a.rope = rope;
  a.scores = scores;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.reuse = reuse;
  if (kv.dtype == 0) {
    if (kv.D == 64) return launch_select_g<float, 64>(kv.G, a, stream);
    return launch_select_g<float, 128>(kv.G, a, stream);
  }
  if (kv.D == 64) return launch_select_g<bf16_t, 64>(kv.G, a, stream);
  return launch_select_g<bf16_t, 128>(kv.G, a, stream);
}

}  // namespace kvsel
